// Arguments of the matrix-core decode kernel, validated on the host.
#pragma once

#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

struct DecodeMfmaArgs {
  void* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  int32_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* context_lens;
  int32_t num_seqs, max_len;
  int32_t num_q_heads, num_kv_heads, head_dim;
  pkv_dtype kv_dtype;
  float scale_log2, v_scale;
  int32_t num_chunks, fixed_chunk;   // the work split (see decode_sched.h)
  int32_t chunks_per_wave;           // consecutive chunks one wave walks
  float* rec_out;                    // partials of sequences that span chunks
  float* rec_ml;
  void* stream;
  // int4 caches: float scales per (block, kv head, slot); nvfp4 caches: E4M3
  // block-scale bytes per (block, kv head, slot, 16 elements)
  const void* k_scales = nullptr;
  const void* v_scales = nullptr;
  int32_t window = 0;                // sliding window in tokens (0 = none)
  // append: the new token's K and V rows ([num_seqs][kv heads][D] bf16) are
  // written at position len - 1 before the attention (nullptr = no append);
  // an fp8 cache encodes them with k_scale (K) and v_scale (V)
  const void* new_k = nullptr;
  const void* new_v = nullptr;
  float k_scale = 1.0f;
  // kv heads per wave: 1, or 2 (see decode_mfma_heads_per_wave)
  int32_t heads_per_wave = 1;
};

// bf16 queries with a bf16 or fp8 E4M3 cache (head_dim 64 or 128), or an int4
// per token-head or nvfp4-style cache (head_dim 128); group <= 16.
bool decode_mfma_supported(pkv_dtype q_dtype, pkv_dtype kv_dtype, int head_dim, int group);
// kv heads one wave of the chunk kernel serves: 2 for fp8 caches whose query
// groups fit two to a wave's 16 columns (group <= 8) and for bf16 caches with
// one query head per kv head, given an even number of kv heads; else 1.
int decode_mfma_heads_per_wave(pkv_dtype kv_dtype, int group, int num_kv_heads);
// Chunks between the records a sequence's partials leave for the merge:
// chunks_per_wave for the caches whose kernel folds a wave's chunks of one
// sequence into one record (bf16, fp8), 1 for the others.
int decode_mfma_record_stride(pkv_dtype kv_dtype, int chunks_per_wave);
// Launches the chunk kernel only; the caller launches the merge.
pkv_status launch_decode_mfma(const DecodeMfmaArgs& a);

}  // namespace pkv
