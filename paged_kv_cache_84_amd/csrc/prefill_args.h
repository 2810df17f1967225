// Arguments of one paged_attention_prefill_chunk call, validated on the host.
#pragma once

#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

struct PrefillArgs {
  void* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  int32_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* query_start_loc;
  const int32_t* num_computed_tokens;
  int32_t num_reqs, num_q_tokens, max_query_len;
  int32_t num_q_heads, num_kv_heads, head_dim;
  float softmax_scale;
  pkv_dtype q_dtype, kv_dtype;
  float k_scale, v_scale;
  void* stream;
};

// Vector-unit path (any supported dtype and head size).
pkv_status launch_prefill_rows(const PrefillArgs& a);
// MFMA path (bf16 q and cache, head_dim 128).
pkv_status launch_prefill_mfma(const PrefillArgs& a);

}  // namespace pkv
