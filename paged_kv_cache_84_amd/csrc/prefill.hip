// paged_attention_prefill_chunk: host validation and dispatch.
//
// Prompt chunks share a step with decodes under the unified schedule
// ("vLLM 引擎解剖", section "V1：统一调度预填充与解码", Fig. 3); each chunk row
// attends causally to everything before it, including the rows of its own
// chunk, through its request's block table ("v1/v0 区别", §3.1 "Token 预算").

#include "abi_util.h"
#include "prefill_args.h"

using namespace pkv;

extern "C" pkv_status paged_attention_prefill_chunk(
    void* out, const void* query, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* query_start_loc, const int32_t* num_computed_tokens,
    int32_t num_reqs, int32_t num_q_tokens, int32_t max_query_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    float softmax_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype, float k_scale,
    float v_scale, void* stream) {
  if (num_reqs < 0 || num_q_tokens < 0 || max_query_len < 0 || num_blocks < 0 ||
      max_blocks_per_seq < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (num_q_heads / num_kv_heads > 8) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  const bool f32 = q_dtype == PKV_F32 && kv_dtype == PKV_F32;
  const bool bf16 = q_dtype == PKV_BF16 && kv_dtype == PKV_BF16;
  const bool fp8 = q_dtype == PKV_BF16 && kv_dtype == PKV_FP8_E4M3;
  if (!(f32 || bf16 || fp8)) return PKV_ERR_UNSUPPORTED;
  if (!fp8) k_scale = v_scale = 1.0f;
  if (!(k_scale > 0.f && v_scale > 0.f)) return PKV_ERR_SHAPE;
  if (num_reqs == 0 || num_q_tokens == 0) return PKV_OK;
  if (num_blocks == 0) return PKV_ERR_SHAPE;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !query_start_loc ||
      !num_computed_tokens)
    return PKV_ERR_NULL;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_tables, 4) ||
      !aligned(query_start_loc, 4) || !aligned(num_computed_tokens, 4))
    return PKV_ERR_ALIGN;
  PrefillArgs a{out, query, k_cache, v_cache, num_blocks, block_tables,
                max_blocks_per_seq, query_start_loc, num_computed_tokens, num_reqs,
                num_q_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim,
                softmax_scale, q_dtype, kv_dtype, k_scale, v_scale, stream};
  const int group = num_q_heads / num_kv_heads;
  if (bf16 && head_dim == 128 && softmax_scale > 0.f &&
      (group == 1 || group == 2 || group == 4 || group == 8))
    return launch_prefill_mfma(a);
  return launch_prefill_rows(a);
}
