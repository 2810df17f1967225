// Chunked-prefill attention on the gfx950 matrix cores (bf16, head_dim 128):
// the kernel around prefill_tile (prefill_tile.h), one workgroup per (eight
// 16-row units of the requests' rows, kv head).

#include "abi_util.h"
#include "common.h"
#include "prefill_args.h"
#include "prefill_tile.h"

namespace pkv {

__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    int32_t num_blocks, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ num_computed,
    int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t group,
    float scale_log2) {
  __shared__ pf::Stage stage0, stage1;
  prefill_tile(stage0, stage1, blockIdx.x, out, query, k_cache, v_cache, num_blocks,
               block_tables, max_blocks, query_start_loc, num_computed, num_reqs, num_q_heads,
               num_kv_heads, group, scale_log2);
}

// Host launch: grid = (workgroups of units, upper bound) x kv heads, kv head
// fastest.  A request of n tokens has ceil(n group / 16) units, at most
// n group / 16 + 1.  The softmax uses the raw maximum score to decide
// rescaling, which needs a positive scale; the caller routes other scales to
// the vector kernel.
pkv_status launch_prefill_mfma(const PrefillArgs& a) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int64_t units = (int64_t(a.num_q_tokens) * group + pf::kUnitRows - 1) / pf::kUnitRows +
                        a.num_reqs;
  const int64_t pieces = (units + pf::kUnits - 1) / pf::kUnits;
  const int64_t grid = pieces * a.num_kv_heads;
  if (grid > 0x7fffffff || pieces * pf::kUnits > 0x7fffffff) return PKV_ERR_SHAPE;
  hipLaunchKernelGGL(prefill_mfma_kernel, dim3(uint32_t(grid)), dim3(256), 0,
                     as_stream(a.stream), static_cast<uint16_t*>(a.out),
                     static_cast<const uint16_t*>(a.query),
                     static_cast<const uint16_t*>(a.k_cache),
                     static_cast<const uint16_t*>(a.v_cache), a.num_blocks, a.block_tables,
                     a.max_blocks_per_seq, a.query_start_loc, a.num_computed_tokens,
                     a.num_reqs, a.num_q_heads, a.num_kv_heads, group,
                     a.softmax_scale * pf::kLog2e);
  return launch_status();
}

}  // namespace pkv
