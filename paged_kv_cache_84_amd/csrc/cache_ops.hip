// Slot mapping, cache writes and block copies: the byte-moving calls of the
// paged KV cache ("vLLM 引擎解剖", section "PagedAttention：为 KV 缓存分页").
// All three are bound by HBM traffic; they use 16-byte accesses and grids of
// one workgroup per token / per copied block.

#include <float.h>

#include "abi_util.h"
#include "common.h"

namespace pkv {

// ------------------------------------------------------------ slot mapping

// One workgroup per request; its threads walk the request's tokens.
__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ query_start_loc,
    const int32_t* __restrict__ num_computed, int32_t num_blocks,
    int64_t* __restrict__ slots, int32_t num_tokens) {
  const int r = blockIdx.x;
  const int begin = query_start_loc[r];
  const int end = query_start_loc[r + 1];
  const int computed = num_computed[r];
  const int32_t* row = block_tables + int64_t(r) * max_blocks;
  for (int t = begin + threadIdx.x; t < end; t += blockDim.x) {
    if (t < 0 || t >= num_tokens) continue;
    const int64_t p = int64_t(computed) + (t - begin);
    const int64_t j = p / kBlock;
    int64_t slot = -1;
    if (p >= 0 && j < max_blocks) {
      const int32_t b = row[j];
      if (b >= 0 && b < num_blocks) slot = int64_t(b) * kBlock + p % kBlock;
    }
    slots[t] = slot;
  }
}

// ------------------------------------------------------------ cache write

// Eight source elements -> their cache encoding, as 16 (copy of bf16),
// 32 (copy of fp32 = two 16-byte halves) or 8 (fp8) bytes.
template <typename Src, typename Dst>
struct Writer;

// store(v, dst, scale) encodes the 16 source bytes v; run loads them first.
template <>
struct Writer<BF16, BF16> {
  static constexpr int kElems = 8;
  PKV_DEVICE static void store(u32x4 v, uint16_t* dst, float) { store16(dst, v); }
  PKV_DEVICE static void run(const uint16_t* src, uint16_t* dst, float s) {
    store(load16(src), dst, s);
  }
};

template <>
struct Writer<F32, F32> {
  static constexpr int kElems = 4;
  PKV_DEVICE static void store(u32x4 v, float* dst, float) { store16(dst, v); }
  PKV_DEVICE static void run(const float* src, float* dst, float s) {
    store(load16(src), dst, s);
  }
};

template <>
struct Writer<BF16, FP8> {
  static constexpr int kElems = 8;
  PKV_DEVICE static void run(const uint16_t* src, uint8_t* dst, float scale) {
    store(load16(src), dst, scale);
  }
  PKV_DEVICE static void store(u32x4 v, uint8_t* dst, float scale) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lo |= uint32_t(f32_to_e4m3(bf16_lo(v[i]) / scale)) << (16 * i);
      lo |= uint32_t(f32_to_e4m3(bf16_hi(v[i]) / scale)) << (16 * i + 8);
      hi |= uint32_t(f32_to_e4m3(bf16_lo(v[i + 2]) / scale)) << (16 * i);
      hi |= uint32_t(f32_to_e4m3(bf16_hi(v[i + 2]) / scale)) << (16 * i + 8);
    }
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  }
};

template <>
struct Writer<F32, FP8> {
  static constexpr int kElems = 4;
  PKV_DEVICE static void run(const float* src, uint8_t* dst, float scale) {
    store(load16(src), dst, scale);
  }
  PKV_DEVICE static void store(u32x4 v, uint8_t* dst, float scale) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w |= uint32_t(f32_to_e4m3(__uint_as_float(v[i]) / scale)) << (8 * i);
    *reinterpret_cast<uint32_t*>(dst) = w;
  }
};

// One workgroup per token: all kv heads of its K and V.
template <typename Src, typename Dst>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const typename Src::storage* __restrict__ key,
    const typename Src::storage* __restrict__ value,
    typename Dst::storage* __restrict__ k_cache,
    typename Dst::storage* __restrict__ v_cache,
    const int64_t* __restrict__ slots, int32_t num_kv_heads, int32_t head_dim,
    int32_t num_blocks, float k_scale, float v_scale) {
  using W = Writer<Src, Dst>;
  const int t = blockIdx.x;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= int64_t(num_blocks) * kBlock) return;
  const int64_t block = slot / kBlock;
  const int offset = int(slot % kBlock);
  const int vecs_per_head = head_dim / W::kElems;
  const int vecs = num_kv_heads * vecs_per_head;
  const int64_t src_base = int64_t(t) * num_kv_heads * head_dim;
  for (int i = threadIdx.x; i < 2 * vecs; i += blockDim.x) {
    const bool is_v = i >= vecs;
    const int iv = is_v ? i - vecs : i;
    const int h = iv / vecs_per_head;
    const int d = (iv % vecs_per_head) * W::kElems;
    const int64_t dst =
        ((block * num_kv_heads + h) * kBlock + offset) * head_dim + d;
    const int64_t src = src_base + int64_t(h) * head_dim + d;
    if (is_v)
      W::run(value + src, v_cache + dst, v_scale);
    else
      W::run(key + src, k_cache + dst, k_scale);
  }
}

// ---------------------------------------- slot mapping + cache write in one
// One wave per token t, four tokens per workgroup.  The token's K/V loads go
// out first; meanwhile the wave finds t's request: lanes load
// query_start_loc and num_computed_tokens of kSearchBatch x 64 requests at
// once and the lane whose request holds t wins a ballot.  Then one load of
// the block-table entry gives the slot (the same formula and the same -1
// cases as slot_mapping_kernel); lane 0 stores it, and the rows go to the
// cache.  Two dependent trips to memory instead of the four of the two
// separate kernels.  The work per token is small and latency-bound, so a
// wave per token (not a workgroup) lets the whole step's tokens be in flight
// at once.
constexpr int kSearchBatch = 4;
constexpr int kHeldVecs = 4;      // 16-byte source pieces a lane holds while searching
constexpr int kSchedTokensPerWg = 4;

template <typename Src, typename Dst>
__global__ __launch_bounds__(256) void reshape_and_cache_sched_kernel(
    const typename Src::storage* __restrict__ key,
    const typename Src::storage* __restrict__ value,
    typename Dst::storage* __restrict__ k_cache, typename Dst::storage* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ num_computed,
    int32_t num_reqs, int64_t* __restrict__ slots_out, int32_t num_tokens, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_blocks, float k_scale, float v_scale) {
  using W = Writer<Src, Dst>;
  const int t = int(blockIdx.x) * kSchedTokensPerWg + int(threadIdx.x) / kWave;
  if (t >= num_tokens) return;      // the wave's token is past the last
  const int lane = lane_id();
  const int vecs_per_head = head_dim / W::kElems;
  const int vecs = num_kv_heads * vecs_per_head;
  const int64_t src_base = int64_t(t) * num_kv_heads * head_dim;
  auto src_of = [&](int i) {   // source piece i: K pieces, then V pieces
    const int iv = i >= vecs ? i - vecs : i;
    return (i >= vecs ? value : key) + src_base + int64_t(iv / vecs_per_head) * head_dim +
           (iv % vecs_per_head) * W::kElems;
  };
  u32x4 held[kHeldVecs];
#pragma unroll
  for (int n = 0; n < kHeldVecs; ++n) {
    const int i = lane + n * kWave;
    if (i < 2 * vecs) held[n] = load16(src_of(i));
  }

  // request of token t: query_start_loc[r] <= t < query_start_loc[r + 1]
  int req = -1, begin = 0, computed = 0;
  for (int base = 0; base < num_reqs; base += kSearchBatch * kWave) {
    int lo[kSearchBatch], hi[kSearchBatch], cc[kSearchBatch];
#pragma unroll
    for (int b = 0; b < kSearchBatch; ++b) {
      const int r = base + b * kWave + lane;
      const bool ok = r < num_reqs;
      lo[b] = ok ? query_start_loc[r] : 0;
      hi[b] = ok ? query_start_loc[r + 1] : 0;
      cc[b] = ok ? num_computed[r] : 0;
    }
    int found = -1, f_lo = 0, f_c = 0;
#pragma unroll
    for (int b = 0; b < kSearchBatch; ++b)
      if (lo[b] <= t && t < hi[b]) {
        found = base + b * kWave + lane;
        f_lo = lo[b];
        f_c = cc[b];
      }
    const uint64_t hit = __ballot(found >= 0);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      req = __shfl(found, src, kWave);
      begin = __shfl(f_lo, src, kWave);
      computed = __shfl(f_c, src, kWave);
      break;
    }
  }
  int64_t slot = -1;
  if (req >= 0) {
    const int64_t p = int64_t(computed) + (t - begin);
    const int64_t j = p / kBlock;
    if (p >= 0 && j < max_blocks) {
      const int32_t b = block_tables[int64_t(req) * max_blocks + j];
      if (b >= 0 && b < num_blocks) slot = int64_t(b) * kBlock + p % kBlock;
    }
  }
  if (slots_out != nullptr && lane == 0) slots_out[t] = slot;
  if (slot < 0) return;
  const int64_t block = slot / kBlock;
  const int offset = int(slot % kBlock);
  auto dst_of = [&](int i, typename Dst::storage* kc, typename Dst::storage* vc) {
    const int iv = i >= vecs ? i - vecs : i;
    return (i >= vecs ? vc : kc) +
           ((block * num_kv_heads + iv / vecs_per_head) * kBlock + offset) * head_dim +
           (iv % vecs_per_head) * W::kElems;
  };
#pragma unroll
  for (int n = 0; n < kHeldVecs; ++n) {
    const int i = lane + n * kWave;
    if (i < 2 * vecs) W::store(held[n], dst_of(i, k_cache, v_cache), i >= vecs ? v_scale : k_scale);
  }
  for (int i = lane + kHeldVecs * kWave; i < 2 * vecs; i += kWave)
    W::run(src_of(i), dst_of(i, k_cache, v_cache), i >= vecs ? v_scale : k_scale);
}

// ------------------------------------------------- int4 per token-head write
// One wave per (token, K|V, kv head) row: lane L quantises elements 2L and
// 2L + 1.  s = max|x| / 7 (a wave-wide max, then a binary32 division),
// q = round half to even of x / s, stored as the nibbles q + 8, element 2L in
// the low nibble of byte L; a zero row gets s = 0 and q = 0.

PKV_DEVICE float src_to_f32(uint16_t bits) { return bf16_to_f32(bits); }
PKV_DEVICE float src_to_f32(float v) { return v; }

template <typename Src>
__global__ __launch_bounds__(256) void reshape_and_cache_int4_kernel(
    const typename Src::storage* __restrict__ key,
    const typename Src::storage* __restrict__ value, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, float* __restrict__ k_scales, float* __restrict__ v_scales,
    const int64_t* __restrict__ slots, int32_t num_kv_heads, int32_t head_dim,
    int32_t num_blocks) {
  const int t = blockIdx.x;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= int64_t(num_blocks) * kBlock) return;
  const int64_t block = slot / kBlock;
  const int offset = int(slot % kBlock);
  const int lane = lane_id();
  const int wave = int(threadIdx.x) / kWave;
  const bool on = 2 * lane < head_dim;
  for (int row = wave; row < 2 * num_kv_heads; row += int(blockDim.x) / kWave) {
    const bool is_v = row >= num_kv_heads;
    const int h = is_v ? row - num_kv_heads : row;
    const typename Src::storage* src = (is_v ? value : key) + (int64_t(t) * num_kv_heads + h) * head_dim;
    const float x0 = on ? src_to_f32(src[2 * lane]) : 0.f;
    const float x1 = on ? src_to_f32(src[2 * lane + 1]) : 0.f;
    float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, shfl_xor(amax, o));
    const float s = amax / 7.0f;
    int q0 = 0, q1 = 0;
    if (s > 0.f) {
      q0 = min(7, max(-8, int(rintf(x0 / s))));
      q1 = min(7, max(-8, int(rintf(x1 / s))));
    }
    const int64_t r = (block * num_kv_heads + h) * kBlock + offset;
    if (on) (is_v ? v_cache : k_cache)[r * (head_dim / 2) + lane] = uint8_t((q0 + 8) | ((q1 + 8) << 4));
    if (lane == 0) (is_v ? v_scales : k_scales)[r] = s;
  }
}

// ------------------------------------------------------ nvfp4-style write
// One wave per (token, K|V, kv head) row: lane L encodes elements 2L and
// 2L + 1; the eight lanes of a 16-element block share its scale.
//   scale code  c = E4M3(fp32(fp32(max|x| / 6) / g))
//   element     E2M1(fp32(x / fp32(S * g))), S the value of c (codes 0 if S = 0)
// Element 2L goes to the low nibble of byte L; lane 8b writes block b's
// scale byte.

// binary32 -> E2M1 code: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the
// even mantissa (so 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2,
// 3.5 -> 4, 5 -> 4), above 6 saturates; the sign bit is kept (also of zero).
// Each comparison adds one step of the magnitude code; `>` where the tie
// stays below, `>=` where it goes up.
PKV_DEVICE uint32_t f32_to_e2m1(float y) {
  const float a = fabsf(y);
  const uint32_t mag = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) +
                       uint32_t(a >= 1.75f) + uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) +
                       uint32_t(a > 5.0f);
  return mag | ((__float_as_uint(y) >> 28) & 8u);
}

template <typename Src>
__global__ __launch_bounds__(256) void reshape_and_cache_nvfp4_kernel(
    const typename Src::storage* __restrict__ key,
    const typename Src::storage* __restrict__ value, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, uint8_t* __restrict__ k_bscales,
    uint8_t* __restrict__ v_bscales, const int64_t* __restrict__ slots, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_blocks, float k_scale, float v_scale) {
  const int t = blockIdx.x;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= int64_t(num_blocks) * kBlock) return;
  const int64_t block = slot / kBlock;
  const int offset = int(slot % kBlock);
  const int lane = lane_id();
  const int wave = int(threadIdx.x) / kWave;
  const bool on = 2 * lane < head_dim;
  for (int row = wave; row < 2 * num_kv_heads; row += int(blockDim.x) / kWave) {
    const bool is_v = row >= num_kv_heads;
    const int h = is_v ? row - num_kv_heads : row;
    const typename Src::storage* src =
        (is_v ? value : key) + (int64_t(t) * num_kv_heads + h) * head_dim;
    const float x0 = on ? src_to_f32(src[2 * lane]) : 0.f;
    const float x1 = on ? src_to_f32(src[2 * lane + 1]) : 0.f;
    float amax = fmaxf(fabsf(x0), fabsf(x1));
    amax = fmaxf(amax, shfl_xor(amax, 1));
    amax = fmaxf(amax, shfl_xor(amax, 2));
    amax = fmaxf(amax, shfl_xor(amax, 4));
    const float g = is_v ? v_scale : k_scale;
    const uint8_t sc = f32_to_e4m3((amax / 6.0f) / g);
    float s, unused;
    fp8x2_to_f32<false>(uint32_t(sc), s, unused);
    uint32_t c0 = 0, c1 = 0;
    if (s > 0.f) {
      const float den = s * g;
      c0 = f32_to_e2m1(x0 / den);
      c1 = f32_to_e2m1(x1 / den);
    }
    const int64_t r = (block * num_kv_heads + h) * kBlock + offset;
    if (on) {
      (is_v ? v_cache : k_cache)[r * (head_dim / 2) + lane] = uint8_t(c0 | (c1 << 4));
      if (lane % 8 == 0) (is_v ? v_bscales : k_bscales)[r * (head_dim / 16) + lane / 8] = sc;
    }
  }
}

// ------------------------------------------------------------ block copies

constexpr int kMaxLayersPerLaunch = 64;
struct LayerPtrs {
  void* k[kMaxLayersPerLaunch];
  void* v[kMaxLayersPerLaunch];
};

// grid: (pair, layer in this launch, K or V); 16-byte vector copy.
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    LayerPtrs ptrs, const int64_t* __restrict__ mapping, int32_t num_blocks,
    int64_t block_bytes) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y;
  const int64_t src = mapping[2 * pair];
  const int64_t dst = mapping[2 * pair + 1];
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return;
  char* base = static_cast<char*>(blockIdx.z == 0 ? ptrs.k[layer] : ptrs.v[layer]);
  const u32x4* s = reinterpret_cast<const u32x4*>(base + src * block_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(base + dst * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

// grid: (pair, layer in this launch, K or V).  Whole blocks between two
// pools, either of which may be pinned host memory mapped into the device's
// address space (the loads or the stores then cross the host link, so each
// thread keeps four 16-byte loads in flight).
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    LayerPtrs src, LayerPtrs dst, const int64_t* __restrict__ mapping,
    int32_t num_src_blocks, int32_t num_dst_blocks, int64_t block_bytes) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y;
  const int64_t s_blk = mapping[2 * pair];
  const int64_t d_blk = mapping[2 * pair + 1];
  if (s_blk < 0 || d_blk < 0 || s_blk >= num_src_blocks || d_blk >= num_dst_blocks) return;
  const char* sb = static_cast<const char*>(blockIdx.z == 0 ? src.k[layer] : src.v[layer]);
  char* db = static_cast<char*>(blockIdx.z == 0 ? dst.k[layer] : dst.v[layer]);
  const u32x4* s = reinterpret_cast<const u32x4*>(sb + s_blk * block_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(db + d_blk * block_bytes);
  const int64_t n = block_bytes / 16;
  const int64_t stride = blockDim.x;
  int64_t i = threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = s[i], b = s[i + stride], c = s[i + 2 * stride], e = s[i + 3 * stride];
    d[i] = a;
    d[i + stride] = b;
    d[i + 2 * stride] = c;
    d[i + 3 * stride] = e;
  }
  for (; i < n; i += stride) d[i] = s[i];
}

}  // namespace pkv

// ===================================================================== ABI

using namespace pkv;

extern "C" pkv_status compute_slot_mapping(const int32_t* block_tables,
                                           int32_t max_blocks_per_seq,
                                           const int32_t* query_start_loc,
                                           const int32_t* num_computed_tokens,
                                           int32_t num_reqs, int32_t num_blocks,
                                           int64_t* slot_mapping,
                                           int32_t num_tokens, void* stream) {
  if (num_reqs < 0 || num_tokens < 0 || max_blocks_per_seq < 0 || num_blocks < 0)
    return PKV_ERR_SHAPE;
  if (num_reqs == 0 || num_tokens == 0) return PKV_OK;
  if (!block_tables || !query_start_loc || !num_computed_tokens || !slot_mapping)
    return PKV_ERR_NULL;
  if (!aligned(slot_mapping, 8)) return PKV_ERR_ALIGN;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(num_reqs), dim3(256), 0,
                     as_stream(stream), block_tables, max_blocks_per_seq,
                     query_start_loc, num_computed_tokens, num_blocks,
                     slot_mapping, num_tokens);
  return launch_status();
}

template <typename Src, typename Dst>
static pkv_status launch_write(const void* key, const void* value, void* kc,
                               void* vc, const int64_t* slots, int32_t t,
                               int32_t hkv, int32_t d, int32_t nb, float ks,
                               float vs, void* stream) {
  hipLaunchKernelGGL((reshape_and_cache_kernel<Src, Dst>), dim3(t), dim3(256), 0,
                     as_stream(stream),
                     static_cast<const typename Src::storage*>(key),
                     static_cast<const typename Src::storage*>(value),
                     static_cast<typename Dst::storage*>(kc),
                     static_cast<typename Dst::storage*>(vc), slots, hkv, d, nb,
                     ks, vs);
  return launch_status();
}

extern "C" pkv_status reshape_and_cache(const void* key, const void* value,
                                        void* k_cache, void* v_cache,
                                        const int64_t* slot_mapping,
                                        int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t num_blocks,
                                        pkv_dtype src_dtype,
                                        pkv_dtype cache_dtype, float k_scale,
                                        float v_scale, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0)
    return PKV_ERR_SHAPE;
  if (head_dim % 8 != 0) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
    return PKV_ERR_ALIGN;
  if (cache_dtype == PKV_FP8_E4M3 && !(k_scale > 0.f && v_scale > 0.f))
    return PKV_ERR_SHAPE;
  if (src_dtype == PKV_BF16 && cache_dtype == PKV_BF16)
    return launch_write<BF16, BF16>(key, value, k_cache, v_cache, slot_mapping,
                                    num_tokens, num_kv_heads, head_dim,
                                    num_blocks, k_scale, v_scale, stream);
  if (src_dtype == PKV_F32 && cache_dtype == PKV_F32)
    return launch_write<F32, F32>(key, value, k_cache, v_cache, slot_mapping,
                                  num_tokens, num_kv_heads, head_dim, num_blocks,
                                  k_scale, v_scale, stream);
  if (src_dtype == PKV_BF16 && cache_dtype == PKV_FP8_E4M3)
    return launch_write<BF16, FP8>(key, value, k_cache, v_cache, slot_mapping,
                                   num_tokens, num_kv_heads, head_dim,
                                   num_blocks, k_scale, v_scale, stream);
  if (src_dtype == PKV_F32 && cache_dtype == PKV_FP8_E4M3)
    return launch_write<F32, FP8>(key, value, k_cache, v_cache, slot_mapping,
                                  num_tokens, num_kv_heads, head_dim, num_blocks,
                                  k_scale, v_scale, stream);
  return PKV_ERR_UNSUPPORTED;
}

template <typename Src, typename Dst>
static pkv_status launch_write_sched(const void* key, const void* value, void* kc, void* vc,
                                     const int32_t* bt, int32_t maxb, const int32_t* qsl,
                                     const int32_t* computed, int32_t reqs, int64_t* slots,
                                     int32_t t, int32_t hkv, int32_t d, int32_t nb, float ks,
                                     float vs, void* stream) {
  hipLaunchKernelGGL((reshape_and_cache_sched_kernel<Src, Dst>),
                     dim3((t + kSchedTokensPerWg - 1) / kSchedTokensPerWg),
                     dim3(kWave * kSchedTokensPerWg), 0,
                     as_stream(stream), static_cast<const typename Src::storage*>(key),
                     static_cast<const typename Src::storage*>(value),
                     static_cast<typename Dst::storage*>(kc),
                     static_cast<typename Dst::storage*>(vc), bt, maxb, qsl, computed, reqs,
                     slots, t, hkv, d, nb, ks, vs);
  return launch_status();
}

extern "C" pkv_status reshape_and_cache_from_schedule(
    const void* key, const void* value, void* k_cache, void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* query_start_loc,
    const int32_t* num_computed_tokens, int32_t num_reqs, int64_t* slot_mapping,
    int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
    pkv_dtype src_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale, void* stream) {
  if (num_tokens < 0 || num_reqs < 0 || max_blocks_per_seq < 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || num_blocks < 0)
    return PKV_ERR_SHAPE;
  if (head_dim % 8 != 0) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !block_tables || !query_start_loc ||
      !num_computed_tokens)
    return PKV_ERR_NULL;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8) || !aligned(block_tables, 4) ||
      !aligned(query_start_loc, 4) || !aligned(num_computed_tokens, 4))
    return PKV_ERR_ALIGN;
  if (cache_dtype == PKV_FP8_E4M3 && !(k_scale > 0.f && v_scale > 0.f)) return PKV_ERR_SHAPE;
#define PKV_SCHED_ARGS key, value, k_cache, v_cache, block_tables, max_blocks_per_seq, \
    query_start_loc, num_computed_tokens, num_reqs, slot_mapping, num_tokens, num_kv_heads, \
    head_dim, num_blocks, k_scale, v_scale, stream
  if (src_dtype == PKV_BF16 && cache_dtype == PKV_BF16)
    return launch_write_sched<BF16, BF16>(PKV_SCHED_ARGS);
  if (src_dtype == PKV_F32 && cache_dtype == PKV_F32)
    return launch_write_sched<F32, F32>(PKV_SCHED_ARGS);
  if (src_dtype == PKV_BF16 && cache_dtype == PKV_FP8_E4M3)
    return launch_write_sched<BF16, FP8>(PKV_SCHED_ARGS);
  if (src_dtype == PKV_F32 && cache_dtype == PKV_FP8_E4M3)
    return launch_write_sched<F32, FP8>(PKV_SCHED_ARGS);
#undef PKV_SCHED_ARGS
  return PKV_ERR_UNSUPPORTED;
}

extern "C" pkv_status reshape_and_cache_int4(const void* key, const void* value,
                                             void* k_cache, void* v_cache, float* k_scales,
                                             float* v_scales, const int64_t* slot_mapping,
                                             int32_t num_tokens, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t num_blocks,
                                             pkv_dtype src_dtype, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0)
    return PKV_ERR_SHAPE;
  if (head_dim % 2 != 0 || head_dim > 2 * kWave) return PKV_ERR_UNSUPPORTED;
  if (src_dtype != PKV_BF16 && src_dtype != PKV_F32) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !k_scales || !v_scales || !slot_mapping)
    return PKV_ERR_NULL;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(k_scales, 4) || !aligned(v_scales, 4) ||
      !aligned(slot_mapping, 8))
    return PKV_ERR_ALIGN;
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  if (src_dtype == PKV_BF16)
    hipLaunchKernelGGL(reshape_and_cache_int4_kernel<BF16>, dim3(num_tokens), dim3(256), 0,
                       as_stream(stream), static_cast<const uint16_t*>(key),
                       static_cast<const uint16_t*>(value), kc, vc, k_scales, v_scales,
                       slot_mapping, num_kv_heads, head_dim, num_blocks);
  else
    hipLaunchKernelGGL(reshape_and_cache_int4_kernel<F32>, dim3(num_tokens), dim3(256), 0,
                       as_stream(stream), static_cast<const float*>(key),
                       static_cast<const float*>(value), kc, vc, k_scales, v_scales,
                       slot_mapping, num_kv_heads, head_dim, num_blocks);
  return launch_status();
}

extern "C" pkv_status reshape_and_cache_nvfp4(const void* key, const void* value,
                                              void* k_cache, void* v_cache, void* k_bscales,
                                              void* v_bscales, const int64_t* slot_mapping,
                                              int32_t num_tokens, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t num_blocks,
                                              pkv_dtype src_dtype, float k_scale,
                                              float v_scale, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0)
    return PKV_ERR_SHAPE;
  if (!(k_scale > 0.f && v_scale > 0.f && k_scale <= FLT_MAX && v_scale <= FLT_MAX))
    return PKV_ERR_SHAPE;
  if (head_dim % 16 != 0 || head_dim > 2 * kWave) return PKV_ERR_UNSUPPORTED;
  if (src_dtype != PKV_BF16 && src_dtype != PKV_F32) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !k_bscales || !v_bscales || !slot_mapping)
    return PKV_ERR_NULL;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(k_bscales, 16) || !aligned(v_bscales, 16) ||
      !aligned(slot_mapping, 8))
    return PKV_ERR_ALIGN;
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  auto* ks = static_cast<uint8_t*>(k_bscales);
  auto* vs = static_cast<uint8_t*>(v_bscales);
  if (src_dtype == PKV_BF16)
    hipLaunchKernelGGL(reshape_and_cache_nvfp4_kernel<BF16>, dim3(num_tokens), dim3(256), 0,
                       as_stream(stream), static_cast<const uint16_t*>(key),
                       static_cast<const uint16_t*>(value), kc, vc, ks, vs, slot_mapping,
                       num_kv_heads, head_dim, num_blocks, k_scale, v_scale);
  else
    hipLaunchKernelGGL(reshape_and_cache_nvfp4_kernel<F32>, dim3(num_tokens), dim3(256), 0,
                       as_stream(stream), static_cast<const float*>(key),
                       static_cast<const float*>(value), kc, vc, ks, vs, slot_mapping,
                       num_kv_heads, head_dim, num_blocks, k_scale, v_scale);
  return launch_status();
}

extern "C" pkv_status copy_blocks(void* const* k_caches, void* const* v_caches,
                                  int32_t num_layers,
                                  const int64_t* block_mapping,
                                  int32_t num_pairs, int32_t num_blocks,
                                  int64_t block_bytes, void* stream) {
  if (num_layers < 0 || num_pairs < 0 || num_blocks < 0 || block_bytes <= 0 ||
      block_bytes % 16 != 0)
    return PKV_ERR_SHAPE;
  if (num_layers == 0 || num_pairs == 0) return PKV_OK;
  if (!k_caches || !v_caches || !block_mapping) return PKV_ERR_NULL;
  if (!aligned(block_mapping, 8)) return PKV_ERR_ALIGN;
  for (int l = 0; l < num_layers; ++l) {
    if (!k_caches[l] || !v_caches[l]) return PKV_ERR_NULL;
    if (!aligned(k_caches[l], 16) || !aligned(v_caches[l], 16)) return PKV_ERR_ALIGN;
  }
  for (int first = 0; first < num_layers; first += kMaxLayersPerLaunch) {
    const int n = num_layers - first < kMaxLayersPerLaunch ? num_layers - first
                                                           : kMaxLayersPerLaunch;
    LayerPtrs ptrs = {};
    for (int i = 0; i < n; ++i) {
      ptrs.k[i] = k_caches[first + i];
      ptrs.v[i] = v_caches[first + i];
    }
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, n, 2), dim3(256), 0,
                       as_stream(stream), ptrs, block_mapping, num_blocks,
                       block_bytes);
    const pkv_status st = launch_status();
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

extern "C" pkv_status swap_blocks(void* const* src_k_caches, void* const* src_v_caches,
                                  void* const* dst_k_caches, void* const* dst_v_caches,
                                  int32_t num_layers, const int64_t* block_mapping,
                                  int32_t num_pairs, int32_t num_src_blocks,
                                  int32_t num_dst_blocks, int64_t block_bytes, void* stream) {
  if (num_layers < 0 || num_pairs < 0 || num_src_blocks < 0 || num_dst_blocks < 0 ||
      block_bytes <= 0 || block_bytes % 16 != 0)
    return PKV_ERR_SHAPE;
  if (num_layers == 0 || num_pairs == 0) return PKV_OK;
  if (!src_k_caches || !src_v_caches || !dst_k_caches || !dst_v_caches || !block_mapping)
    return PKV_ERR_NULL;
  if (!aligned(block_mapping, 8)) return PKV_ERR_ALIGN;
  for (int l = 0; l < num_layers; ++l) {
    if (!src_k_caches[l] || !src_v_caches[l] || !dst_k_caches[l] || !dst_v_caches[l])
      return PKV_ERR_NULL;
    if (!aligned(src_k_caches[l], 16) || !aligned(src_v_caches[l], 16) ||
        !aligned(dst_k_caches[l], 16) || !aligned(dst_v_caches[l], 16))
      return PKV_ERR_ALIGN;
  }
  for (int first = 0; first < num_layers; first += kMaxLayersPerLaunch) {
    const int n = num_layers - first < kMaxLayersPerLaunch ? num_layers - first
                                                           : kMaxLayersPerLaunch;
    LayerPtrs src = {}, dst = {};
    for (int i = 0; i < n; ++i) {
      src.k[i] = src_k_caches[first + i];
      src.v[i] = src_v_caches[first + i];
      dst.k[i] = dst_k_caches[first + i];
      dst.v[i] = dst_v_caches[first + i];
    }
    hipLaunchKernelGGL(swap_blocks_kernel, dim3(num_pairs, n, 2), dim3(256), 0,
                       as_stream(stream), src, dst, block_mapping, num_src_blocks,
                       num_dst_blocks, block_bytes);
    const pkv_status st = launch_status();
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}
