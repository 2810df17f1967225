// Paged decode attention on the matrix cores of gfx950 (bf16 queries; bf16,
// fp8 E4M3, int4 per token-head or nvfp4-style cache).
//
// Decode reads every K/V block of a sequence once per step and is bound by
// HBM bandwidth ("vLLM 引擎解剖", section "预填充、解码与三个时延指标"); the
// blocks are reached through the sequence's block table (section
// "PagedAttention：为 KV 缓存分页", Fig. 2).  What this kernel minimises is
// the vector-unit work per block, so that the wave is back to issuing loads
// as soon as a tile arrives.
//
// One wave per (work chunk, kv head) holds all query heads of the kv head's
// group as the 16 columns of MFMA tiles (unused columns carry zero queries).
// With an fp8 cache and a group of at most 8, one wave serves two adjacent
// kv heads (NH = 2): their groups take columns 0-7 and 8-15, S^T is one
// product chain per head with each column keeping its own head's, the
// softmax and the table walk serve both, and each head's PV products see
// P^T with the other head's columns zeroed, so both accumulate into one set.
// Per 16-token block:
//   S^T (16 keys x 16 heads) = K (16 x D) . Q^T      D/32 v_mfma_f32_16x16x32_bf16
//     K is loaded straight into A-operand registers: lane l holds 16 bytes of
//     key row l%16; Q^T lives in B-operand registers for the whole segment.
//   online softmax on S^T: lane l holds keys 4(l/16)..+3 of head l%16, so the
//     running max and sum are per lane (one head each), no cross-lane work
//     except on the rare raise of the max;
//   O^T (D x 16 heads) += V^T (D x 16 keys) . P^T   2 D/16 v_mfma_f32_16x16x16_bf16
//     P^T is the S^T register layout itself (the B operand of a 16x16x16
//     product holds keys 4(l/16)..+3 of column l%16), split into a bf16 high
//     part and a bf16 remainder so the product keeps fp32-level accuracy.
//     V^T comes from the V tile staged in LDS (row per key) through the
//     transposing LDS read ds_read_b64_tr_b16: within each 16-lane group,
//     lane j receives element j%4 of the 4-element rows addressed by lanes
//     4e + j/4 (e = 0..3), so lane 4k + q addressing key k, dims 4q..4q+3 of
//     a 16-dim slice hands every lane the 4 keys of its dim.
// fp8 tiles are widened to bf16 in registers (exact); k_scale is folded into
// the softmax scale and v_scale into the final normalisation.  nvfp4 tiles
// are widened the same way: each E2M1 code times its 16-element block's E4M3
// scale has at most six significant bits, so the bf16 result is exact.

#include <math.h>

#include <type_traits>

#include "abi_util.h"
#include "common.h"
#include "decode_mfma.h"
#include "decode_sched.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kRaiseM = 8.0f;   // log2 units, as in the vector kernel
constexpr float kNoMax = -1e30f;

PKV_DEVICE f32x4_t mfma_k32(u32x4 a, u32x4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
PKV_DEVICE f32x4_t mfma_k16(i16x4_t a, i16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
PKV_DEVICE uint32_t pack_bf16_rne(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// int4 per token-head cache: two codes u = q + 8 per byte (element 2i in the
// low nibble), the binary32 scale of each (block, kv head, slot) row in a
// separate array.  `bytes` is 0 so that byte-based formulas cannot be used
// for it by mistake.
struct INT4 {
  using storage = uint8_t;
  static constexpr int bytes = 0;
};
template <typename KVT>
constexpr bool kInt4 = std::is_same<KVT, INT4>::value;

// nvfp4-style cache: two E2M1 codes per byte (element 2i in the low nibble),
// one E4M3 scale byte per 16 elements of a row in a separate array
// [block][kv head][16][D / 16]; the per-tensor scales are the k_scale and
// v_scale of the fp8 cache.
struct NVFP4 {
  using storage = uint8_t;
  static constexpr int bytes = 0;
};
template <typename KVT>
constexpr bool kNvfp4 = std::is_same<KVT, NVFP4>::value;
template <typename KVT>
constexpr bool kPacked4 = kInt4<KVT> || kNvfp4<KVT>;   // 4-bit codes, two per byte
template <typename KVT>
constexpr int kElemBits = kPacked4<KVT> ? 4 : 8 * KVT::bytes;

// 136 in bf16: an int4 K element enters the products as 128 + u = 136 + q
// (a bf16 with the nibble in its low mantissa bits), and 136 * (sum of the
// other operand) is subtracted afterwards.
constexpr uint32_t kBf16x2_136 = 0x43084308u;
// An int4 V element enters the PV products as 1 + u/16 = 1.5 + q/16 (the
// nibble in the top four mantissa bits of 1.0): the sum over the keys then
// carries 1.5 sum p beside the wanted sum p q / 16, three times the wanted
// part at most instead of seventeen with 136 + q, so removing the offset
// after a long context cancels far fewer bits of the fp32 sum.  The factor
// 16 is applied with the offset's removal (exact).
constexpr float kInt4VOffset = 1.5f;
constexpr float kInt4VFactor = 16.0f;

// Eight nibbles (elements 0..7 of a little-endian dword) -> four dwords of
// bf16 pairs 128 + u: dword e holds elements 2e (low half) and 2e + 1.
PKV_DEVICE u32x4 int4x8_to_bf16_offset(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;           // elements 0, 2, 4, 6 (bytes 0..3)
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;    // elements 1, 3, 5, 7
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // v_perm: selector byte e picks lo's byte e, 4 + e picks hi's byte e,
    // 0x0C gives a zero byte
    const uint32_t sel = 0x0C000C00u | (uint32_t(4 + e) << 16) | uint32_t(e);
    o[e] = __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
  }
  return o;
}
// Eight nibbles -> four dwords of bf16 pairs 1 + u/16: the nibbles moved to
// bits 3..6 of their bytes, and the exponent of 1.0 (0x3F80) or'ed in.
PKV_DEVICE u32x4 int4x8_to_bf16_v(uint32_t w) {
  const uint32_t lo = (w << 3) & 0x78787878u;    // elements 0, 2, 4, 6
  const uint32_t hi = (w >> 1) & 0x78787878u;    // elements 1, 3, 5, 7
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t sel = 0x0C000C00u | (uint32_t(4 + e) << 16) | uint32_t(e);
    o[e] = __builtin_amdgcn_perm(hi, lo, sel) | 0x3F803F80u;
  }
  return o;
}

template <typename KVT, int D>
struct MGeom {
  static constexpr int kKSteps = D / 32;               // QK products per block
  static constexpr int kMTiles = D / 16;               // 16-dim slices of V
  static constexpr int kRowBytes = D * kElemBits<KVT> / 8;   // one cache row
  static constexpr int kTileBytes = kBlock * kRowBytes;
  static constexpr int kVLoads = kTileBytes / (kWave * 16);  // 16-byte V pieces per lane
  static constexpr int kKLoads = kPacked4<KVT> ? kKSteps / 4 : KVT::bytes == 2 ? kKSteps : kKSteps / 2;
  static constexpr int kVStride = D * 2 + 32;          // LDS bytes per staged bf16 V row
  static_assert(kKSteps >= 2 && kVLoads >= 1, "unsupported head size");
  static_assert(!kPacked4<KVT> || D == 128, "4-bit caches: head_dim 128");
};

// First dim of the 8 consecutive dims that lane group j feeds to QK product ks
// (any assignment works as long as K and Q use the same one; for fp8 it makes
// each lane's 16-byte load cover two products).
template <typename KVT>
PKV_DEVICE int qk_dim(int j, int ks) {
  if constexpr (kPacked4<KVT>) return 32 * j + 8 * ks;   // one 16-byte load = 32 dims
  else return KVT::bytes == 2 ? 8 * j + 32 * ks : 16 * j + 64 * (ks / 2) + 8 * (ks % 2);
}

template <typename KVT, int D>
struct KRegs {
  u32x4 v[MGeom<KVT, D>::kKLoads];
  u32x4 sc;       // int4: the scales of this lane's four keys; nvfp4: see load_bscales
};
template <typename KVT, int D>
struct VRegs {
  u32x4 v[MGeom<KVT, D>::kVLoads];
  u32x4 sc;       // int4: the scales of this lane's four keys; nvfp4: see load_bscales
};

// int4: the scales of keys 4 (lane/16) .. + 3 of one (block, kv head) row
// set of a scale array (16 floats per (block, kv head)).
PKV_DEVICE u32x4 load_scales(const float* row16, int lane) {
  return buffer_load16(tile_resource(row16, kBlock * 4), uint32_t((lane / 16) * 16));
}

// nvfp4: the two block-scale bytes of this lane's 32 dims -- dims 32 q .. +31
// of row r are blocks 2q and 2q + 1, bytes 8 r + 2q and + 1 of the (block,
// kv head) scale tile (128 bytes); K lanes hold row lane%16, q = lane/16, V
// lanes row lane/4, q = lane%4.  The aligned dword holding the pair is
// loaded and the pair moved to the low half of sc[0].
PKV_DEVICE uint32_t load_bscales(const uint8_t* tile128, uint32_t byte_offset) {
  const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(
      tile_resource(tile128, kBlock * 8), byte_offset & ~3u, 0, 0);
  return (byte_offset & 2u) ? (w >> 16) : w;
}
PKV_DEVICE uint32_t k_bscale_offset(int lane) { return uint32_t((lane % 16) * 8 + (lane / 16) * 2); }
PKV_DEVICE uint32_t v_bscale_offset(int lane) { return uint32_t(lane * 2); }

// nvfp4: eight E2M1 codes (a little-endian dword, element 2e in the low
// nibble of byte e) times the block scale s -> four dwords of bf16 pairs.
// The codes are widened with unit scale (the converter applies only the
// exponent of its scale operand), then multiplied by s in binary32: exact,
// as is the bf16 truncation of the product.
template <int kByte>
PKV_DEVICE uint32_t fp4x2_to_bf16(uint32_t w, float s) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, kByte);
  return pack_bf16_rne(f[0] * s, f[1] * s);
}
PKV_DEVICE u32x4 fp4x8_to_bf16(uint32_t w, float s) {
  return u32x4{fp4x2_to_bf16<0>(w, s), fp4x2_to_bf16<1>(w, s), fp4x2_to_bf16<2>(w, s),
               fp4x2_to_bf16<3>(w, s)};
}
// The two block scales of a lane (bytes 0, 1 of `pair`) as binary32 values.
PKV_DEVICE void bscales_f32(uint32_t pair, float& s0, float& s1) {
  fp8x2_to_f32<false>(pair, s0, s1);
}

template <typename KVT, int D>
PKV_DEVICE void load_k(KRegs<KVT, D>& r, const typename KVT::storage* tile, int lane) {
  using M = MGeom<KVT, D>;
  const auto rs = tile_resource(tile, M::kTileBytes);
  const uint32_t off = uint32_t((lane % 16) * M::kRowBytes + (lane / 16) * 16);
#pragma unroll
  for (int i = 0; i < M::kKLoads; ++i) r.v[i] = buffer_load16(rs, off, i * 64);
}

template <typename KVT, int D>
PKV_DEVICE void load_v(VRegs<KVT, D>& r, const typename KVT::storage* tile, int lane) {
  using M = MGeom<KVT, D>;
  const auto rs = tile_resource(tile, M::kTileBytes);
#pragma unroll
  for (int i = 0; i < M::kVLoads; ++i) r.v[i] = buffer_load16(rs, uint32_t(lane * 16), i * 1024);
}

// The A operand of QK product ks from the K registers.
template <typename KVT, int D>
PKV_DEVICE u32x4 k_operand(const KRegs<KVT, D>& r, int ks) {
  if constexpr (kInt4<KVT>) {
    return int4x8_to_bf16_offset(r.v[0][ks]);
  } else if constexpr (kNvfp4<KVT>) {
    // dword ks holds dims 32 (lane/16) + 8 ks .. + 7: block 2 (lane/16) + ks/2
    float s0, s1;
    bscales_f32(r.sc[0], s0, s1);
    return fp4x8_to_bf16(r.v[0][ks], ks < 2 ? s0 : s1);
  } else if constexpr (KVT::bytes == 2) {
    return r.v[ks];
  } else {
    const u32x4 x = r.v[ks / 2];
    const uint32_t w0 = (ks % 2) ? x[2] : x[0];
    const uint32_t w1 = (ks % 2) ? x[3] : x[1];
    return u32x4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                 fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1)};
  }
}

// V tile -> LDS as bf16 rows; rows at or past `rows` (unused slots of a last
// block, whose bytes may be anything) become zeros, since 0 * NaN would
// reach the accumulators.
template <typename KVT, int D>
PKV_DEVICE void stage_v(VRegs<KVT, D>& r, char* vl, int lane, int rows) {
  using M = MGeom<KVT, D>;
  if constexpr (kNvfp4<KVT>) {
    // lane L holds dims 32 (L%4) .. + 31 of key L/4 (dwords 0, 1: block
    // 2 (L%4); dwords 2, 3: the next); rows past `rows` may hold any byte,
    // NaN scales included, and become zeros
    char* dst = vl + (lane / 4) * M::kVStride + (lane % 4) * 64;
    float s0, s1;
    bscales_f32(r.sc[0], s0, s1);
    const bool live = lane / 4 < rows;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      *reinterpret_cast<u32x4*>(dst + 16 * w) =
          live ? fp4x8_to_bf16(r.v[0][w], w < 2 ? s0 : s1) : u32x4{0, 0, 0, 0};
    return;
  }
  if constexpr (kInt4<KVT>) {
    // lane L holds dims 32 (L%4) .. + 31 of key L/4; every code is a finite
    // bf16 (1 + u/16), and rows past `rows` get zero weight, so nothing is
    // cleared here
    char* dst = vl + (lane / 4) * M::kVStride + (lane % 4) * 64;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      *reinterpret_cast<u32x4*>(dst + 16 * w) = int4x8_to_bf16_v(r.v[0][w]);
    return;
  }
  if (rows < kBlock) {
#pragma unroll
    for (int i = 0; i < M::kVLoads; ++i)
      if ((lane * 16 + i * 1024) / M::kRowBytes >= rows) r.v[i] = u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < M::kVLoads; ++i) {
    const int o = lane * 16 + i * 1024;         // byte offset in the cache tile
    const int row = o / M::kRowBytes;
    const int col = (o % M::kRowBytes) / (kPacked4<KVT> ? 1 : KVT::bytes);
    char* dst = vl + row * M::kVStride + col * 2;
    if constexpr (KVT::bytes == 2) {
      *reinterpret_cast<u32x4*>(dst) = r.v[i];
    } else {
      const u32x4 x = r.v[i];
      *reinterpret_cast<u32x4*>(dst) =
          u32x4{fp8x2_to_bf16x2<false>(x[0]), fp8x2_to_bf16x2<true>(x[0]),
                fp8x2_to_bf16x2<false>(x[1]), fp8x2_to_bf16x2<true>(x[1])};
      *reinterpret_cast<u32x4*>(dst + 16) =
          u32x4{fp8x2_to_bf16x2<false>(x[2]), fp8x2_to_bf16x2<true>(x[2]),
                fp8x2_to_bf16x2<false>(x[3]), fp8x2_to_bf16x2<true>(x[3])};
    }
  }
}

}  // namespace

// K/V blocks a wave keeps in flight ahead of the one it multiplies (1 or 2),
// per cache type; each adds one register set of the block's pieces.  Two
// measured slower for every cache type on the 8B and 70B batches (the
// per-CU address and L1 path, not the loads in flight, bounds these
// kernels; the second set also costs occupancy).
#ifndef PKV_DEPTH_BF16
#define PKV_DEPTH_BF16 1
#endif
#ifndef PKV_DEPTH_FP8
#define PKV_DEPTH_FP8 1
#endif
#ifndef PKV_DEPTH_4BIT
#define PKV_DEPTH_4BIT 1
#endif
template <typename KVT>
constexpr int prefetch_depth() {
  return kPacked4<KVT> ? PKV_DEPTH_4BIT : KVT::bytes == 2 ? PKV_DEPTH_BF16 : PKV_DEPTH_FP8;
}

// Whether the kernel holds a finished segment's result in registers and
// folds a wave's chunks of one sequence into one record (section on the
// result below), per cache type.  The 4-bit kernels store each result at
// once: the held result's 34 registers would cost them one of the four
// waves per SIMD their split asks for, which measured slower than the
// stores.
#ifndef PKV_DEFER_BF16
#define PKV_DEFER_BF16 1
#endif
#ifndef PKV_DEFER_FP8
#define PKV_DEFER_FP8 1
#endif
template <typename KVT>
constexpr bool defers_results() {
  return kPacked4<KVT> ? false : KVT::bytes == 2 ? PKV_DEFER_BF16 : PKV_DEFER_FP8;
}

// Where a block-range cursor stands: sequence s holds the n blocks
// [before, before + n) of the flattened batch.
struct SeqCursor {
  int s, before, n, len;
  int first;   // first block read (sliding window), 0 otherwise
};

// Move the cursor forward to the sequence holding block x (x below the
// batch's block count, so the walk ends inside the batch).
PKV_DEVICE void cursor_to(SeqCursor& c, int x, const BatchScan& sc, const int32_t* lens,
                          int max_len, int window) {
  while (x >= c.before + c.n) {
    c.before += c.n;
    ++c.s;
    c.len = seq_len(sc, lens, c.s, max_len);
    c.n = window_blocks(c.len, window);
    c.first = first_block(c.len, window);
  }
}

// NH kv heads per wave (1, or 2 for groups of at most 8): with two, the
// wave's 16 MFMA columns hold both heads' query groups (columns 0..7 the
// first kv head's, 8..15 the second's), so the softmax, the cursor and table
// walk and the loop control are shared by two heads' tiles; each product is
// taken once per head and each column keeps the one of its own head.
template <typename KVT, int D, int NH>
__global__ __launch_bounds__(64) void decode_mfma_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    // not __restrict__: the append path stores into the caches it then reads
    const typename KVT::storage* k_cache, const typename KVT::storage* v_cache,
    int32_t num_blocks,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t max_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t group, float scale_log2,
    float v_scale, int32_t num_chunks, int32_t fixed_chunk, int32_t chunks_per_wave,
    float* __restrict__ rec_out, float* __restrict__ rec_ml,
    const void* __restrict__ k_scales, const void* __restrict__ v_scales, int32_t window,
    const uint16_t* __restrict__ new_k, const uint16_t* __restrict__ new_v, float k_scale) {
  using M = MGeom<KVT, D>;
  static_assert(NH == 1 || (NH == 2 && !kPacked4<KVT>), "two heads per wave: bf16 or fp8");
  __shared__ __align__(16) char vl_all[NH][kBlock * M::kVStride];
  const int kv_groups = num_kv_heads / NH;
  const int kvh0 = (blockIdx.x % kv_groups) * NH;   // first kv head of this wave
  const int wg = blockIdx.x / kv_groups;
  const int lane = lane_id();
  const int n16 = lane % 16;          // head column of this lane
  const int j = lane / 16;            // lane group
  const int half = NH == 2 ? n16 / 8 : 0;            // which of the wave's kv heads
  const int hcol = NH == 2 ? n16 % 8 : n16;          // column within that head's group
  const bool head_ok = hcol < group;
  const int kvh = kvh0 + half;                        // this lane's kv head
  const int head = kvh * group + (head_ok ? hcol : 0);

  // This wave walks the blocks [b0, b1) of the flattened batch: chunks
  // wg * chunks_per_wave .. + chunks_per_wave - 1, each of c blocks.
  const BatchScan sc = scan_batch(context_lens, num_seqs, max_len, window);
  const int c = chunk_blocks(sc.total, num_chunks, fixed_chunk);
  const int b0 = wg * chunks_per_wave * c;
  if (b0 >= sc.total) return;
  const int b1 = min(b0 + chunks_per_wave * c, sc.total);

  const int64_t head_stride = int64_t(kBlock) * M::kRowBytes /
                              int64_t(sizeof(typename KVT::storage));
  const int64_t block_stride = int64_t(num_kv_heads) * head_stride;
  auto tile = [&](const typename KVT::storage* base, int32_t b, int e = 0) {
    return base + int64_t(b) * block_stride + int64_t(kvh0 + e) * head_stride;
  };
  auto valid = [&](int32_t b) { return b >= 0 && b < num_blocks; };
  // int4: the 16 float scales of (block b, kvh); nvfp4: its 128-byte tile
  // of block scales
  auto scale_row = [&](const void* base, int32_t b) {
    return static_cast<const float*>(base) + (int64_t(b) * num_kv_heads + kvh) * kBlock;
  };
  auto bscale_tile = [&](const void* base, int32_t b) {
    return static_cast<const uint8_t*>(base) + (int64_t(b) * num_kv_heads + kvh) * kBlock * 8;
  };
  auto table_id = [&](const SeqCursor& q, int x) -> int32_t {
    const int i = x - q.before + q.first;
    return i < max_blocks ? load_scalar(block_tables, int64_t(q.s) * max_blocks + i) : -1;
  };
  // Q^T of sequence s as B operands (zero columns past the group)
  auto load_q = [&](int s, u32x4 (&qb)[M::kKSteps]) {
    const auto rq = tile_resource(query + (int64_t(s) * num_q_heads + head) * D,
                                  head_ok ? D * 2 : 0);
#pragma unroll
    for (int ks = 0; ks < M::kKSteps; ++ks)
      qb[ks] = buffer_load16_cached(rq, uint32_t(qk_dim<KVT>(j, ks) * 2));
  };
  // tr-read address of this lane: key lane/4, dims 4 (lane%4) of each slice
  typedef __attribute__((address_space(3))) char lds_char_t;
  auto vt_base = [&](int e) {
    return reinterpret_cast<lds_i16x4_t*>((lds_char_t*)vl_all[e] + (lane / 4) * M::kVStride +
                                          (lane % 4) * 8);
  };

  // Three cursors walk the range: `cc` at the block being multiplied, `lc`
  // one block ahead (its K/V pieces and, on entering a sequence, its Q are
  // in flight) and `ic` two blocks ahead (its block id is in flight through
  // the scalar cache).  Loads therefore cross sequence and chunk boundaries
  // without a pause; past b1 they re-read a block already read.
  SeqCursor cc;
  locate(sc, context_lens, max_len, b0, cc.s, cc.before, window);
  cc.len = seq_len(sc, context_lens, cc.s, max_len);
  cc.n = window_blocks(cc.len, window);
  cc.first = first_block(cc.len, window);
  SeqCursor lc = cc, ic = cc;

  // Append (new_k != nullptr): a decode row's new token sits at position
  // len - 1, in its sequence's last block, and the wave whose range holds
  // that block is the only one that reads it.  So this wave writes the new
  // K and V rows of those sequences (slot = table[s][(len-1)/16] * 16 +
  // (len-1) % 16, skipped for an unusable id) before it reads anything, and
  // waits for the stores once.
  if constexpr (!kPacked4<KVT>) {
    if (new_k != nullptr) {
      SeqCursor wc = cc;
      for (;;) {
        const int last = wc.before + wc.n - 1;        // flattened index of its last block
        if (wc.n > 0 && last >= b0 && last < b1) {
          const int pos = wc.len - 1;
          const int i = pos / kBlock;
          const int32_t id =
              i < max_blocks ? load_scalar(block_tables, int64_t(wc.s) * max_blocks + i) : -1;
#pragma unroll
          for (int e = 0; e < NH; ++e) {
          if (valid(id) && 2 * lane < D) {
            const int64_t row = int64_t(pos % kBlock) * D + 2 * lane;
            const int64_t src = (int64_t(wc.s) * num_kv_heads + kvh0 + e) * D + 2 * lane;
            const uint32_t kw = *reinterpret_cast<const uint32_t*>(new_k + src);
            const uint32_t vw = *reinterpret_cast<const uint32_t*>(new_v + src);
            typename KVT::storage* kd =
                const_cast<typename KVT::storage*>(tile(k_cache, id, e)) + row;
            typename KVT::storage* vd =
                const_cast<typename KVT::storage*>(tile(v_cache, id, e)) + row;
            if constexpr (KVT::bytes == 2) {
              *reinterpret_cast<uint32_t*>(kd) = kw;
              *reinterpret_cast<uint32_t*>(vd) = vw;
            } else {
              *reinterpret_cast<uint16_t*>(kd) =
                  uint16_t(f32_to_e4m3(bf16_lo(kw) / k_scale) | (f32_to_e4m3(bf16_hi(kw) / k_scale) << 8));
              *reinterpret_cast<uint16_t*>(vd) =
                  uint16_t(f32_to_e4m3(bf16_lo(vw) / v_scale) | (f32_to_e4m3(bf16_hi(vw) / v_scale) << 8));
            }
          }
          }
        }
        if (wc.before + wc.n >= b1 || wc.s + 1 >= num_seqs) break;
        wc.before += wc.n;
        ++wc.s;
        wc.len = seq_len(sc, context_lens, wc.s, max_len);
        wc.n = window_blocks(wc.len, window);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): the rows are stored
      __atomic_signal_fence(__ATOMIC_SEQ_CST);   // and no read moves above them
    }
  }

  u32x4 qb[M::kKSteps], qn[M::kKSteps];
  load_q(cc.s, qb);
  // int4: 136 * (sum of the column's query), the offset's share of S^T
  auto offset_share = [&]() {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < M::kKSteps; ++ks)
      c = mfma_k32(u32x4{kBf16x2_136, kBf16x2_136, kBf16x2_136, kBf16x2_136}, qb[ks], c);
    return c[0];
  };
  float kcorr = 0.f;
  if constexpr (kInt4<KVT>) kcorr = offset_share();
  // Block ids: ids[k] is the id of block x + k for k = 0 .. kDepth (those
  // of the blocks in flight and of the next to request); the id of block
  // x + kDepth + 1 is requested once ids[kDepth] has been used.
  constexpr int kDepth = prefetch_depth<KVT>();
  int32_t ids[kDepth + 1];
  ids[0] = table_id(cc, b0);
#pragma unroll
  for (int k = 1; k <= kDepth; ++k) {
    ids[k] = -1;
    if (b0 + k < b1) {
      cursor_to(ic, b0 + k, sc, context_lens, max_len, window);
      ids[k] = table_id(ic, b0 + k);
    }
  }
  const int32_t b_any = valid(ids[0]) ? ids[0] : 0;   // a block to re-read
  // kDepth register sets: set k holds the K/V of the blocks b0 + k,
  // b0 + k + kDepth, ... (past b1 or for an unusable id, a re-read of b_any)
  KRegs<KVT, D> kr[kDepth][NH];
  VRegs<KVT, D> vr[kDepth][NH];
  auto load_block_v = [&](VRegs<KVT, D> (&r)[NH], int32_t b) {
#pragma unroll
    for (int e = 0; e < NH; ++e) load_v<KVT, D>(r[e], tile(v_cache, b, e), lane);
    if constexpr (kInt4<KVT>) r[0].sc = load_scales(scale_row(v_scales, b), lane);
    if constexpr (kNvfp4<KVT>) r[0].sc[0] = load_bscales(bscale_tile(v_scales, b), v_bscale_offset(lane));
  };
  auto load_block_k = [&](KRegs<KVT, D> (&r)[NH], int32_t b) {
#pragma unroll
    for (int e = 0; e < NH; ++e) load_k<KVT, D>(r[e], tile(k_cache, b, e), lane);
    if constexpr (kInt4<KVT>) r[0].sc = load_scales(scale_row(k_scales, b), lane);
    if constexpr (kNvfp4<KVT>) r[0].sc[0] = load_bscales(bscale_tile(k_scales, b), k_bscale_offset(lane));
  };
  // V before K, block by block, the order of the loop's own loads, so that
  // each wait inside the loop covers exactly the pieces it needs
#pragma unroll
  for (int k = 0; k < kDepth; ++k) {
    const int32_t b = (k == 0 || (b0 + k < b1 && valid(ids[k]))) ? (k == 0 ? b_any : ids[k]) : b_any;
    load_block_v(vr[k], b);
    __builtin_amdgcn_sched_barrier(0);
    load_block_k(kr[k], b);
    __builtin_amdgcn_sched_barrier(0);
  }

  // O^T: column n of the accumulators is the output of column n's own head
  // (with two heads per wave, each head's products see P^T with the other
  // head's columns zeroed, so both accumulate into one set)
  f32x4_t acc[M::kMTiles];
#pragma unroll
  for (int mt = 0; mt < M::kMTiles; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // running max starts finite: a fully masked block then gives weights
  // 2^-inf = 0 instead of 2^(-inf + inf)
  float m = kNoMax, l = 0.f;
  float lp = 0.f;                     // int4: sum of the weights the products used
  int seg_start = b0;
  int chunk = b0 / c;                 // chunk of the current segment
  int chunk_end = b0 + c;             // its end

  // The result of the segments walked so far of one sequence.  With
  // kDefer it is held in registers and stored only when the wave moves on
  // to a second sequence or ends: a store inside the loop enters the same
  // in-order memory counter as the block loads, so every later wait for a
  // block would also wait for the store's completion.  Consecutive chunks of
  // one sequence then fold into it with the merge's log-sum-exp rescale, and
  // a wave leaves one record per sequence it walks part of, at the chunk
  // where that part starts.  Without kDefer every segment's result is stored
  // at its end, one record per chunk.
  constexpr bool kDefer = defers_results<KVT>();
  f32x4_t pend[M::kMTiles];
  float pend_m = kNoMax, pend_l = 0.f;
  int pend_s = -1;                    // its sequence, -1: nothing held
  int pend_chunk = 0;
  bool pend_first = false;            // it starts at the sequence's first block
  bool pend_last = false;             // it ends at the sequence's last block
  auto flush = [&]() {
    if (pend_s < 0) return;
    if (head_ok) {
      if (pend_first && pend_last) {
        // the whole sequence: the output itself
        const float f = v_scale / pend_l;
        uint16_t* op = out + (int64_t(pend_s) * num_q_heads + head) * D + 4 * j;
#pragma unroll
        for (int mt = 0; mt < M::kMTiles; ++mt) {
          const uint2 w = {pack_bf16_rne(pend[mt][0] * f, pend[mt][1] * f),
                           pack_bf16_rne(pend[mt][2] * f, pend[mt][3] * f)};
          *reinterpret_cast<uint2*>(op + mt * 16) = w;
        }
      } else {
        // the record of (pend_chunk, sequence) -> record pend_chunk + sequence
        const int64_t idx = int64_t(pend_chunk + pend_s) * num_q_heads + head;
        float* po = rec_out + idx * D + 4 * j;
#pragma unroll
        for (int mt = 0; mt < M::kMTiles; ++mt)
          *reinterpret_cast<float4*>(po + mt * 16) =
              make_float4(pend[mt][0], pend[mt][1], pend[mt][2], pend[mt][3]);
        if (j == 0) reinterpret_cast<float2*>(rec_ml)[idx] = make_float2(pend_m, pend_l);
      }
    }
    pend_s = -1;
  };

  // One block: x, whose K/V sit in register set P (x - b0 = P mod kDepth).
  auto step = [&](auto set, int x) {
    constexpr int P = decltype(set)::value;

    const int i = x - cc.before + cc.first;            // block of sequence cc.s
    const int rows = valid(ids[0]) ? min(kBlock, cc.len - i * kBlock) : 0;
    // sliding window: keys before `first_key` (in this block) are out of sight
    const int first_key = window > 0 ? cc.len - window - i * kBlock : 0;
    const bool more = x + 1 < b1;
    // the block kDepth ahead (possibly of a later sequence), into the set
    // this block frees, or a re-read past b1
    const int32_t bn = (x + kDepth < b1 && valid(ids[kDepth])) ? ids[kDepth] : b_any;
#pragma unroll
    for (int e = 0; e < NH; ++e) stage_v<KVT, D>(vr[P][e], vl_all[e], lane, rows);
    const u32x4 vsc = vr[P][0].sc;    // int4: this block's V scales (before the reload)
    __builtin_amdgcn_sched_barrier(0);
    load_block_v(vr[P], bn);
    __builtin_amdgcn_sched_barrier(0);
    // Q of a sequence entered by the next block
    const bool new_seq = more && x + 1 >= lc.before + lc.n;
    if (new_seq) {
      cursor_to(lc, x + 1, sc, context_lens, max_len, window);
      load_q(lc.s, qn);
    }
    // the id kDepth + 1 blocks ahead, requested only once bn has been
    // consumed: waiting for one scalar load waits for all of them
    int32_t id_new = -1;
    if (x + kDepth + 1 < b1) {
      cursor_to(ic, x + kDepth + 1, sc, context_lens, max_len, window);
      id_new = table_id(ic, x + kDepth + 1);
    }
    // S^T = K . Q^T, per head of the wave; a column keeps its own head's
    f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < M::kKSteps; ++ks) st = mfma_k32(k_operand<KVT, D>(kr[P][0], ks), qb[ks], st);
    if constexpr (NH == 2) {
      f32x4_t st1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < M::kKSteps; ++ks)
        st1 = mfma_k32(k_operand<KVT, D>(kr[P][NH - 1], ks), qb[ks], st1);
#pragma unroll
      for (int r = 0; r < 4; ++r) st[r] = half ? st1[r] : st[r];
    }
    const u32x4 ksc = kr[P][0].sc;    // int4: this block's K scales (before the reload)
    load_block_k(kr[P], bn);
    // online softmax over this lane's 4 keys of its head
    float sv[4];
    bool raise = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t;
      if constexpr (kInt4<KVT>)
        t = (st[r] - kcorr) * __uint_as_float(ksc[r]) * scale_log2;
      else
        t = st[r] * scale_log2;
      sv[r] = (4 * j + r < rows && 4 * j + r >= first_key) ? t : -INFINITY;
      raise |= sv[r] > m + kRaiseM;
    }
    if (__builtin_expect(__ballot(raise) != 0, 0)) {
      float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      bm = fmaxf(bm, shfl_xor(bm, 16));
      bm = fmaxf(bm, shfl_xor(bm, 32));
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mn);
      m = mn;
      l *= alpha;
      if constexpr (kInt4<KVT>) lp *= alpha;
#pragma unroll
      for (int mt = 0; mt < M::kMTiles; ++mt) acc[mt] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(sv[r] - m);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    // int4: the V scale of each key joins its weight (masked keys keep
    // weight 0 whatever their scale slot holds)
    if constexpr (kInt4<KVT>) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p[r] = (4 * j + r < rows && 4 * j + r >= first_key) ? p[r] * __uint_as_float(vsc[r]) : 0.f;
    }
    // P^T = hi + lo, both bf16
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t a = __float_as_uint(p[2 * w]), b = __float_as_uint(p[2 * w + 1]);
      hi[w] = (b & 0xffff0000u) | (a >> 16);
      lo[w] = pack_bf16_rne(p[2 * w] - __uint_as_float(a & 0xffff0000u),
                            p[2 * w + 1] - __uint_as_float(b & 0xffff0000u));
      if constexpr (kInt4<KVT>)   // the weights exactly as the products see them
        lp += (__uint_as_float(a & 0xffff0000u) + __uint_as_float(lo[w] << 16)) +
              (__uint_as_float(b & 0xffff0000u) + __uint_as_float(lo[w] & 0xffff0000u));
    }
    const i16x4_t phi = __builtin_bit_cast(i16x4_t, uint2{hi[0], hi[1]});
    const i16x4_t plo = __builtin_bit_cast(i16x4_t, uint2{lo[0], lo[1]});
    // O^T += V^T . P^T (head e's V against the columns of head e only)
#pragma unroll
    for (int e = 0; e < NH; ++e) {
      const i16x4_t zero = {0, 0, 0, 0};
      const i16x4_t ph = NH == 1 || half == e ? phi : zero;
      const i16x4_t pl = NH == 1 || half == e ? plo : zero;
#pragma unroll
      for (int mt = 0; mt < M::kMTiles; ++mt) {
        const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vt_base(e) + mt * 4);
        acc[mt] = mfma_k16(a, ph, acc[mt]);
        acc[mt] = mfma_k16(a, pl, acc[mt]);
      }
    }
#pragma unroll
    for (int k = 0; k < kDepth; ++k) ids[k] = ids[k + 1];
    ids[kDepth] = id_new;

    // A segment ends with its sequence, at a chunk boundary, or at b1.
    const int seq_end = cc.before + cc.n;
    if (x + 1 == seq_end || x + 1 == chunk_end || !more) {
      // sum of weights of each head over the four lane groups
      float lt = l + shfl_xor(l, 16);
      lt += shfl_xor(lt, 32);
      if constexpr (kInt4<KVT>) {
        // remove the offset: O = 16 (sum p (1.5 + q/16) - 1.5 sum p)
        float lpt = lp + shfl_xor(lp, 16);
        lpt += shfl_xor(lpt, 32);
#pragma unroll
        for (int mt = 0; mt < M::kMTiles; ++mt)
          acc[mt] = (acc[mt] - kInt4VOffset * lpt) * kInt4VFactor;
      }
      auto hold = [&]() {
#pragma unroll
        for (int mt = 0; mt < M::kMTiles; ++mt) pend[mt] = acc[mt];
        pend_m = m;
        pend_l = lt;
        pend_s = cc.s;
        pend_chunk = chunk;
        pend_first = seg_start == cc.before;
        pend_last = x + 1 == seq_end;
      };
      if constexpr (kDefer) {
        if (pend_s == cc.s) {
          // an earlier chunk of this sequence, walked by this wave: fold
          // (max a, sum A, O_a) and (b, B, O_b) into (c, A 2^(a-c) + B 2^(b-c),
          // O_a 2^(a-c) + O_b 2^(b-c)), c = max(a, b)
          const float mn = fmaxf(pend_m, m);
          const float wa = fast_exp2(pend_m - mn), wb = fast_exp2(m - mn);
#pragma unroll
          for (int mt = 0; mt < M::kMTiles; ++mt) pend[mt] = pend[mt] * wa + acc[mt] * wb;
          pend_l = pend_l * wa + lt * wb;
          pend_m = mn;
          pend_last = x + 1 == seq_end;
        } else {
          flush();
          hold();
        }
      } else {
        hold();
        flush();
      }
#pragma unroll
      for (int mt = 0; mt < M::kMTiles; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m = kNoMax;
      l = 0.f;
      lp = 0.f;
      seg_start = x + 1;
      if (x + 1 == chunk_end) {
        ++chunk;
        chunk_end += c;
      }
      if (x + 1 == seq_end && more) {
        cursor_to(cc, x + 1, sc, context_lens, max_len, window);
#pragma unroll
        for (int ks = 0; ks < M::kKSteps; ++ks) qb[ks] = qn[ks];
        if constexpr (kInt4<KVT>) kcorr = offset_share();
      }
    }
  };
  for (int x = b0; x < b1; x += kDepth) {
    step(std::integral_constant<int, 0>{}, x);
    if constexpr (kDepth == 2) {
      if (x + 1 >= b1) break;
      step(std::integral_constant<int, kDepth - 1>{}, x + 1);
    }
  }
  if constexpr (kDefer) flush();
}

template <typename KVT, int D, int NH = 1>
static pkv_status launch_one(const DecodeMfmaArgs& a) {
  const int waves = (a.num_chunks + a.chunks_per_wave - 1) / a.chunks_per_wave;
  hipLaunchKernelGGL((decode_mfma_kernel<KVT, D, NH>), dim3(waves * (a.num_kv_heads / NH)),
                     dim3(kWave), 0, as_stream(a.stream), static_cast<uint16_t*>(a.out),
                     static_cast<const uint16_t*>(a.query),
                     static_cast<const typename KVT::storage*>(a.k_cache),
                     static_cast<const typename KVT::storage*>(a.v_cache), a.num_blocks,
                     a.block_tables, a.max_blocks, a.context_lens, a.num_seqs, a.max_len,
                     a.num_q_heads, a.num_kv_heads, a.num_q_heads / a.num_kv_heads,
                     a.scale_log2, a.v_scale, a.num_chunks, a.fixed_chunk,
                     a.chunks_per_wave, a.rec_out, a.rec_ml, a.k_scales, a.v_scales,
                     a.window, static_cast<const uint16_t*>(a.new_k),
                     static_cast<const uint16_t*>(a.new_v), a.k_scale);
  return launch_status();
}

#ifndef PKV_DECODE_PAIR_FP8
#define PKV_DECODE_PAIR_FP8 1
#endif
// bf16 caches pair kv heads only up to this group size: one head per kv
// head (MHA) leaves 15 of a wave's 16 columns empty, and pairing measured
// 2.9% faster on the 32-layer MHA step (20.69 vs 21.31 ms), while at group 4
// (the 8B batch) it measured slower (0.105-0.107 vs 0.099-0.101 ms).
#ifndef PKV_DECODE_PAIR_BF16_MAX_GROUP
#define PKV_DECODE_PAIR_BF16_MAX_GROUP 1
#endif
int decode_mfma_record_stride(pkv_dtype kv_dtype, int chunks_per_wave) {
  switch (kv_dtype) {
    case PKV_BF16: return defers_results<BF16>() ? chunks_per_wave : 1;
    case PKV_FP8_E4M3: return defers_results<FP8>() ? chunks_per_wave : 1;
    default: return 1;
  }
}

int decode_mfma_heads_per_wave(pkv_dtype kv_dtype, int group, int num_kv_heads) {
  const bool pair = kv_dtype == PKV_FP8_E4M3
                        ? PKV_DECODE_PAIR_FP8
                        : kv_dtype == PKV_BF16 && group <= PKV_DECODE_PAIR_BF16_MAX_GROUP;
  return (pair && group <= 8 && num_kv_heads % 2 == 0) ? 2 : 1;
}

bool decode_mfma_supported(pkv_dtype q_dtype, pkv_dtype kv_dtype, int head_dim, int group) {
  if (kv_dtype == PKV_INT4 || kv_dtype == PKV_NVFP4)
    return q_dtype == PKV_BF16 && head_dim == 128 && group >= 1 && group <= 16;
  return q_dtype == PKV_BF16 && (kv_dtype == PKV_BF16 || kv_dtype == PKV_FP8_E4M3) &&
         (head_dim == 64 || head_dim == 128) && group >= 1 && group <= 16;
}

pkv_status launch_decode_mfma(const DecodeMfmaArgs& a) {
  if (a.kv_dtype == PKV_INT4) return launch_one<INT4, 128>(a);
  if (a.kv_dtype == PKV_NVFP4) return launch_one<NVFP4, 128>(a);
  if (a.kv_dtype == PKV_BF16) {
    if (a.heads_per_wave == 2)
      return a.head_dim == 64 ? launch_one<BF16, 64, 2>(a) : launch_one<BF16, 128, 2>(a);
    return a.head_dim == 64 ? launch_one<BF16, 64>(a) : launch_one<BF16, 128>(a);
  }
  if (a.heads_per_wave == 2)
    return a.head_dim == 64 ? launch_one<FP8, 64, 2>(a) : launch_one<FP8, 128, 2>(a);
  return a.head_dim == 64 ? launch_one<FP8, 64>(a) : launch_one<FP8, 128>(a);
}

}  // namespace pkv
