// Paged decode attention for gfx950.
//
// Decode streams a sequence's whole K/V history once per step and is bound by
// HBM bandwidth ("vLLM 引擎解剖", section "预填充、解码与三个时延指标"); the K/V
// of a sequence sit in 16-token blocks reached through its block table
// (section "PagedAttention：为 KV 缓存分页", Fig. 2).
//
// Work decomposition: one workgroup per (sequence, kv head, partition of the
// context).  Each wavefront of the workgroup owns up to four query heads of
// the kv head's group and walks the partition block by block; both waves of a
// two-wave workgroup read the same tiles, so the second read hits cache.
//
// Per block, one (block, kv head) tile of K and of V (16 rows x head_dim) is
// fetched with 16-byte loads:
//   K: lane = 4 * row + k; the four lanes of a quad read 64 contiguous bytes
//      of their row per load, so a quad holds the whole row after
//      head_dim*bytes/64 loads and the q.k dot product finishes with two DPP
//      quad exchanges;
//   V: consecutive lanes read consecutive 16-byte pieces (1 KiB per load);
//      a lane owns a fixed column slice and accumulates p * v over the rows
//      it loads.
// Scores go through LDS (16 x heads floats) from the K layout to the V
// layout.  Softmax is online, in base 2, with a running maximum shared by
// the wave that is only raised when a score exceeds it by more than 8 (a
// factor 256 in the weights, harmless in fp32), so the rescale branch is
// rare.  Each partition leaves (max, sum of weights, weighted sum of values)
// in the workspace; a second kernel merges the partitions of a sequence with
// the log-sum-exp rule.

#include <math.h>

#include "abi_util.h"
#include "common.h"
#include "prefill_args.h"

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRaiseThreshold = 8.0f;   // log2 units

#ifndef PKV_DECODE_MAX_HEADS_PER_WAVE
#define PKV_DECODE_MAX_HEADS_PER_WAVE 4
#endif
#ifndef PKV_DECODE_WAVES_PER_EU
#define PKV_DECODE_WAVES_PER_EU 3
#endif

template <typename QT, typename KVT, int D>
struct Geom {
  static constexpr int kRowBytes = D * KVT::bytes;
  static constexpr int kElems = 16 / KVT::bytes;       // elements per 16-byte piece
  // K: a row is split over kKLanes consecutive lanes, kKChunks 16-byte pieces
  // each; one pass covers kKRowsPerPass rows, kKPasses passes a tile.
  static constexpr int kKLanes = kRowBytes >= 128 ? 8 : 4;
  static constexpr int kKChunks = kRowBytes / (16 * kKLanes);
  static constexpr int kKRowsPerPass = kWave / kKLanes;
  static constexpr int kKPasses = kBlock / kKRowsPerPass;
  static constexpr int kKLoads = kKPasses * kKChunks;  // K loads per lane per tile
  // V: consecutive lanes read consecutive 16-byte pieces
  static constexpr int kVLanesPerRow = kRowBytes / 16;
  static constexpr int kVRowsPerLoad = kWave / kVLanesPerRow;
  static constexpr int kVLoads = kBlock / kVRowsPerLoad;  // V loads per lane per tile
  // q words per head per K piece (q dtype elements matching kElems)
  static constexpr int kQWords = kElems * QT::bytes / 4;
  static_assert(kKChunks >= 1 && kKPasses >= 1 && kVLoads >= 1, "unsupported row size");
};


// q . k over one 16-byte piece of a K row.
template <typename QT, typename KVT>
struct Dot;

template <>
struct Dot<BF16, BF16> {
  PKV_DEVICE static float run(const uint32_t* q, u32x4 k, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = dot2_bf16(q[i], k[i], acc);
    return acc;
  }
};

template <>
struct Dot<BF16, FP8> {
  PKV_DEVICE static float run(const uint32_t* q, u32x4 k, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = dot2_bf16(q[2 * i], fp8x2_to_bf16x2<false>(k[i]), acc);
      acc = dot2_bf16(q[2 * i + 1], fp8x2_to_bf16x2<true>(k[i]), acc);
    }
    return acc;
  }
};

template <>
struct Dot<F32, F32> {
  PKV_DEVICE static float run(const uint32_t* q, u32x4 k, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(q[i]), __uint_as_float(k[i]), acc);
    return acc;
  }
};

// A 16-byte piece of a V row -> its elements as fp32.
template <typename KVT>
struct Unpack;

template <>
struct Unpack<BF16> {
  PKV_DEVICE static void run(u32x4 v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_lo(v[i]);
      out[2 * i + 1] = bf16_hi(v[i]);
    }
  }
};

template <>
struct Unpack<FP8> {
  PKV_DEVICE static void run(u32x4 v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fp8x2_to_f32<false>(v[i], out[4 * i], out[4 * i + 1]);
      fp8x2_to_f32<true>(v[i], out[4 * i + 2], out[4 * i + 3]);
    }
  }
};

template <>
struct Unpack<F32> {
  PKV_DEVICE static void run(u32x4 v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  }
};

template <typename QT, typename KVT, int D, int GW>
struct DecodeWave {
  using G = Geom<QT, KVT, D>;
  using KS = typename KVT::storage;
  static constexpr int kQPieces = G::kQWords / 4;   // 16-byte q pieces per K piece
  // LDS of one wave: the q rows of its heads (read back as fragments every
  // block, so they cost no registers) and the 16 x GW weights of a block.
  static constexpr int kQBytes = GW * D * QT::bytes;
  static constexpr int kLdsBytes = kQBytes + kBlock * GW * 4;

  float acc[GW][G::kElems];
  float m[GW];      // running max of scaled scores (log2 units), wave-uniform
  float l[GW];      // this lane's share of the sum of weights
  int lane, krow, kq, vrow0, vcol;
  char* lds;        // this wave's LDS

  PKV_DEVICE const u32x4* qpiece(int h, int c, int w4) const {
    // 16-byte piece w4 of K piece (c * kKLanes + kq) of head h
    return reinterpret_cast<const u32x4*>(
        lds + h * D * QT::bytes + ((c * G::kKLanes + kq) * kQPieces + w4) * 16);
  }
  PKV_DEVICE float* plds() const { return reinterpret_cast<float*>(lds + kQBytes); }

  PKV_DEVICE void init(const typename QT::storage* qrow[GW], char* wave_lds) {
    lane = lane_id();
    krow = lane / G::kKLanes;
    kq = lane % G::kKLanes;
    vrow0 = lane / G::kVLanesPerRow;
    vcol = lane % G::kVLanesPerRow;
    lds = wave_lds;
    // q rows -> LDS, 16 bytes per lane per step
    constexpr int kRowPieces = D * QT::bytes / 16;
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      for (int pc = lane; pc < kRowPieces; pc += kWave)
        *reinterpret_cast<u32x4*>(lds + h * D * QT::bytes + pc * 16) =
            load16(reinterpret_cast<const char*>(qrow[h]) + pc * 16);
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < G::kElems; ++e) acc[h][e] = 0.f;
    }
    __builtin_amdgcn_wave_barrier();
  }

  // The K and V pieces of one tile, issued separately.  Each (block, kv head)
  // tile is addressed through a buffer resource (base and size in scalar
  // registers) plus a fixed per-lane offset, so the loads need no per-step
  // vector address arithmetic and cannot reach outside the tile.
  static constexpr int kTileBytes = kBlock * G::kRowBytes;
  PKV_DEVICE void load_k(u32x4 (&k)[G::kKLoads], const KS* ktile) const {
    const auto rk = tile_resource(ktile, kTileBytes);
    const uint32_t koff = uint32_t(krow * G::kRowBytes + kq * 16);
#pragma unroll
    for (int ps = 0; ps < G::kKPasses; ++ps)
#pragma unroll
      for (int c = 0; c < G::kKChunks; ++c)
        k[ps * G::kKChunks + c] = buffer_load16(
            rk, koff + (ps * G::kKRowsPerPass * G::kRowBytes + c * 16 * G::kKLanes));
  }
  PKV_DEVICE void load_v(u32x4 (&v)[G::kVLoads], const KS* vtile) const {
    const auto rv = tile_resource(vtile, kTileBytes);
    const uint32_t voff = uint32_t(lane * 16);
#pragma unroll
    for (int j = 0; j < G::kVLoads; ++j) v[j] = buffer_load16(rv, voff + j * 1024);
  }

  // Scores of one tile's rows (scaled, base 2), masked past valid_rows, and
  // whether any of them exceeds the running max by more than the threshold.
  PKV_DEVICE bool scores(const u32x4 (&k)[G::kKLoads], int valid_rows, float scale_log2,
                         float (&s)[G::kKPasses][GW]) const {
    bool raise = false;
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      uint32_t qf[G::kKChunks][G::kQWords];
#pragma unroll
      for (int c = 0; c < G::kKChunks; ++c)
#pragma unroll
        for (int w4 = 0; w4 < kQPieces; ++w4) {
          const u32x4 x = *qpiece(h, c, w4);
          qf[c][4 * w4] = x[0];
          qf[c][4 * w4 + 1] = x[1];
          qf[c][4 * w4 + 2] = x[2];
          qf[c][4 * w4 + 3] = x[3];
        }
#pragma unroll
      for (int ps = 0; ps < G::kKPasses; ++ps) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < G::kKChunks; ++c)
          a = Dot<QT, KVT>::run(qf[c], k[ps * G::kKChunks + c], a);
        a = quad_sum(a);
        if (G::kKLanes == 8) a += half_mirror(a);
        a *= scale_log2;
        a = (krow + ps * G::kKRowsPerPass < valid_rows) ? a : -INFINITY;
        s[ps][h] = a;
        raise |= a > m[h] + kRaiseThreshold;
      }
    }
    return raise;
  }

  // Raise the running max where a score exceeds it by more than the
  // threshold (rare: the branch only computes the new maxima; the rescale
  // itself is a multiply by 1 in the common case, which keeps the
  // accumulators in place instead of forking them across the branch), then
  // the weights -> LDS.
  PKV_DEVICE void weights(float (&s)[G::kKPasses][GW], bool raise) {
    float alpha[GW];
#pragma unroll
    for (int h = 0; h < GW; ++h) alpha[h] = 1.0f;
    if (__builtin_expect(__ballot(raise) != 0, 0)) {
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        float bm = s[0][h];
#pragma unroll
        for (int ps = 1; ps < G::kKPasses; ++ps) bm = fmaxf(bm, s[ps][h]);
        const float mn = fmaxf(m[h], wave_max(bm));
        alpha[h] = fast_exp2(m[h] - mn);
        m[h] = mn;
      }
    }
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      l[h] *= alpha[h];
#pragma unroll
      for (int e = 0; e < G::kElems; ++e) acc[h][e] *= alpha[h];
    }
    float* pl = plds();
#pragma unroll
    for (int ps = 0; ps < G::kKPasses; ++ps)
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        const float p = fast_exp2(s[ps][h] - m[h]);
        l[h] += p;
        if (kq == 0) pl[(krow + ps * G::kKRowsPerPass) * GW + h] = p;
      }
    __builtin_amdgcn_wave_barrier();
  }

  // acc += p * V over the tile's rows; rows past valid_rows hold anything
  // (unused slots), so their values are replaced by zeros.
  PKV_DEVICE void accumulate(const u32x4 (&v)[G::kVLoads], int valid_rows) {
    const float* pl = plds();
#pragma unroll
    for (int j = 0; j < G::kVLoads; ++j) {
      const int row = vrow0 + j * G::kVRowsPerLoad;
      float x[G::kElems];
      Unpack<KVT>::run(v[j], x);
      if (valid_rows < kBlock) {
        if (row >= valid_rows) {
#pragma unroll
          for (int e = 0; e < G::kElems; ++e) x[e] = 0.f;
        }
      }
#pragma unroll
      for (int h = 0; h < GW; ++h) {
        const float ph = pl[row * GW + h];
#pragma unroll
        for (int e = 0; e < G::kElems; ++e) acc[h][e] = fmaf(ph, x[e], acc[h][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
};

template <typename QT>
PKV_DEVICE void store_out(typename QT::storage* p, float v);
template <>
PKV_DEVICE void store_out<F32>(float* p, float v) { *p = v; }
template <>
PKV_DEVICE void store_out<BF16>(uint16_t* p, float v) { *p = f32_to_bf16(v); }


// Attend one wave's heads to tokens [start, end) of one sequence.
template <typename QT, typename KVT, int D, int GW>
PKV_DEVICE void attend_range(DecodeWave<QT, KVT, D, GW>& w,
                             const typename KVT::storage* k_cache,
                             const typename KVT::storage* v_cache,
                             int32_t num_blocks, const int32_t* table,
                             int32_t max_blocks, int kvh, int num_kv_heads,
                             int start, int end, float scale_log2) {
  using G = Geom<QT, KVT, D>;
  const int first_block = start / kBlock;
  const int nblocks = (end - start + kBlock - 1) / kBlock;
  const int last_rows = end - (first_block + nblocks - 1) * kBlock;
  const int64_t head_stride = int64_t(kBlock) * D;
  const int64_t block_stride = int64_t(num_kv_heads) * head_stride;
  auto tile_ptr = [&](const typename KVT::storage* base, int32_t b) {
    return base + int64_t(b) * block_stride + int64_t(kvh) * head_stride;
  };
  // Block ids come through the scalar cache, one block ahead of their use.
  auto id_at = [&](int blk) -> int32_t {
    const int lb = first_block + blk;
    return (blk < nblocks && lb < max_blocks) ? table[lb] : -1;
  };
  auto valid = [&](int32_t b) { return b >= 0 && b < num_blocks; };
  // One K and one V buffer: a block's K pieces are replaced by the next
  // block's as soon as its scores are computed, its V pieces as soon as they
  // are accumulated, so the next tile is always in flight while the current
  // one is worked on.  Past the last block (or for an invalid id) the loads
  // re-read the current block, a cache hit, and the tile is fully masked:
  // every step has the same loads in flight on every path.
  u32x4 kt[G::kKLoads], vt[G::kVLoads];
  int32_t id_cur = id_at(0);
  int32_t id_nxt = id_at(1);
  {
    const int32_t b0 = valid(id_cur) ? id_cur : 0;
    w.load_k(kt, tile_ptr(k_cache, b0));
    // keep K ahead of V in the memory queue, as inside the loop
    __builtin_amdgcn_sched_barrier(0);
    w.load_v(vt, tile_ptr(v_cache, b0));
  }
  for (int i = 0; i < nblocks; ++i) {
    const int32_t id_after = id_at(i + 2);
    const int rows = valid(id_cur) ? (i + 1 < nblocks ? kBlock : last_rows) : 0;
    const int32_t bn = valid(id_nxt) ? id_nxt : (valid(id_cur) ? id_cur : 0);
    float s[G::kKPasses][GW];
    const bool raise = w.scores(kt, rows, scale_log2, s);
    w.load_k(kt, tile_ptr(k_cache, bn));
    w.weights(s, raise);
    w.accumulate(vt, rows);
    w.load_v(vt, tile_ptr(v_cache, bn));
    id_cur = id_nxt;
    id_nxt = id_after;
  }
  // merge the row groups that share a column slice, and the rows' sums
  using G = Geom<QT, KVT, D>;
#pragma unroll
  for (int h = 0; h < GW; ++h) {
#pragma unroll
    for (int e = 0; e < G::kElems; ++e) {
      float a = w.acc[h][e];
#pragma unroll
      for (int mask = G::kVLanesPerRow; mask < kWave; mask <<= 1) a += shfl_xor(a, mask);
      w.acc[h][e] = a;
    }
    w.l[h] = wave_sum(w.kq == 0 ? w.l[h] : 0.f);
  }
}

// Decode: grid (partition, kv head, sequence); writes per-partition partials.
template <typename QT, typename KVT, int D, int GW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PKV_DECODE_WAVES_PER_EU))) void decode_partition_kernel(
    const typename QT::storage* __restrict__ query,
    const typename KVT::storage* __restrict__ k_cache,
    const typename KVT::storage* __restrict__ v_cache, int32_t num_blocks,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t group, float scale_log2,
    int32_t partition_tokens, int32_t max_parts, float* __restrict__ part_out,
    float* __restrict__ part_ml) {
  using G = Geom<QT, KVT, D>;
  using W = DecodeWave<QT, KVT, D, GW>;
  __shared__ __align__(16) char lds_all[4][W::kLdsBytes];
  // (sequence, kv head) pairs are the fastest grid dimension: consecutive
  // workgroups are dealt to the eight XCDs in turn, so each XCD gets an even
  // share of every partition index (partitions past a short sequence's end
  // exit at once and would otherwise pile the work onto a few XCDs).
  const int kvh = blockIdx.x % num_kv_heads;
  const int seq = blockIdx.x / num_kv_heads;
  const int part = blockIdx.y;
  const int wave = threadIdx.x / kWave;
  const int len = min(context_lens[seq], max_parts * partition_tokens);
  const int start = part * partition_tokens;
  if (start >= len) return;
  const int end = min(len, start + partition_tokens);

  const int head0 = kvh * group + wave * GW;
  const int heads_here = min(GW, group - wave * GW);
  const typename QT::storage* qrow[GW];
#pragma unroll
  for (int h = 0; h < GW; ++h)
    qrow[h] = query + (int64_t(seq) * num_q_heads + head0 + (h < heads_here ? h : 0)) * D;
  W w;
  w.init(qrow, lds_all[wave]);
  attend_range(w, k_cache, v_cache, num_blocks, block_tables + int64_t(seq) * max_blocks,
               max_blocks, kvh, num_kv_heads, start, end, scale_log2);
  if (w.lane < G::kVLanesPerRow) {
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      if (h >= heads_here) break;
      const int64_t idx = (int64_t(seq) * num_q_heads + head0 + h) * max_parts + part;
      float* o = part_out + idx * D + w.vcol * G::kElems;
#pragma unroll
      for (int e = 0; e < G::kElems; e += 4)
        *reinterpret_cast<float4*>(o + e) =
            make_float4(w.acc[h][e], w.acc[h][e + 1], w.acc[h][e + 2], w.acc[h][e + 3]);
      if (w.lane == 0) {
        part_ml[2 * idx] = w.m[h];
        part_ml[2 * idx + 1] = w.l[h];
      }
    }
  }
}

// Chunked prefill on the vector units (dtypes and head sizes without an
// MFMA kernel): grid (1, kv head, query row); each query row attends to its
// whole causal context, so the output is final.
template <typename QT, typename KVT, int D, int GW>
__global__ __launch_bounds__(256) void prefill_rows_kernel(
    typename QT::storage* __restrict__ out,
    const typename QT::storage* __restrict__ query,
    const typename KVT::storage* __restrict__ k_cache,
    const typename KVT::storage* __restrict__ v_cache, int32_t num_blocks,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ query_start_loc,
    const int32_t* __restrict__ num_computed, int32_t num_reqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t group, float scale_log2,
    float v_scale) {
  using G = Geom<QT, KVT, D>;
  using W = DecodeWave<QT, KVT, D, GW>;
  __shared__ __align__(16) char lds_all[4][W::kLdsBytes];
  const int kvh = blockIdx.x % num_kv_heads;
  const int row = blockIdx.x / num_kv_heads;
  const int wave = threadIdx.x / kWave;
  // the request owning this row: last r with query_start_loc[r] <= row
  int lo = 0, hi = num_reqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (query_start_loc[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  const int len = num_computed[r] + (row - query_start_loc[r]) + 1;
  const int head0 = kvh * group + wave * GW;
  const int heads_here = min(GW, group - wave * GW);
  const typename QT::storage* qrow[GW];
#pragma unroll
  for (int h = 0; h < GW; ++h)
    qrow[h] = query + (int64_t(row) * num_q_heads + head0 + (h < heads_here ? h : 0)) * D;
  W w;
  w.init(qrow, lds_all[wave]);
  const int cap = min(len, max_blocks * kBlock);
  if (cap > 0)
    attend_range(w, k_cache, v_cache, num_blocks, block_tables + int64_t(r) * max_blocks,
                 max_blocks, kvh, num_kv_heads, 0, cap, scale_log2);
  if (w.lane < G::kVLanesPerRow) {
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      if (h >= heads_here) break;
      typename QT::storage* o =
          out + (int64_t(row) * num_q_heads + head0 + h) * D + w.vcol * G::kElems;
      const float f = cap > 0 ? v_scale / w.l[h] : 0.f;
#pragma unroll
      for (int e = 0; e < G::kElems; ++e) store_out<QT>(o + e, w.acc[h][e] * f);
    }
  }
}

// One workgroup (one wave) per (head, sequence): merge the partitions,
//   out = sum_k e^{m_k - M} o_k / sum_k e^{m_k - M} l_k,   M = max_k m_k
// (m in log2 units).  The weights of up to 64 partitions at a time are
// computed one per lane and passed through LDS, so the partials' loads do not
// wait on each other.
template <typename QT, int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(
    typename QT::storage* __restrict__ out, const float* __restrict__ part_out,
    const float* __restrict__ part_ml, const int32_t* __restrict__ context_lens,
    int32_t num_q_heads, int32_t partition_tokens, int32_t max_parts,
    float v_scale) {
  constexpr int kPer = D / kWave;
  __shared__ float wts[kWave];
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int lane = threadIdx.x;
  const int len = min(context_lens[seq], max_parts * partition_tokens);
  typename QT::storage* o = out + (int64_t(seq) * num_q_heads + h) * D;
  if (len <= 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) store_out<QT>(o + lane + i * kWave, 0.f);
    return;
  }
  const int nparts = (len + partition_tokens - 1) / partition_tokens;
  const int64_t base = (int64_t(seq) * num_q_heads + h) * max_parts;
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + base;
  float big = -INFINITY;
  for (int k = lane; k < nparts; k += kWave) big = fmaxf(big, ml[k].x);
  big = wave_max(big);
  float acc[kPer] = {};
  float den = 0.f;
  for (int k0 = 0; k0 < nparts; k0 += kWave) {
    const int k = k0 + lane;
    float w = 0.f;
    if (k < nparts) {
      const float2 x = ml[k];
      w = fast_exp2(x.x - big);
      den = fmaf(w, x.y, den);
    }
    wts[lane] = w;
    __syncthreads();
    const int n = min(kWave, nparts - k0);
    const float* po = part_out + (base + k0) * D + lane;
    int j = 0;
    for (; j + 4 <= n; j += 4) {
      float x[4][kPer];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < kPer; ++i) x[u][i] = po[(j + u) * D + i * kWave];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < kPer; ++i) acc[i] = fmaf(wts[j + u], x[u][i], acc[i]);
    }
    for (; j < n; ++j)
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] = fmaf(wts[j], po[j * D + i * kWave], acc[i]);
    __syncthreads();
  }
  den = wave_sum(den);
  const float f = v_scale / den;
#pragma unroll
  for (int i = 0; i < kPer; ++i) store_out<QT>(o + lane + i * kWave, acc[i] * f);
}

// ------------------------------------------------------------------ host

// 512 tokens (32 blocks) per partition: long enough to amortise a
// workgroup's start and the merge, short enough that the longest per-wave
// chain of dependent block loads stays well under the kernel's duration.
int32_t choose_partition(int32_t max_context_len, int32_t requested) {
  (void)max_context_len;
  return requested > 0 ? requested : 512;
}

static size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

struct WorkspaceLayout {
  int32_t part_tokens, max_parts;
  size_t out_bytes, ml_bytes;
};

static WorkspaceLayout layout(int32_t s, int32_t hq, int32_t d, int32_t max_len,
                              int32_t requested) {
  WorkspaceLayout w;
  w.part_tokens = choose_partition(max_len, requested);
  w.max_parts = max_len <= 0 ? 1 : (max_len + w.part_tokens - 1) / w.part_tokens;
  w.out_bytes = align256(size_t(s) * hq * w.max_parts * d * sizeof(float));
  w.ml_bytes = align256(size_t(s) * hq * w.max_parts * 2 * sizeof(float));
  return w;
}

template <typename QT, typename KVT, int D, int GW>
static pkv_status launch_decode(void* out, const void* q, const void* kc,
                                const void* vc, int32_t nb, const int32_t* bt,
                                int32_t maxb, const int32_t* lens, int32_t s,
                                int32_t hq, int32_t hkv, float scale_log2,
                                float v_scale, const WorkspaceLayout& lay,
                                void* ws, hipStream_t st) {
  const int group = hq / hkv;
  const int waves = (group + GW - 1) / GW;
  float* part_out = static_cast<float*>(ws);
  float* part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.out_bytes);
  hipLaunchKernelGGL((decode_partition_kernel<QT, KVT, D, GW>),
                     dim3(s * hkv, lay.max_parts), dim3(kWave * waves), 0, st,
                     static_cast<const typename QT::storage*>(q),
                     static_cast<const typename KVT::storage*>(kc),
                     static_cast<const typename KVT::storage*>(vc), nb, bt, maxb,
                     lens, hq, hkv, group, scale_log2, lay.part_tokens,
                     lay.max_parts, part_out, part_ml);
  if (launch_status() != PKV_OK) return PKV_ERR_LAUNCH;
  hipLaunchKernelGGL((decode_reduce_kernel<QT, D>), dim3(hq, s), dim3(kWave), 0, st,
                     static_cast<typename QT::storage*>(out), part_out, part_ml,
                     lens, hq, lay.part_tokens, lay.max_parts, v_scale);
  return launch_status();
}

template <typename QT, typename KVT, int D>
static pkv_status dispatch_gw(int gw, void* out, const void* q, const void* kc,
                              const void* vc, int32_t nb, const int32_t* bt,
                              int32_t maxb, const int32_t* lens, int32_t s,
                              int32_t hq, int32_t hkv, float sl2, float vs,
                              const WorkspaceLayout& lay, void* ws, hipStream_t st) {
  switch (gw) {
    case 1: return launch_decode<QT, KVT, D, 1>(out, q, kc, vc, nb, bt, maxb, lens, s, hq, hkv, sl2, vs, lay, ws, st);
    case 2: return launch_decode<QT, KVT, D, 2>(out, q, kc, vc, nb, bt, maxb, lens, s, hq, hkv, sl2, vs, lay, ws, st);
    case 3: return launch_decode<QT, KVT, D, 3>(out, q, kc, vc, nb, bt, maxb, lens, s, hq, hkv, sl2, vs, lay, ws, st);
    case 4: return launch_decode<QT, KVT, D, 4>(out, q, kc, vc, nb, bt, maxb, lens, s, hq, hkv, sl2, vs, lay, ws, st);
    default: return PKV_ERR_UNSUPPORTED;
  }
}

template <typename QT, typename KVT, int D, int GW>
static pkv_status launch_rows(const PrefillArgs& a, int waves) {
  hipLaunchKernelGGL((prefill_rows_kernel<QT, KVT, D, GW>),
                     dim3(a.num_kv_heads * a.num_q_tokens), dim3(kWave * waves), 0,
                     as_stream(a.stream), static_cast<typename QT::storage*>(a.out),
                     static_cast<const typename QT::storage*>(a.query),
                     static_cast<const typename KVT::storage*>(a.k_cache),
                     static_cast<const typename KVT::storage*>(a.v_cache),
                     a.num_blocks, a.block_tables, a.max_blocks_per_seq,
                     a.query_start_loc, a.num_computed_tokens, a.num_reqs,
                     a.num_q_heads, a.num_kv_heads, a.num_q_heads / a.num_kv_heads,
                     a.softmax_scale * a.k_scale * kLog2e, a.v_scale);
  return launch_status();
}

template <typename QT, typename KVT, int D>
static pkv_status rows_gw(const PrefillArgs& a, int gw, int waves) {
  switch (gw) {
    case 1: return launch_rows<QT, KVT, D, 1>(a, waves);
    case 2: return launch_rows<QT, KVT, D, 2>(a, waves);
    case 3: return launch_rows<QT, KVT, D, 3>(a, waves);
    case 4: return launch_rows<QT, KVT, D, 4>(a, waves);
    default: return PKV_ERR_UNSUPPORTED;
  }
}

// Prefill chunks on the vector units: one workgroup per (query row, kv head).
pkv_status launch_prefill_rows(const PrefillArgs& a) {
  const bool f32 = a.q_dtype == PKV_F32 && a.kv_dtype == PKV_F32;
  const bool bf16 = a.q_dtype == PKV_BF16 && a.kv_dtype == PKV_BF16;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int max_gw = (f32 && a.head_dim == 128) ? 2 : 4;
  const int waves = (group + max_gw - 1) / max_gw;
  const int gw = (group + waves - 1) / waves;
  if (f32)
    return a.head_dim == 64 ? rows_gw<F32, F32, 64>(a, gw, waves)
                            : rows_gw<F32, F32, 128>(a, gw, waves);
  if (bf16)
    return a.head_dim == 64 ? rows_gw<BF16, BF16, 64>(a, gw, waves)
                            : rows_gw<BF16, BF16, 128>(a, gw, waves);
  return a.head_dim == 64 ? rows_gw<BF16, FP8, 64>(a, gw, waves)
                          : rows_gw<BF16, FP8, 128>(a, gw, waves);
}

}  // namespace pkv

using namespace pkv;

extern "C" int32_t paged_attention_decode_partition_tokens(int32_t num_seqs,
                                                           int32_t num_kv_heads,
                                                           int32_t max_context_len,
                                                           int32_t partition_tokens) {
  (void)num_seqs;
  (void)num_kv_heads;
  return choose_partition(max_context_len, partition_tokens);
}

extern "C" size_t paged_attention_decode_workspace_size(int32_t num_seqs,
                                                        int32_t num_q_heads,
                                                        int32_t num_kv_heads,
                                                        int32_t head_dim,
                                                        int32_t max_context_len,
                                                        int32_t partition_tokens) {
  (void)num_kv_heads;
  if (num_seqs < 0 || num_q_heads < 0 || head_dim < 0 || max_context_len < 0)
    return 0;
  const WorkspaceLayout w =
      layout(num_seqs, num_q_heads, head_dim, max_context_len, partition_tokens);
  return w.out_bytes + w.ml_bytes;
}

extern "C" pkv_status paged_attention_decode(
    void* out, const void* query, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    float softmax_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype, float k_scale,
    float v_scale, int32_t partition_tokens, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq < 0 ||
      max_context_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0)
    return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (int64_t(max_blocks_per_seq) * kBlock < max_context_len) return PKV_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  if (group > 8) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (partition_tokens < 0 || partition_tokens % kBlock != 0 || partition_tokens > 1024)
    return PKV_ERR_SHAPE;
  const bool f32 = q_dtype == PKV_F32 && kv_dtype == PKV_F32;
  const bool bf16 = q_dtype == PKV_BF16 && kv_dtype == PKV_BF16;
  const bool fp8 = q_dtype == PKV_BF16 && kv_dtype == PKV_FP8_E4M3;
  if (!(f32 || bf16 || fp8)) return PKV_ERR_UNSUPPORTED;
  if (!fp8) k_scale = v_scale = 1.0f;
  if (!(k_scale > 0.f && v_scale > 0.f)) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (num_blocks == 0) return PKV_ERR_SHAPE;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens)
    return PKV_ERR_NULL;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PKV_ERR_ALIGN;
  const WorkspaceLayout lay =
      layout(num_seqs, num_q_heads, head_dim, max_context_len, partition_tokens);
  if (!workspace || workspace_bytes < lay.out_bytes + lay.ml_bytes)
    return PKV_ERR_WORKSPACE;
  if (lay.max_parts > 65535 || int64_t(num_seqs) * num_kv_heads > 0x7fffffff)
    return PKV_ERR_SHAPE;
  if (!aligned(workspace, 16)) return PKV_ERR_ALIGN;

  // fp32 q with head_dim 128 keeps at most two heads per wave (registers)
  const int max_gw = (f32 && head_dim == 128) ? 2 : PKV_DECODE_MAX_HEADS_PER_WAVE;
  const int waves = (group + max_gw - 1) / max_gw;
  const int gw = (group + waves - 1) / waves;
  const float scale_log2 = softmax_scale * k_scale * kLog2e;
  hipStream_t st = as_stream(stream);
  const int32_t nb = num_blocks, maxb = max_blocks_per_seq;
#define PKV_DECODE_ARGS gw, out, query, k_cache, v_cache, nb, block_tables, maxb, \
    context_lens, num_seqs, num_q_heads, num_kv_heads, scale_log2, v_scale, lay, workspace, st
  if (f32) {
    return head_dim == 64 ? dispatch_gw<F32, F32, 64>(PKV_DECODE_ARGS)
                          : dispatch_gw<F32, F32, 128>(PKV_DECODE_ARGS);
  }
  if (bf16) {
    return head_dim == 64 ? dispatch_gw<BF16, BF16, 64>(PKV_DECODE_ARGS)
                          : dispatch_gw<BF16, BF16, 128>(PKV_DECODE_ARGS);
  }
  return head_dim == 64 ? dispatch_gw<BF16, FP8, 64>(PKV_DECODE_ARGS)
                        : dispatch_gw<BF16, FP8, 128>(PKV_DECODE_ARGS);
#undef PKV_DECODE_ARGS
}
