// Paged decode attention for gfx950.
//
// Decode streams a sequence's whole K/V history once per step and is bound by
// HBM bandwidth ("vLLM 引擎解剖", section "预填充、解码与三个时延指标"); the K/V
// of a sequence sit in 16-token blocks reached through its block table
// (section "PagedAttention：为 KV 缓存分页", Fig. 2).
//
// Work decomposition (decode_sched.h): the batch's blocks are laid end to
// end -- sequence 0's, then sequence 1's, ... -- and cut into equal chunks.
// The vector kernel below runs one workgroup per (chunk, kv head); each wave
// of it owns up to four query heads of the kv head's group and walks the
// chunk block by block, crossing sequence boundaries (a wave that finishes a
// sequence inside its chunk writes that sequence's output).  A sequence that
// spans several chunks leaves one partial per chunk, in record (chunk +
// sequence) of the workspace; decode_merge_kernel combines them.  (The
// matrix-core kernel, decode_mfma.hip, whose waves may walk several chunks,
// folds a wave's chunks of one sequence into one record, at the chunk where
// that wave's part of the sequence starts; the merge is told how many chunks
// a wave walks.)
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
// rare.  Each partial is (max, sum of weights, weighted sum of values), and
// the merge combines a sequence's partials with the log-sum-exp rule.

#include <math.h>

#include <algorithm>

#include <type_traits>

#include "abi_util.h"
#include "common.h"
#include "decode_mfma.h"
#include "decode_sched.h"
#include "prefill_args.h"

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRaiseThreshold = 8.0f;   // log2 units
// Running max before any key: finite, so that a fully masked block gives
// weights 2^-inf = 0 rather than 2^(-inf + inf).
constexpr float kNoMax = -1e30f;

#ifndef PKV_DECODE_DEPTH
#define PKV_DECODE_DEPTH 1
#endif
#ifndef PKV_DECODE_MAX_HEADS_PER_WAVE
#define PKV_DECODE_MAX_HEADS_PER_WAVE 4
#endif
// bf16 queries go to the matrix-core kernel (decode_mfma.hip); 0 keeps every
// dtype on the vector kernel below.
#ifndef PKV_DECODE_USE_MFMA
#define PKV_DECODE_USE_MFMA 1
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

  PKV_DEVICE void init(char* wave_lds) {
    lane = lane_id();
    krow = lane / G::kKLanes;
    kq = lane % G::kKLanes;
    vrow0 = lane / G::kVLanesPerRow;
    vcol = lane % G::kVLanesPerRow;
    lds = wave_lds;
#pragma unroll
    for (int h = 0; h < GW; ++h) {
      m[h] = kNoMax;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < G::kElems; ++e) acc[h][e] = 0.f;
    }
  }

  // The wave's q rows in 16-byte pieces, a few per lane, fetched into
  // registers and later staged to LDS (where they are read as fragments).
  static constexpr int kQRowPieces = D * QT::bytes / 16;
  static constexpr int kQLanePieces = (GW * kQRowPieces + kWave - 1) / kWave;
  struct QFetch {
    u32x4 v[kQLanePieces];
  };
  // `rows` points at the first of the wave's heads (consecutive in memory);
  // pieces of heads past `heads` read as zeros through the buffer bounds.
  PKV_DEVICE QFetch fetch_q(const typename QT::storage* rows, int heads) const {
    const auto rq = tile_resource(rows, heads * kQRowPieces * 16);
    QFetch f;
#pragma unroll
    for (int i = 0; i < kQLanePieces; ++i) f.v[i] = buffer_load16_cached(rq, (i * kWave + lane) * 16);
    return f;
  }
  PKV_DEVICE void stage_q(const QFetch& f) {
#pragma unroll
    for (int i = 0; i < kQLanePieces; ++i) {
      const int piece = i * kWave + lane;
      if (piece < GW * kQRowPieces) *reinterpret_cast<u32x4*>(lds + piece * 16) = f.v[i];
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


// The table entries of the first PKV_DECODE_DEPTH + 1 blocks from `first_block`
// (-1 past the table's end), read before the range itself is known so that
// these scalar loads overlap the others at the start of a kernel.
PKV_DEVICE void prefetch_ids(const int32_t* table, int first_block, int max_blocks,
                             int32_t (&ids)[PKV_DECODE_DEPTH + 1]) {
#pragma unroll
  for (int d = 0; d <= PKV_DECODE_DEPTH; ++d)
    ids[d] = first_block + d < max_blocks ? table[first_block + d] : -1;
}

// Attend one wave's heads to tokens [start, end) of one sequence.
template <typename QT, typename KVT, int D, int GW>
PKV_DEVICE void attend_range(DecodeWave<QT, KVT, D, GW>& w,
                             const typename KVT::storage* k_cache,
                             const typename KVT::storage* v_cache,
                             int32_t num_blocks, const int32_t* table,
                             int32_t max_blocks, int kvh, int num_kv_heads,
                             int start, int end, float scale_log2,
                             const typename DecodeWave<QT, KVT, D, GW>::QFetch& qv,
                             const int32_t (&first_ids)[PKV_DECODE_DEPTH + 1]) {
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
  // kDepth K buffers and kDepth V buffers used in turn: a block's K pieces are
  // replaced by those of the block kDepth ahead as soon as its scores are
  // computed, its V pieces as soon as they are accumulated, so the next
  // kDepth tiles are always in flight while the current one is worked on.
  // Past the last block (or for an invalid id) the loads re-read a block
  // already read, a cache hit, and the tile is fully masked: every step has
  // the same loads in flight on every path, so every wait is exact.
  constexpr int kDepth = PKV_DECODE_DEPTH;
  u32x4 kt[kDepth][G::kKLoads], vt[kDepth][G::kVLoads];
  int32_t ids[kDepth + 1];
#pragma unroll
  for (int d = 0; d <= kDepth; ++d) ids[d] = d < nblocks ? first_ids[d] : -1;
  const int32_t b_first = valid(ids[0]) ? ids[0] : 0;
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    const int32_t b = valid(ids[d]) ? ids[d] : b_first;
    w.load_k(kt[d], tile_ptr(k_cache, b));
    // keep each K ahead of its V in the memory queue, as inside the loop
    __builtin_amdgcn_sched_barrier(0);
    w.load_v(vt[d], tile_ptr(v_cache, b));
    __builtin_amdgcn_sched_barrier(0);
  }
  // q was fetched before the tiles: staging it waits only for its own load
  w.stage_q(qv);
  auto step = [&](auto slot_c, int i) {
    constexpr int S = decltype(slot_c)::value;
    // ids[0] is block i, ids[kDepth] block i + kDepth
    const int32_t id_cur = ids[0];
    const int rows = valid(id_cur) ? (i + 1 < nblocks ? kBlock : last_rows) : 0;
    const int32_t bn = valid(ids[kDepth]) ? ids[kDepth] : (valid(id_cur) ? id_cur : b_first);
    const int32_t id_new = id_at(i + kDepth + 1);
    float s[G::kKPasses][GW];
    const bool raise = w.scores(kt[S], rows, scale_log2, s);
    w.load_k(kt[S], tile_ptr(k_cache, bn));
    w.weights(s, raise);
    w.accumulate(vt[S], rows);
    w.load_v(vt[S], tile_ptr(v_cache, bn));
#pragma unroll
    for (int d = 0; d < kDepth; ++d) ids[d] = ids[d + 1];
    ids[kDepth] = id_new;
  };
  for (int i = 0; i < nblocks; i += kDepth) {
    step(std::integral_constant<int, 0>{}, i);
    if (kDepth > 1) {
      if (i + 1 >= nblocks) break;
      step(std::integral_constant<int, (kDepth > 1 ? 1 : 0)>{}, i + 1);
    }
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

// Decode: one workgroup per (chunk, kv head); each wave owns up to GW query
// heads of the kv head.
template <typename QT, typename KVT, int D, int GW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PKV_DECODE_WAVES_PER_EU))) void decode_chunk_kernel(
    typename QT::storage* __restrict__ out,
    const typename QT::storage* __restrict__ query,
    const typename KVT::storage* __restrict__ k_cache,
    const typename KVT::storage* __restrict__ v_cache, int32_t num_blocks,
    const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t max_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t group, float scale_log2,
    float v_scale, int32_t num_chunks, int32_t fixed_chunk, float* __restrict__ rec_out,
    float* __restrict__ rec_ml) {
  using G = Geom<QT, KVT, D>;
  using W = DecodeWave<QT, KVT, D, GW>;
  __shared__ __align__(16) char lds_all[4][W::kLdsBytes];
  // kv heads are the fastest grid dimension: the workgroups of one chunk
  // read neighbouring tiles of the same blocks
  const int kvh = blockIdx.x % num_kv_heads;
  const int g = blockIdx.x / num_kv_heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int head0 = kvh * group + wave * GW;
  const int heads_here = min(GW, group - wave * GW);

  const BatchScan sc = scan_batch(context_lens, num_seqs, max_len);
  const int c = chunk_blocks(sc.total, num_chunks, fixed_chunk);
  const int b0 = g * c;
  if (b0 >= sc.total) return;
  const int b1 = min(b0 + c, sc.total);
  int s, before;
  locate(sc, context_lens, max_len, b0, s, before);
  W w;
  for (;;) {
    const int len = seq_len(sc, context_lens, s, max_len);
    const int n = blocks_of(len);
    const int lo = max(b0, before), hi = min(b1, before + n);
    if (lo < hi) {
      const bool whole = lo == before && hi == before + n;
      w.init(lds_all[wave]);
      const auto qv = w.fetch_q(query + (int64_t(s) * num_q_heads + head0) * D, heads_here);
      const int32_t* table = block_tables + int64_t(s) * max_blocks;
      int32_t ids[PKV_DECODE_DEPTH + 1];
      prefetch_ids(table, lo - before, max_blocks, ids);
      attend_range(w, k_cache, v_cache, num_blocks, table, max_blocks, kvh, num_kv_heads,
                   (lo - before) * kBlock, min(len, (hi - before) * kBlock), scale_log2, qv,
                   ids);
      if (w.lane < G::kVLanesPerRow) {
#pragma unroll
        for (int h = 0; h < GW; ++h) {
          if (h >= heads_here) break;
          if (whole) {
            typename QT::storage* o =
                out + (int64_t(s) * num_q_heads + head0 + h) * D + w.vcol * G::kElems;
            const float f = v_scale / w.l[h];
#pragma unroll
            for (int e = 0; e < G::kElems; ++e) store_out<QT>(o + e, w.acc[h][e] * f);
          } else {
            const int64_t idx = int64_t(g + s) * num_q_heads + head0 + h;
            float* o = rec_out + idx * D + w.vcol * G::kElems;
#pragma unroll
            for (int e = 0; e < G::kElems; e += 4)
              *reinterpret_cast<float4*>(o + e) =
                  make_float4(w.acc[h][e], w.acc[h][e + 1], w.acc[h][e + 2], w.acc[h][e + 3]);
            if (w.lane == 0) reinterpret_cast<float2*>(rec_ml)[idx] = make_float2(w.m[h], w.l[h]);
          }
        }
      }
    }
    before += n;
    ++s;
    if (before >= b1 || s >= num_seqs) break;
  }
}

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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
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
  W w;
  w.init(lds_all[wave]);
  const auto qv = w.fetch_q(query + (int64_t(row) * num_q_heads + head0) * D, heads_here);
  const int32_t* table = block_tables + int64_t(r) * max_blocks;
  int32_t ids[PKV_DECODE_DEPTH + 1];
  prefetch_ids(table, 0, max_blocks, ids);
  const int cap = min(len, max_blocks * kBlock);
  if (cap > 0)
    attend_range(w, k_cache, v_cache, num_blocks, table, max_blocks, kvh, num_kv_heads, 0,
                 cap, scale_log2, qv, ids);
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

// One workgroup of W waves per (head, sequence): merge the partials of a
// sequence that spans several chunks,
//   out = sum_k e^{m_k - M} o_k / sum_k e^{m_k - M} l_k,   M = max_k m_k
// (m in log2 units).  Sequences inside one chunk were written by the chunk
// kernel; empty ones get zeros here.  The weights are computed one partial
// per lane, so the partials' vector loads do not wait on each other.
// W = 4 for fixed partitions, which leave tens to hundreds of partials per
// sequence: wave w of the unit takes partials w, w + 4, w + 8, ..., reads
// each weight back from its lane, loads eight partials' vectors before using
// any, and the waves' sums meet in LDS at the end.  W = 1 for the library's
// own split, which leaves a few: up to kFewParts of them are merged from one
// round of loads, pairs and vectors together; more go in groups of 64 whose
// weights pass through LDS.
constexpr int kFewParts = 8;   // partials merged by the single-load path
// With W = 1 a workgroup carries this many (head, sequence) units, one per
// wave, each on its own (no workgroup barrier): a quarter of the workgroups
// to dispatch.
constexpr int kMergeUnits = 4;

template <int W>
constexpr int merge_waves() { return W == 1 ? kMergeUnits : W; }

template <typename QT, int D, int W>
__global__ __launch_bounds__(kWave * merge_waves<W>()) void decode_merge_kernel(
    typename QT::storage* __restrict__ out, const float* __restrict__ rec_out,
    const float* __restrict__ rec_ml, const int32_t* __restrict__ context_lens,
    int32_t num_seqs, int32_t max_len, int32_t num_q_heads, int32_t num_chunks,
    int32_t fixed_chunk, int32_t chunks_per_wave, float v_scale, int32_t window) {
  constexpr int kPer = D / kWave;
  __shared__ float wts[merge_waves<W>()][kWave];
  __shared__ float part[W][D + 2];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int h = W == 1 ? int(blockIdx.x) * kMergeUnits + wave : int(blockIdx.x);
  const int seq = blockIdx.y;
  if (W == 1 && h >= num_q_heads) return;
  const BatchScan sc = scan_batch(context_lens, num_seqs, max_len, window);
  const int owner = seq / sc.k;
  int before = __builtin_amdgcn_readlane(sc.first, owner);
  for (int t = owner * sc.k; t < seq; ++t)
    before += window_blocks(seq_len(sc, context_lens, t, max_len), window);
  const int n = window_blocks(seq_len(sc, context_lens, seq, max_len), window);
  typename QT::storage* o = out + (int64_t(seq) * num_q_heads + h) * D;
  if (n == 0) {
    if (W == 1 || wave == 0) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) store_out<QT>(o + lane + i * kWave, 0.f);
    }
    return;
  }
  const int c = chunk_blocks(sc.total, num_chunks, fixed_chunk);
  const int g0 = before / c, g1 = (before + n - 1) / c;
  // one record per wave that walked part of the sequence (a wave walks
  // chunks_per_wave consecutive chunks): wave w0 + k's record sits at chunk
  // g0 (k = 0) or (w0 + k) * chunks_per_wave, in record chunk + seq
  const int w0 = g0 / chunks_per_wave, w1 = g1 / chunks_per_wave;
  if (w0 == w1) return;              // one wave walked it all and wrote it
  const int nparts = w1 - w0 + 1;
  const int64_t base = int64_t(g0 + seq) * num_q_heads + h;
  const int64_t stride = num_q_heads;
  // record offset of part k from `base`, in records of one head
  auto at = [&](int k) -> int64_t {
    return (k == 0 ? 0 : int64_t(w0 + k) * chunks_per_wave - g0) * stride;
  };
  const float2* ml = reinterpret_cast<const float2*>(rec_ml) + base;
  if (W == 1 && nparts <= kFewParts) {
    // A few partials (the library's own split): their (max, sum) pairs and
    // their vectors are loaded at once, so the vectors do not wait for the
    // weights; lane k < nparts holds partial k's pair.
    float x[kFewParts][kPer];
    const float* po = rec_out + base * D + lane;
#pragma unroll
    for (int j = 0; j < kFewParts; ++j)
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        x[j][i] = j < nparts ? po[at(j) * D + i * kWave] : 0.f;
    const float2 mine = lane < nparts ? ml[at(lane)] : make_float2(-INFINITY, 0.f);
    // the pairs sit in lanes 0..kFewParts-1 (the rest hold -inf, 0): read
    // lane by lane; the weighted sum in the tree a butterfly over the wave
    // would take, ((d0 + d1) + (d2 + d3)) + ((d4 + d5) + (d6 + d7))
    static_assert(kFewParts == 8, "the sum tree below is written for eight partials");
    auto lane_f = [](float v, int k) {
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
    };
    float big = lane_f(mine.x, 0);
#pragma unroll
    for (int k = 1; k < kFewParts; ++k) big = fmaxf(big, lane_f(mine.x, k));
    const float wk = lane < nparts ? fast_exp2(mine.x - big) : 0.f;
    const float dk = wk * mine.y;
    float d[kFewParts];
#pragma unroll
    for (int k = 0; k < kFewParts; ++k) d[k] = lane_f(dk, k);
    const float den = ((d[0] + d[1]) + (d[2] + d[3])) + ((d[4] + d[5]) + (d[6] + d[7]));
    float acc[kPer] = {};
#pragma unroll
    for (int j = 0; j < kFewParts; ++j) {
      const float wj = lane_f(wk, j);
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] = fmaf(wj, x[j][i], acc[i]);
    }
    const float f = v_scale / den;
#pragma unroll
    for (int i = 0; i < kPer; ++i) store_out<QT>(o + lane + i * kWave, acc[i] * f);
    return;
  }
  const float* po = rec_out + base * D + lane;
  if constexpr (W == 1) {
    // each wave is a unit of its own and takes its partials in groups of 64
    float big = -INFINITY;
    for (int k = lane; k < nparts; k += kWave) big = fmaxf(big, ml[at(k)].x);
    big = wave_max(big);
    float acc[kPer] = {};
    float den = 0.f;
    for (int k0 = 0; k0 < nparts; k0 += kWave) {
      const int k = k0 + lane;
      float wk = 0.f;
      if (k < nparts) {
        const float2 x = ml[at(k)];
        wk = fast_exp2(x.x - big);
        den = fmaf(wk, x.y, den);
      }
      wts[wave][lane] = wk;
      __builtin_amdgcn_wave_barrier();
      const int cnt = min(kWave, nparts - k0);
      int j = 0;
      for (; j + 4 <= cnt; j += 4) {
        float x[4][kPer];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < kPer; ++i) x[u][i] = po[at(k0 + j + u) * D + i * kWave];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < kPer; ++i) acc[i] = fmaf(wts[wave][j + u], x[u][i], acc[i]);
      }
      for (; j < cnt; ++j)
#pragma unroll
        for (int i = 0; i < kPer; ++i) acc[i] = fmaf(wts[wave][j], po[at(k0 + j) * D + i * kWave], acc[i]);
      __builtin_amdgcn_wave_barrier();
    }
    den = wave_sum(den);
    const float f = v_scale / den;
#pragma unroll
    for (int i = 0; i < kPer; ++i) store_out<QT>(o + lane + i * kWave, acc[i] * f);
  } else {
    // W waves share the unit: wave w takes partials w, w + W, w + 2W, ...,
    // kGroup at a time, loading a group's (max, sum) pairs (lane u holds the
    // group's u-th) and vectors in one round; the wave keeps its own running
    // max, and the waves' results meet in LDS with the same rescale.
    constexpr int kGroup = 32;
    const int mine = (nparts - wave + W - 1) / W;    // partials of this wave
    float mw = -INFINITY, den = 0.f;
    float acc[kPer] = {};
    for (int i0 = 0; i0 < mine; i0 += kGroup) {
      const int cnt = min(kGroup, mine - i0);
      // past cnt, lanes and vector slots re-read the group's last partial
      // with weight 0
      const int ku = wave + W * (i0 + min(lane, cnt - 1));
      const float2 x = ml[at(ku)];
      float v[kGroup][kPer];
#pragma unroll
      for (int u = 0; u < kGroup; ++u)
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          v[u][i] = po[at(wave + W * (i0 + min(u, cnt - 1))) * D + i * kWave];
      const float gm = wave_max(lane < cnt ? x.x : -INFINITY);
      const float mn = fmaxf(mw, gm);
      const float r = fast_exp2(mw - mn);        // 0 while mw is -inf
      const float wk = lane < cnt ? fast_exp2(x.x - mn) : 0.f;
      den = den * r + wave_sum(wk * x.y);
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] *= r;
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), u));
#pragma unroll
        for (int i = 0; i < kPer; ++i) acc[i] = fmaf(wu, v[u][i], acc[i]);
      }
      mw = mn;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) part[wave][lane + i * kWave] = acc[i];
    if (lane == 0) {
      part[wave][D] = den;
      part[wave][D + 1] = mw;
    }
    __syncthreads();
    if (wave != 0) return;
    float big = part[0][D + 1];
#pragma unroll
    for (int w = 1; w < W; ++w) big = fmaxf(big, part[w][D + 1]);
    float fw[W];
    float dsum = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      fw[w] = fast_exp2(part[w][D + 1] - big);   // 0 for a wave with no partials
      dsum = fmaf(fw[w], part[w][D], dsum);
    }
    const float f = v_scale / dsum;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) a = fmaf(fw[w], part[w][lane + i * kWave], a);
      store_out<QT>(o + lane + i * kWave, a * f);
    }
  }
}

// ------------------------------------------------------------------ host

// Chunks per kv head when the caller leaves the split to the library: about
// one wave per SIMD (1024 on 256 CUs).  All waves are then resident at once
// and none shares its SIMD: when two decode waves share one, the older is
// served first and the younger's chunk finishes a third later, which leaves
// the end of the kernel to half the waves.  Never chunks below
// kMinChunkBlocks of the largest possible batch.
#ifndef PKV_DECODE_TARGET_WAVES
#define PKV_DECODE_TARGET_WAVES 1024
#endif

static size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

struct DecodePlan {
  int32_t num_chunks;    // chunks per kv head (grid: num_chunks x num_kv_heads)
  int32_t fixed_chunk;   // blocks per chunk, or 0: split the batch evenly
  size_t out_bytes, ml_bytes;
};

// waves_per_simd: how many waves the library's own split aims for per SIMD
// (a bf16 block keeps one wave busy; an int4 block carries a quarter of the
// bytes for the same products, so int4 caches ask for four).
#ifndef PKV_INT4_WAVES_PER_SIMD
#define PKV_INT4_WAVES_PER_SIMD 4
#endif
constexpr int kInt4WavesPerSimd = PKV_INT4_WAVES_PER_SIMD;
// nvfp4 blocks carry about as many bytes as int4 ones, with more vector work
// per block (the block scales are applied before the products).
#ifndef PKV_NVFP4_WAVES_PER_SIMD
#define PKV_NVFP4_WAVES_PER_SIMD 4
#endif
constexpr int kNvfp4WavesPerSimd = PKV_NVFP4_WAVES_PER_SIMD;
// paged_attention_decode_workspace_size sizes for the finest split any
// cache type asks for
constexpr int kSplitWavesMax = 4;
static_assert(kNvfp4WavesPerSimd <= kSplitWavesMax && kInt4WavesPerSimd <= kSplitWavesMax,
              "workspace sized by the finest split");
static bool make_plan(int32_t s, int32_t hq, int32_t hkv, int32_t d, int32_t max_len,
                      int32_t partition_tokens, DecodePlan& p, int waves_per_simd = 1) {
  if (s < 0 || hq <= 0 || hkv <= 0 || d <= 0 || max_len < 0 || hq % hkv != 0) return false;
  const int64_t bound = int64_t(s) * ((max_len + kBlock - 1) / kBlock);
  int64_t chunks;
  if (partition_tokens > 0) {
    p.fixed_chunk = partition_tokens / kBlock;
    chunks = (bound + p.fixed_chunk - 1) / p.fixed_chunk;
  } else {
    p.fixed_chunk = 0;
    // one chunk per wave slot and kv head (the matrix-core kernel runs a
    // whole query group in one wave; the vector kernel's second wave for
    // groups above four shares its chunk's tiles through the cache)
    chunks = int64_t(PKV_DECODE_TARGET_WAVES) * waves_per_simd / int64_t(hkv);
    chunks = std::min<int64_t>(chunks, (bound + kMinChunkBlocks - 1) / kMinChunkBlocks);
  }
  chunks = std::max<int64_t>(chunks, 1);
  if (chunks * hkv > 0x7fffffff) return false;
  p.num_chunks = int32_t(chunks);
  // partial of (chunk g, sequence s) -> record g + s
  const size_t records = size_t(chunks) + size_t(s);
  p.out_bytes = align256(records * hq * d * sizeof(float));
  p.ml_bytes = align256(records * hq * 2 * sizeof(float));
  return true;
}

// Waves per SIMD the library's own split plans for: a wave serving two kv
// heads of an fp8 cache covers a chunk of both, so the split doubles the
// chunks to keep PKV_FP8_PAIR_WAVES_PER_SIMD waves on every SIMD.  One: since
// the kernel holds its results in registers, one such wave per SIMD walking
// twice the chunks measured 9% faster than two on the 70B long-context batch
// (and leaves half the records to merge).
#ifndef PKV_FP8_PAIR_WAVES_PER_SIMD
#define PKV_FP8_PAIR_WAVES_PER_SIMD 1
#endif
#ifndef PKV_BF16_WAVES_PER_SIMD
#define PKV_BF16_WAVES_PER_SIMD 1
#endif
static int split_waves_per_simd(pkv_dtype kv_dtype, int group, int num_kv_heads) {
#if PKV_DECODE_USE_MFMA
  if (decode_mfma_heads_per_wave(kv_dtype, group, num_kv_heads) == 2)
    return 2 * PKV_FP8_PAIR_WAVES_PER_SIMD;
  if (kv_dtype == PKV_BF16) return PKV_BF16_WAVES_PER_SIMD;
#endif
  return 1;
}
static_assert(2 * PKV_FP8_PAIR_WAVES_PER_SIMD <= kSplitWavesMax,
              "workspace sized by the finest split");

template <typename QT, int D>
static pkv_status launch_merge(void* out, const int32_t* lens, int32_t s, int32_t max_len,
                               int32_t hq, float v_scale, const DecodePlan& plan, void* ws,
                               hipStream_t st, int32_t window = 0,
                               int32_t chunks_per_wave = 1) {
  const float* rec_out = static_cast<const float*>(ws);
  const float* rec_ml =
      reinterpret_cast<const float*>(static_cast<const char*>(ws) + plan.out_bytes);
  if (plan.fixed_chunk > 0)
    hipLaunchKernelGGL((decode_merge_kernel<QT, D, 4>), dim3(hq, s), dim3(kWave * 4), 0, st,
                       static_cast<typename QT::storage*>(out), rec_out, rec_ml, lens, s,
                       max_len, hq, plan.num_chunks, plan.fixed_chunk, chunks_per_wave,
                       v_scale, window);
  else
    hipLaunchKernelGGL((decode_merge_kernel<QT, D, 1>),
                       dim3((hq + kMergeUnits - 1) / kMergeUnits, s), dim3(kWave * kMergeUnits), 0, st,
                       static_cast<typename QT::storage*>(out), rec_out, rec_ml, lens, s,
                       max_len, hq, plan.num_chunks, plan.fixed_chunk, chunks_per_wave,
                       v_scale, window);
  return launch_status();
}

template <typename QT, typename KVT, int D, int GW>
static pkv_status launch_decode(void* out, const void* q, const void* kc,
                                const void* vc, int32_t nb, const int32_t* bt,
                                int32_t maxb, const int32_t* lens, int32_t s,
                                int32_t max_len, int32_t hq, int32_t hkv,
                                float scale_log2, float v_scale, const DecodePlan& plan,
                                void* ws, hipStream_t st) {
  const int group = hq / hkv;
  const int waves = (group + GW - 1) / GW;
  float* rec_out = static_cast<float*>(ws);
  float* rec_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + plan.out_bytes);
  hipLaunchKernelGGL((decode_chunk_kernel<QT, KVT, D, GW>),
                     dim3(plan.num_chunks * hkv), dim3(kWave * waves), 0, st,
                     static_cast<typename QT::storage*>(out),
                     static_cast<const typename QT::storage*>(q),
                     static_cast<const typename KVT::storage*>(kc),
                     static_cast<const typename KVT::storage*>(vc), nb, bt, maxb, lens, s,
                     max_len, hq, hkv, group, scale_log2, v_scale, plan.num_chunks,
                     plan.fixed_chunk, rec_out, rec_ml);
  if (launch_status() != PKV_OK) return PKV_ERR_LAUNCH;
  return launch_merge<QT, D>(out, lens, s, max_len, hq, v_scale, plan, ws, st);
}

template <typename QT, typename KVT, int D>
static pkv_status dispatch_gw(int gw, void* out, const void* q, const void* kc,
                              const void* vc, int32_t nb, const int32_t* bt,
                              int32_t maxb, const int32_t* lens, int32_t s,
                              int32_t ml, int32_t hq, int32_t hkv, float sl2, float vs,
                              const DecodePlan& lay, void* ws, hipStream_t st) {
  switch (gw) {
    case 1: return launch_decode<QT, KVT, D, 1>(out, q, kc, vc, nb, bt, maxb, lens, s, ml, hq, hkv, sl2, vs, lay, ws, st);
    case 2: return launch_decode<QT, KVT, D, 2>(out, q, kc, vc, nb, bt, maxb, lens, s, ml, hq, hkv, sl2, vs, lay, ws, st);
    case 3: return launch_decode<QT, KVT, D, 3>(out, q, kc, vc, nb, bt, maxb, lens, s, ml, hq, hkv, sl2, vs, lay, ws, st);
    case 4: return launch_decode<QT, KVT, D, 4>(out, q, kc, vc, nb, bt, maxb, lens, s, ml, hq, hkv, sl2, vs, lay, ws, st);
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

namespace pkv {

// The matrix-core decode: the chunk kernel, then the merge of split
// sequences.  Fixed partitions are walked several to a wave, so that a short
// partition does not cost a wave start (and the wave's loads run on across
// the partitions' boundaries).  A bf16 block keeps one wave per SIMD busy; an
// fp8 or int4 block carries a half or a quarter of the bytes for the same
// products, so those caches get PKV_FP8_WAVES_PER_SIMD waves per SIMD.
#ifndef PKV_FP8_WAVES_PER_SIMD
#define PKV_FP8_WAVES_PER_SIMD 3
#endif

static pkv_status mfma_decode(void* out, const void* query, const void* k_cache,
                              const void* v_cache, const void* k_scales,
                              const void* v_scales, int32_t num_blocks,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_context_len, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, float scale_log2,
                              pkv_dtype kv_dtype, float v_scale, const DecodePlan& lay,
                              void* workspace, void* stream, int32_t window = 0,
                              const void* new_k = nullptr, const void* new_v = nullptr,
                              float k_scale = 1.0f) {
  const int nh = decode_mfma_heads_per_wave(kv_dtype, num_q_heads / num_kv_heads, num_kv_heads);
  const int64_t target = int64_t(PKV_DECODE_TARGET_WAVES) *
                         (nh == 2 ? PKV_FP8_PAIR_WAVES_PER_SIMD
                                  : kv_dtype == PKV_BF16 ? 1 : PKV_FP8_WAVES_PER_SIMD);
  const int64_t per_wave =
      lay.fixed_chunk > 0
          ? std::max<int64_t>(1, (int64_t(lay.num_chunks) * (num_kv_heads / nh) + target - 1) /
                                     target)
          : 1;
  DecodeMfmaArgs a{out, query, k_cache, v_cache, num_blocks, block_tables,
                   max_blocks_per_seq, context_lens, num_seqs, max_context_len,
                   num_q_heads, num_kv_heads, head_dim, kv_dtype, scale_log2, v_scale,
                   lay.num_chunks, lay.fixed_chunk, int32_t(per_wave),
                   static_cast<float*>(workspace),
                   reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.out_bytes),
                   stream, k_scales, v_scales, window, new_k, new_v, k_scale};
  a.heads_per_wave = nh;
  if (launch_decode_mfma(a) != PKV_OK) return PKV_ERR_LAUNCH;
  hipStream_t st = as_stream(stream);
  const int32_t stride = decode_mfma_record_stride(kv_dtype, int32_t(per_wave));
  return head_dim == 64
             ? launch_merge<BF16, 64>(out, context_lens, num_seqs, max_context_len,
                                      num_q_heads, v_scale, lay, workspace, st, window,
                                      stride)
             : launch_merge<BF16, 128>(out, context_lens, num_seqs, max_context_len,
                                       num_q_heads, v_scale, lay, workspace, st, window,
                                       stride);
}

}  // namespace pkv

extern "C" int32_t paged_attention_decode_num_chunks(int32_t num_seqs,
                                                     int32_t num_q_heads,
                                                     int32_t num_kv_heads,
                                                     int32_t max_context_len,
                                                     int32_t partition_tokens) {
  DecodePlan p;
  if (partition_tokens < 0 || partition_tokens % kBlock != 0 ||
      !make_plan(num_seqs, num_q_heads, num_kv_heads, 1, max_context_len, partition_tokens, p))
    return -1;
  return p.num_chunks;
}

extern "C" size_t paged_attention_decode_workspace_size(int32_t num_seqs,
                                                        int32_t num_q_heads,
                                                        int32_t num_kv_heads,
                                                        int32_t head_dim,
                                                        int32_t max_context_len,
                                                        int32_t partition_tokens) {
  // large enough for every cache dtype's plan
  DecodePlan p;
  if (partition_tokens < 0 || partition_tokens % kBlock != 0 ||
      !make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                 partition_tokens, p, kSplitWavesMax))
    return 0;
  return p.out_bytes + p.ml_bytes;
}

static pkv_status decode_impl(
    void* out, const void* query, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    float softmax_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype, float k_scale,
    float v_scale, int32_t partition_tokens, void* workspace,
    size_t workspace_bytes, void* stream, int32_t window, const void* new_key = nullptr,
    const void* new_value = nullptr) {
  if (window < 0) return PKV_ERR_SHAPE;
  if (num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq < 0 ||
      max_context_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0)
    return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (int64_t(max_blocks_per_seq) * kBlock < max_context_len) return PKV_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  if (group > 8) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (partition_tokens < 0 || partition_tokens % kBlock != 0) return PKV_ERR_SHAPE;
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
  DecodePlan lay;
  if (!make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                 partition_tokens, lay, split_waves_per_simd(kv_dtype, group, num_kv_heads)) ||
      int64_t(num_seqs) * num_q_heads > 0x7fffffff)
    return PKV_ERR_SHAPE;
  if (!workspace || workspace_bytes < lay.out_bytes + lay.ml_bytes)
    return PKV_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return PKV_ERR_ALIGN;

  const bool append = new_key != nullptr;
  if (append && !(aligned(new_key, 16) && aligned(new_value, 16))) return PKV_ERR_ALIGN;
#if PKV_DECODE_USE_MFMA
  if (decode_mfma_supported(q_dtype, kv_dtype, head_dim, group))
    return mfma_decode(out, query, k_cache, v_cache, nullptr, nullptr, num_blocks, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len,
                       num_q_heads, num_kv_heads, head_dim, softmax_scale * k_scale * kLog2e,
                       kv_dtype, v_scale, lay, workspace, stream, window, new_key, new_value,
                       k_scale);
#endif
  // the append is built into the matrix-core kernel only
  if (append) return PKV_ERR_UNSUPPORTED;
  // the sliding window is built into the matrix-core kernel only
  if (window > 0) return PKV_ERR_UNSUPPORTED;
  // fp32 q with head_dim 128 keeps at most two heads per wave (registers)
  const int max_gw = (f32 && head_dim == 128) ? 2 : PKV_DECODE_MAX_HEADS_PER_WAVE;
  const int waves = (group + max_gw - 1) / max_gw;
  const int gw = (group + waves - 1) / waves;
  const float scale_log2 = softmax_scale * k_scale * kLog2e;
  hipStream_t st = as_stream(stream);
  const int32_t nb = num_blocks, maxb = max_blocks_per_seq;
#define PKV_DECODE_ARGS gw, out, query, k_cache, v_cache, nb, block_tables, maxb, \
    context_lens, num_seqs, max_context_len, num_q_heads, num_kv_heads, scale_log2, v_scale, lay, workspace, st
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

extern "C" pkv_status paged_attention_decode(
    void* out, const void* query, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    float softmax_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype, float k_scale,
    float v_scale, int32_t partition_tokens, void* workspace,
    size_t workspace_bytes, void* stream) {
  return decode_impl(out, query, k_cache, v_cache, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_q_heads,
                     num_kv_heads, head_dim, softmax_scale, q_dtype, kv_dtype, k_scale, v_scale,
                     partition_tokens, workspace, workspace_bytes, stream, 0);
}

extern "C" pkv_status paged_attention_decode_sliding(
    void* out, const void* query, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    float softmax_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype, float k_scale,
    float v_scale, int32_t sliding_window, int32_t partition_tokens, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (sliding_window <= 0) return PKV_ERR_SHAPE;
  return decode_impl(out, query, k_cache, v_cache, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_q_heads,
                     num_kv_heads, head_dim, softmax_scale, q_dtype, kv_dtype, k_scale, v_scale,
                     partition_tokens, workspace, workspace_bytes, stream, sliding_window);
}

extern "C" pkv_status paged_attention_decode_int4(
    void* out, const void* query, const void* k_cache, const void* v_cache,
    const float* k_scales, const float* v_scales, int32_t num_blocks,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float softmax_scale, pkv_dtype q_dtype, int32_t partition_tokens,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_context_len < 0 ||
      num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (int64_t(max_blocks_per_seq) * kBlock < max_context_len) return PKV_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  if (group > 8 || head_dim != 128 || q_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (partition_tokens < 0 || partition_tokens % kBlock != 0) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (num_blocks == 0) return PKV_ERR_SHAPE;
  if (!out || !query || !k_cache || !v_cache || !k_scales || !v_scales || !block_tables ||
      !context_lens)
    return PKV_ERR_NULL;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(k_scales, 16) || !aligned(v_scales, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PKV_ERR_ALIGN;
  DecodePlan lay;
  if (!make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                 partition_tokens, lay, kInt4WavesPerSimd) ||
      int64_t(num_seqs) * num_q_heads > 0x7fffffff)
    return PKV_ERR_SHAPE;
  if (!workspace || workspace_bytes < lay.out_bytes + lay.ml_bytes) return PKV_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return PKV_ERR_ALIGN;
  return mfma_decode(out, query, k_cache, v_cache, k_scales, v_scales, num_blocks,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, max_context_len,
                     num_q_heads, num_kv_heads, head_dim, softmax_scale * kLog2e, PKV_INT4,
                     1.0f, lay, workspace, stream);
}

extern "C" pkv_status paged_attention_decode_nvfp4(
    void* out, const void* query, const void* k_cache, const void* v_cache,
    const void* k_bscales, const void* v_bscales, int32_t num_blocks,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float softmax_scale, pkv_dtype q_dtype, float k_scale, float v_scale,
    int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_context_len < 0 ||
      num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (int64_t(max_blocks_per_seq) * kBlock < max_context_len) return PKV_ERR_SHAPE;
  if (!(k_scale > 0.f && v_scale > 0.f)) return PKV_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  if (group > 8 || head_dim != 128 || q_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (partition_tokens < 0 || partition_tokens % kBlock != 0) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (num_blocks == 0) return PKV_ERR_SHAPE;
  if (!out || !query || !k_cache || !v_cache || !k_bscales || !v_bscales || !block_tables ||
      !context_lens)
    return PKV_ERR_NULL;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(k_bscales, 16) || !aligned(v_bscales, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PKV_ERR_ALIGN;
  DecodePlan lay;
  if (!make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                 partition_tokens, lay, kNvfp4WavesPerSimd) ||
      int64_t(num_seqs) * num_q_heads > 0x7fffffff)
    return PKV_ERR_SHAPE;
  if (!workspace || workspace_bytes < lay.out_bytes + lay.ml_bytes) return PKV_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return PKV_ERR_ALIGN;
  return mfma_decode(out, query, k_cache, v_cache, k_bscales, v_bscales, num_blocks,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, max_context_len,
                     num_q_heads, num_kv_heads, head_dim, softmax_scale * k_scale * kLog2e,
                     PKV_NVFP4, v_scale, lay, workspace, stream);
}

extern "C" pkv_status paged_attention_decode_append(
    void* out, const void* query, const void* new_key, const void* new_value, void* k_cache,
    void* v_cache, int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
    pkv_dtype q_dtype, pkv_dtype kv_dtype, float k_scale, float v_scale,
    int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!new_key || !new_value)) return PKV_ERR_NULL;
  if (q_dtype != PKV_BF16 || (kv_dtype != PKV_BF16 && kv_dtype != PKV_FP8_E4M3))
    return PKV_ERR_UNSUPPORTED;
  return decode_impl(out, query, k_cache, v_cache, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_q_heads,
                     num_kv_heads, head_dim, softmax_scale, q_dtype, kv_dtype, k_scale, v_scale,
                     partition_tokens, workspace, workspace_bytes, stream, 0, new_key,
                     new_value);
}

// ---- allocation-free decode ------------------------------------------------
// paged_attention_decode with its partials in a file-scope device array
// instead of a caller workspace, for callers that cannot allocate.  Each GPU
// the library runs on holds its own copy of the array (kDecodeScratchBytes)
// until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns on that device, looked up once per device on
// the first call there.  The decode kernels write every record they later
// read, so nothing in the array needs clearing between calls.
#include <mutex>

namespace {
constexpr size_t kDecodeScratchBytes = size_t(PKV_DECODE_SCRATCH_BYTES);
constexpr int kScratchDevices = 64;
__device__ __align__(256) char scratch[kDecodeScratchBytes];
std::mutex scratch_mutex;
void* scratch_ptr[kScratchDevices];   // per device; null until looked up

pkv_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_LAUNCH;
  if (dev < 0 || dev >= kScratchDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PKV_ERR_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return PKV_OK;
}
}  // namespace

extern "C" pkv_status paged_attention_decode_noalloc(
    void* out, const void* query, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    float softmax_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype, float k_scale,
    float v_scale, int32_t partition_tokens, void* stream) {
  // the size check comes first and touches no device state
  DecodePlan lay;
  if (partition_tokens < 0 || partition_tokens % kBlock != 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 ||
      !make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                 partition_tokens, lay,
                 split_waves_per_simd(kv_dtype, num_q_heads / num_kv_heads, num_kv_heads)))
    return PKV_ERR_SHAPE;
  if (lay.out_bytes + lay.ml_bytes > kDecodeScratchBytes) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  if (num_seqs > 0) {   // an empty batch launches nothing and needs no scratch
    const pkv_status st = device_scratch(&ws);
    if (st != PKV_OK) return st;
  }
  return decode_impl(out, query, k_cache, v_cache, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_q_heads,
                     num_kv_heads, head_dim, softmax_scale, q_dtype, kv_dtype, k_scale, v_scale,
                     partition_tokens, ws, kDecodeScratchBytes, stream, 0);
}
