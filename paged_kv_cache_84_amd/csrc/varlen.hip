// Unified varlen attention: every request of an engine step -- decodes (one
// query token), speculative verification (1 + k tokens) and prompt chunks --
// in one kernel launch (bf16 queries and cache, head_dim 128).
//
// The unified scheduler keeps no prefill or decode phase: each request only
// has a number of computed tokens and a number to reach (input + generated +
// speculative drafts), and a step advances every request by some tokens
// ("01. vLLM：从分页 KV 起家的通用推理引擎", section "调度器：统一的 token 预算";
// V1 EngineCore architecture page, section "统一 token 调度").  Drafts are
// verified by the target model in one step (the "01. vLLM" page, section
// "投机解码"): the 1 + k verified rows attend causally, like a short chunk.
// The rows of one step still differ in cost: a chunk of many rows is a dense
// contraction, a request of a few rows streams its whole history.
//
// So the launch holds two kinds of work, run side by side -- the matrix
// cores on the chunks while the memory system streams the short requests'
// histories:
//   wide   requests with more than 16 query rows (tokens x group): the
//          chunked-prefill tile of prefill_tile.h, one workgroup per (eight
//          16-row units of the wide requests' rows, kv head);
//   narrow requests with at most 16 rows: one wave per (request, kv head,
//          run of kNarrowChunk blocks) holds the request's rows as the 16
//          columns of MFMA tiles and streams the run's blocks (as the decode
//          kernel does), with the causal limit of each row.  A request with
//          several runs leaves one partial per run in the workspace, and a
//          small merge kernel combines them with the log-sum-exp rule.
// How workgroups find their work (a plan kernel, per-XCD queues, persistent
// workgroups paired per compute unit) is described above varlen_kernel.

#include <math.h>

#include <algorithm>

#include "abi_util.h"
#include "common.h"
#include "prefill_tile.h"

namespace pkv {
namespace vl {

using pf::f32x4_t;
using pf::i16x4_t;
using pf::lds_char_t;
using pf::lds_i16x4_t;

constexpr int kD = 128;
constexpr int kNarrowRows = 16;          // query rows of a narrow request at most
constexpr int kNarrowChunk = 64;         // blocks per narrow run
constexpr int kDepth = 3;                // blocks in flight per narrow wave
constexpr int kVStride = kD * 2 + 32;    // LDS bytes per staged V row
constexpr int kKSteps = kD / 32;
constexpr int kMTiles = kD / 16;
constexpr int kTileBytes = kBlock * kD * 2;
constexpr float kRaise = 8.0f;
constexpr float kNoMax = -1e30f;

PKV_DEVICE f32x4_t mfma_k32(u32x4 a, u32x4 b, f32x4_t c) {
  return pf::mfma(a, b, c);
}
PKV_DEVICE f32x4_t mfma_k16(i16x4_t a, i16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Workspace: per (request, kv head, run) a partial: 16 columns x D weighted
// values, and 16 (max, sum) pairs.
struct Workspace {
  float* part_o;
  float2* part_ml;
};

__host__ __device__ inline int runs_of(int nblk) { return (nblk + kNarrowChunk - 1) / kNarrowChunk; }

// One wave: request r, kv head kvh, run `run` of its blocks.
PKV_DEVICE void narrow_unit(char* vl, int r, int kvh, int run, int runs_per_req,
                            uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
                            const uint16_t* __restrict__ k_cache,
                            const uint16_t* __restrict__ v_cache, int32_t num_blocks,
                            const int32_t* __restrict__ block_tables, int32_t max_blocks,
                            const int32_t* __restrict__ query_start_loc,
                            const int32_t* __restrict__ num_computed, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t group, float scale_log2,
                            const Workspace& ws) {
  const int lane = lane_id();
  const int n16 = lane % 16;          // column = query row (token, head) of this lane
  const int j = lane / 16;            // lane group: keys 4j..4j+3 of a block
  const int q0 = load_scalar(query_start_loc, r);
  const int n = load_scalar(query_start_loc, r + 1) - q0;
  const int c = load_scalar(num_computed, r);
  if (n <= 0 || n * group > kNarrowRows || c < 0) return;
  const int len = c + n;                           // keys of the last row
  const int nblk = min((len + kBlock - 1) / kBlock, max_blocks);
  const int runs = min(runs_of(nblk), runs_per_req);   // the minimum only bites if
  if (run >= runs) return;                             // len exceeds max_seq_len
  const int b_lo = run * kNarrowChunk, b_hi = min(nblk, b_lo + kNarrowChunk);
  const bool col_ok = n16 < n * group;
  const int t = col_ok ? n16 / group : 0;          // token of the column
  const int head = kvh * group + (col_ok ? n16 % group : 0);
  const int qpos = c + t;                          // the row sees keys 0 .. qpos

  const int64_t head_stride = int64_t(kBlock) * kD;
  const int64_t block_stride = int64_t(num_kv_heads) * head_stride;
  auto tile = [&](const uint16_t* base, int32_t b) {
    return base + int64_t(b) * block_stride + int64_t(kvh) * head_stride;
  };
  auto valid = [&](int32_t b) { return b >= 0 && b < num_blocks; };
  const int32_t* table = block_tables + int64_t(r) * max_blocks;

  // Q^T as B operands (zero columns past the rows): one buffer resource over
  // the request's rows of this kv head's group, lanes past the rows read
  // beyond its range and get zeros
  u32x4 qb[kKSteps];
  {
    const uint32_t range = uint32_t(((n - 1) * num_q_heads + group) * kD * 2);
    const auto rq = tile_resource(query + (int64_t(q0) * num_q_heads + kvh * group) * kD, range);
    const uint32_t off = col_ok ? uint32_t(((t * num_q_heads + n16 % group) * kD + 8 * j) * 2)
                                : range;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qb[ks] = buffer_load16_cached(rq, off + uint32_t(32 * ks * 2));
  }
  // A block id outside the pool (or a block past the run) gets an empty
  // buffer range: its loads return zeros without touching memory.
  auto load_k = [&](u32x4 (&kr)[kKSteps], int32_t b) {
    const auto rs = tile_resource(tile(k_cache, valid(b) ? b : 0), valid(b) ? kTileBytes : 0);
    const uint32_t off = uint32_t((lane % 16) * kD * 2 + (lane / 16) * 16);
#pragma unroll
    for (int i = 0; i < kKSteps; ++i) kr[i] = buffer_load16(rs, off, i * 64);
  };
  constexpr int kVLoads = kTileBytes / (kWave * 16);
  auto load_v = [&](u32x4 (&vr)[kVLoads], int32_t b) {
    const auto rs = tile_resource(tile(v_cache, valid(b) ? b : 0), valid(b) ? kTileBytes : 0);
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) vr[i] = buffer_load16(rs, uint32_t(lane * 16), i * 1024);
  };
  // V rows at or past `rows` become zeros (unused slots may hold anything)
  auto stage_v = [&](const u32x4 (&vr)[kVLoads], int rows) {
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      const int o = lane * 16 + i * 1024;
      const int row = o / (kD * 2);
      const u32x4 x = row < rows ? vr[i] : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(vl + row * kVStride + (o % (kD * 2))) = x;
    }
  };
  lds_i16x4_t* const vt_base = reinterpret_cast<lds_i16x4_t*>(
      (lds_char_t*)vl + (lane / 4) * kVStride + (lane % 4) * 8);
  // The run's block ids, one per lane (a run has at most 64 blocks): the
  // loop then reads them across lanes, with no memory wait per block.
  static_assert(kNarrowChunk == kWave, "one block id per lane");
  const int32_t lane_blk = b_lo + lane < b_hi ? table[b_lo + lane] : -1;
  auto id_at = [&](int blk) {
    return blk < b_hi ? __builtin_amdgcn_readlane(lane_blk, blk - b_lo) : -1;
  };

  // A ring of kDepth blocks in flight: block i lives in slot i % kDepth,
  // and its slot is refilled with block i + kDepth as soon as it is read.
  u32x4 kr[kDepth][kKSteps], vr[kDepth][kVLoads];
  int32_t ids[kDepth];
#pragma unroll
  for (int q = 0; q < kDepth; ++q) {
    ids[q] = id_at(b_lo + q);
    load_v(vr[q], ids[q]);
    load_k(kr[q], ids[q]);
  }

  f32x4_t acc[kMTiles];
#pragma unroll
  for (int mt = 0; mt < kMTiles; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNoMax, l = 0.f;
  for (int i0 = b_lo; i0 < b_hi; i0 += kDepth) {
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
      const int i = i0 + q;
      const int rows = (i < b_hi && valid(ids[q])) ? min(kBlock, len - i * kBlock) : 0;
      stage_v(vr[q], rows);
      const int32_t id_new = id_at(i + kDepth);
      __builtin_amdgcn_sched_barrier(0);
      load_v(vr[q], id_new);
      __builtin_amdgcn_sched_barrier(0);
      f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) st = mfma_k32(kr[q][ks], qb[ks], st);
      load_k(kr[q], id_new);
      ids[q] = id_new;
      // causal limit of the column's row (keys past the context are past it)
      float sv[4];
      bool raise = false;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = i * kBlock + 4 * j + rr;
        const float x = st[rr] * scale_log2;
        sv[rr] = (4 * j + rr < rows && key <= qpos) ? x : -INFINITY;
        raise |= sv[rr] > m + kRaise;
      }
      if (__builtin_expect(__ballot(raise) != 0, 0)) {
        float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        bm = fmaxf(bm, shfl_xor(bm, 16));
        bm = fmaxf(bm, shfl_xor(bm, 32));
        const float mn = fmaxf(m, bm);
        const float alpha = fast_exp2(m - mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int mt = 0; mt < kMTiles; ++mt) acc[mt] *= alpha;
      }
      float p[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) p[rr] = fast_exp2(sv[rr] - m);
      l += (p[0] + p[1]) + (p[2] + p[3]);
      // P^T = hi + lo, both bf16, so the product keeps fp32-level accuracy
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t a = __float_as_uint(p[2 * w]), b = __float_as_uint(p[2 * w + 1]);
        hi[w] = (b & 0xffff0000u) | (a >> 16);
        lo[w] = pf::pack_bf16(p[2 * w] - __uint_as_float(a & 0xffff0000u),
                              p[2 * w + 1] - __uint_as_float(b & 0xffff0000u));
      }
      const i16x4_t phi = __builtin_bit_cast(i16x4_t, uint2{hi[0], hi[1]});
      const i16x4_t plo = __builtin_bit_cast(i16x4_t, uint2{lo[0], lo[1]});
#pragma unroll
      for (int mt = 0; mt < kMTiles; ++mt) {
        const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vt_base + mt * 4);
        acc[mt] = mfma_k16(a, phi, acc[mt]);
        acc[mt] = mfma_k16(a, plo, acc[mt]);
      }
    }
  }
  // sum of weights of each column over the four lane groups
  float lt = l + shfl_xor(l, 16);
  lt += shfl_xor(lt, 32);
  uint16_t* o = out + (int64_t(q0 + t) * num_q_heads + head) * kD + 4 * j;
  auto store = [&](const f32x4_t (&a)[kMTiles], float f) {
#pragma unroll
    for (int mt = 0; mt < kMTiles; ++mt) {
      const uint2 w = {uint32_t(f32_to_bf16(a[mt][0] * f)) | (uint32_t(f32_to_bf16(a[mt][1] * f)) << 16),
                       uint32_t(f32_to_bf16(a[mt][2] * f)) | (uint32_t(f32_to_bf16(a[mt][3] * f)) << 16)};
      *reinterpret_cast<uint2*>(o + mt * 16) = w;
    }
  };
  if (runs == 1) {
    if (col_ok) store(acc, 1.0f / lt);
    return;
  }
  // several runs: leave the partial; the merge kernel combines them
  const int64_t unit = int64_t(r) * num_kv_heads + kvh;
  const int64_t rec = unit * runs_per_req + run;
  if (!col_ok) return;
  float* po = ws.part_o + (rec * kNarrowRows + n16) * kD + 4 * j;
#pragma unroll
  for (int mt = 0; mt < kMTiles; ++mt)
    *reinterpret_cast<float4*>(po + mt * 16) = make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
  if (j == 0) ws.part_ml[rec * kNarrowRows + n16] = make_float2(m, lt);
}

}  // namespace vl

// Work queues.  Workgroup b runs on XCD b % 8, and the hardware spreads the
// workgroups of an XCD over its compute units in a fixed rotation, so a
// static pattern of kinds in the grid (wide, narrow, wide, ...) would pin each
// kind to a fixed subset of the compute units.  Instead each XCD has two
// ticket counters, one per kind, and the kernel is persistent: about two
// workgroups per compute unit, each drawing the next ticket of a queue of
// its XCD, running the piece of work that ticket names, and drawing again
// until both queues are empty.  The wide queue of XCD x holds the wide
// workgroup indices equal to x mod 8 (tiles numbered kv head fastest, so
// with a multiple of eight kv heads an XCD keeps the tiles of the same kv
// heads and its L2 their shared prefix); the narrow queue likewise.  The
// counters sit 256 bytes apart, so that their atomics do not queue on one
// memory channel.
//
// A one-workgroup plan kernel runs first: it clears the counters and lists
// every wide tile as (request, tile of the request) and every narrow item as
// (request, run), so that a workgroup finds its piece with one load.
constexpr int kQueues = 8;
constexpr int kPlanThreads = 256;
constexpr int kTicketStride = 64;                        // int32 apart: 256 bytes
constexpr int kWideCount = 2 * kQueues * kTicketStride;  // where the plan's totals sit
constexpr int kNarrowCount = kWideCount + 1;
constexpr int kCuSlots = kQueues * 8 * 2 * 16;           // XCD x engine x array x unit
constexpr int kHwIdReg = 4 | (31 << 11);                 // HW_ID, bits 0..31

struct Plan {
  int32_t* tickets;        // counters: wide queue x at x * kTicketStride, narrow queue x
                           // at (8 + x) * kTicketStride; then the totals
  int32_t* cu_slots;       // workgroups arrived per compute unit
  int2* wide_map;          // unit -> (request, 16-row unit of the request)
  int2* narrow_map;        // item -> (request, run)
  int32_t wide_cap, narrow_cap;
};

__global__ __launch_bounds__(kPlanThreads) void varlen_plan_kernel(
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ num_computed,
    int32_t num_reqs, int32_t group, int32_t max_blocks, int32_t runs_per_req, Plan plan) {
  __shared__ int sw[kPlanThreads], sn[kPlanThreads];
  __shared__ int carry[2];
  const int tid = threadIdx.x;
  if (tid < 2 * kQueues) plan.tickets[tid * kTicketStride] = 0;
  for (int i = tid; i < kCuSlots; i += kPlanThreads) plan.cu_slots[i] = 0;
  if (tid < 2) carry[tid] = 0;
  __syncthreads();
  for (int base = 0; base < num_reqs; base += kPlanThreads) {
    const int r = base + tid;
    int wt = 0, ni = 0;
    if (r < num_reqs) {
      const int n = query_start_loc[r + 1] - query_start_loc[r];
      const int c = num_computed[r];
      if (n > 0 && n * group > vl::kNarrowRows)
        wt = (n * group + pf::kUnitRows - 1) / pf::kUnitRows;
      else if (n > 0 && c >= 0)
        ni = min(vl::runs_of(min((c + n + kBlock - 1) / kBlock, max_blocks)), runs_per_req);
    }
    sw[tid] = wt;
    sn[tid] = ni;
    __syncthreads();
    for (int o = 1; o < kPlanThreads; o <<= 1) {     // inclusive scans of both counts
      const int aw = tid >= o ? sw[tid - o] : 0, an = tid >= o ? sn[tid - o] : 0;
      __syncthreads();
      sw[tid] += aw;
      sn[tid] += an;
      __syncthreads();
    }
    const int n0 = carry[1] + sn[tid] - ni;
    // wide units: the threads share the entries (a long chunk has hundreds),
    // each finding the request of its entry by a binary search of the scan
    for (int g = tid; g < sw[kPlanThreads - 1]; g += kPlanThreads) {
      int lo = 0, hi = kPlanThreads - 1;       // first i with sw[i] > g
      while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (sw[mid] > g) hi = mid;
        else lo = mid + 1;
      }
      const int u = carry[0] + g;
      if (u < plan.wide_cap) plan.wide_map[u] = make_int2(base + lo, g - (lo > 0 ? sw[lo - 1] : 0));
    }
    for (int k = 0; k < ni && n0 + k < plan.narrow_cap; ++k)
      plan.narrow_map[n0 + k] = make_int2(r, k);
    __syncthreads();
    if (tid == 0) {
      carry[0] += sw[kPlanThreads - 1];
      carry[1] += sn[kPlanThreads - 1];
    }
    __syncthreads();
  }
  if (tid == 0) {
    plan.tickets[kWideCount] = min(carry[0], plan.wide_cap);
    plan.tickets[kNarrowCount] = min(carry[1], plan.narrow_cap);
  }
}

__global__ __launch_bounds__(256, 2) void varlen_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    int32_t num_blocks, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ num_computed,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t group, float scale_log2,
    int32_t wide_wgs, int32_t narrow_wgs, int32_t runs_per_req, Plan plan,
    float* __restrict__ part_o, float2* __restrict__ part_ml) {
  __shared__ pf::Stage stage0, stage1;
  // tickets are passed through the stages' first word (a separate LDS
  // variable would take the workgroup past 64 KiB of LDS)
  int* const ticket_lds = reinterpret_cast<int*>(&stage0);
  const int x = blockIdx.x % kQueues;
  const int wide_x = (wide_wgs + kQueues - 1 - x) / kQueues;     // queue x's share of each kind
  const int narrow_x = (narrow_wgs + kQueues - 1 - x) / kQueues;
  const int wide_units = load_scalar(plan.tickets, kWideCount);
  const int wide_pieces = (wide_units + pf::kUnits - 1) / pf::kUnits;
  const int narrow_items = load_scalar(plan.tickets, kNarrowCount);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
  // The first workgroup to arrive on a compute unit prefers wide work, the
  // second narrow work, so that each compute unit runs one of each while
  // both queues last: the matrix-core-bound tiles and the memory-bound
  // streams then share every SIMD.  A compute unit is named by its XCD and
  // its place in it (shader engine, array, unit fields of the wave's
  // hardware id).
  if (threadIdx.x == 0) {
    const uint32_t hw = __builtin_amdgcn_s_getreg(kHwIdReg);
    const int key = ((x * 8 + int((hw >> 13) & 7)) * 2 + int((hw >> 12) & 1)) * 16 +
                    int((hw >> 8) & 15);
    *ticket_lds = __hip_atomic_fetch_add(plan.cu_slots + key, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const bool prefer_wide = (*ticket_lds & 1) == 0;
  __syncthreads();
  bool wide_open = true, narrow_open = true;
  while (wide_open || narrow_open) {
    // the preferred queue while it lasts, then the other one
    const bool wide = wide_open && (prefer_wide || !narrow_open);
    if (threadIdx.x == 0)
      *ticket_lds = __hip_atomic_fetch_add(
          plan.tickets + (wide ? x : kQueues + x) * kTicketStride, 1, __ATOMIC_RELAXED,
          __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int k = *ticket_lds;
    __syncthreads();     // every thread holds the ticket before the stages fill
    const int idx = k * kQueues + x;
    // indices only grow along a queue: the first one past the work closes it
    if (wide && (k >= wide_x || idx / num_kv_heads >= wide_pieces)) {
      wide_open = false;
      continue;
    }
    if (!wide && (k >= narrow_x || int64_t(idx) * 4 / num_kv_heads >= narrow_items)) {
      narrow_open = false;
      continue;
    }
    if (wide) {
      // units 8 piece .. +7, lane i < 8 reading unit i's entry
      const int lane = int(threadIdx.x) & (kWave - 1);
      const int u = (idx / num_kv_heads) * pf::kUnits + (lane & (pf::kUnits - 1));
      int2 unit = make_int2(-1, 0);
      if (lane < pf::kUnits && u < wide_units) unit = plan.wide_map[u];
      prefill_units(stage0, stage1, unit.x, unit.y, idx % num_kv_heads, out, query, k_cache,
                    v_cache, num_blocks, block_tables, max_blocks, query_start_loc,
                    num_computed, num_q_heads, num_kv_heads, group, scale_log2);
    } else {
      // narrow: wave w of workgroup idx takes unit idx * 4 + w; a unit is
      // (item, kv head) with the kv head fastest, so the waves of a workgroup
      // usually share an item and take equally long
      const int64_t u = int64_t(idx) * 4 + wave;
      const int kvh = int(u % num_kv_heads);
      const int64_t item = u / num_kv_heads;
      if (item < narrow_items) {
        const int2 piece = plan.narrow_map[item];
        const int r = __builtin_amdgcn_readfirstlane(piece.x);
        const int run = __builtin_amdgcn_readfirstlane(piece.y);
        char* lds = reinterpret_cast<char*>(&stage1) + wave * (kBlock * vl::kVStride);
        vl::narrow_unit(lds, r, kvh, run, runs_per_req, out, query, k_cache, v_cache,
                        num_blocks, block_tables, max_blocks, query_start_loc, num_computed,
                        num_q_heads, num_kv_heads, group, scale_log2,
                        vl::Workspace{part_o, part_ml});
      }
    }
    __syncthreads();     // the stages are free before the next ticket
  }
}

// Merge of the narrow requests that span several runs: one workgroup per
// (request, kv head); thread t combines column t / 16 (a query row), eight of
// its D values, over the runs with the log-sum-exp rule.
__global__ __launch_bounds__(256) void varlen_merge_kernel(
    uint16_t* __restrict__ out, const int32_t* __restrict__ query_start_loc,
    const int32_t* __restrict__ num_computed, int32_t max_blocks, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t group, int32_t runs_per_req,
    const float* __restrict__ part_o, const float2* __restrict__ part_ml) {
  const int r = blockIdx.x / num_kv_heads, kvh = blockIdx.x % num_kv_heads;
  const int q0 = load_scalar(query_start_loc, r);
  const int n = load_scalar(query_start_loc, r + 1) - q0;
  const int c = load_scalar(num_computed, r);
  if (n <= 0 || n * group > vl::kNarrowRows || c < 0) return;
  const int nblk = min((c + n + kBlock - 1) / kBlock, max_blocks);
  const int runs = min(vl::runs_of(nblk), runs_per_req);
  if (runs <= 1) return;
  const int col = threadIdx.x / 16, d0 = (threadIdx.x % 16) * 8;
  if (col >= n * group) return;
  const int64_t rec0 = (int64_t(r) * num_kv_heads + kvh) * runs_per_req;
  float mx = vl::kNoMax;
  for (int k = 0; k < runs; ++k) mx = fmaxf(mx, part_ml[(rec0 + k) * vl::kNarrowRows + col].x);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int k = 0; k < runs; ++k) {
    const int64_t rc = (rec0 + k) * vl::kNarrowRows + col;
    const float2 ml = part_ml[rc];
    const float w = fast_exp2(ml.x - mx);
    den += w * ml.y;
    const float4* po = reinterpret_cast<const float4*>(part_o + rc * vl::kD + d0);
    const float4 a = po[0], b = po[1];
    acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
    acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
  }
  const float f = 1.0f / den;
  const int t = col / group, head = kvh * group + col % group;
  uint16_t* o = out + (int64_t(q0 + t) * num_q_heads + head) * vl::kD + d0;
  uint4 w;
  w.x = uint32_t(f32_to_bf16(acc[0] * f)) | (uint32_t(f32_to_bf16(acc[1] * f)) << 16);
  w.y = uint32_t(f32_to_bf16(acc[2] * f)) | (uint32_t(f32_to_bf16(acc[3] * f)) << 16);
  w.z = uint32_t(f32_to_bf16(acc[4] * f)) | (uint32_t(f32_to_bf16(acc[5] * f)) << 16);
  w.w = uint32_t(f32_to_bf16(acc[6] * f)) | (uint32_t(f32_to_bf16(acc[7] * f)) << 16);
  *reinterpret_cast<uint4*>(o) = w;
}

static size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

struct VarlenPlan {
  int32_t runs_per_req;
  int64_t wide_cap, narrow_cap;     // wide tiles (for groups up to 8), narrow items
  size_t ticket_bytes, wide_bytes, narrow_bytes, o_bytes, ml_bytes;
  size_t total() const { return ticket_bytes + wide_bytes + narrow_bytes + o_bytes + ml_bytes; }
};

static bool varlen_plan(int32_t num_reqs, int32_t num_q_tokens, int32_t num_kv_heads,
                        int32_t head_dim, int32_t max_seq_len, VarlenPlan& p) {
  if (num_reqs < 0 || num_q_tokens < 0 || num_kv_heads <= 0 || head_dim != vl::kD ||
      max_seq_len < 0)
    return false;
  const int nblk = (max_seq_len + kBlock - 1) / kBlock;
  p.runs_per_req = std::max(1, vl::runs_of(nblk));
  // 16-row units: at most n group / 16 + 1 for a request of n tokens, and
  // the group is at most 8
  p.wide_cap = (int64_t(num_q_tokens) + 1) / 2 + num_reqs;
  p.narrow_cap = int64_t(num_reqs) * p.runs_per_req;
  const size_t recs = size_t(p.narrow_cap) * num_kv_heads;
  p.ticket_bytes = align256((kNarrowCount + 1) * sizeof(int32_t)) + kCuSlots * sizeof(int32_t);
  p.wide_bytes = align256(size_t(p.wide_cap) * sizeof(int2));
  p.narrow_bytes = align256(size_t(p.narrow_cap) * sizeof(int2));
  p.o_bytes = align256(recs * vl::kNarrowRows * head_dim * sizeof(float));
  p.ml_bytes = align256(recs * vl::kNarrowRows * 2 * sizeof(float));
  return true;
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t paged_attention_varlen_workspace_size(int32_t num_reqs, int32_t num_q_tokens,
                                                        int32_t num_kv_heads, int32_t head_dim,
                                                        int32_t max_seq_len) {
  VarlenPlan p;
  if (!varlen_plan(num_reqs, num_q_tokens, num_kv_heads, head_dim, max_seq_len, p)) return 0;
  return p.total();
}

extern "C" pkv_status paged_attention_varlen(
    void* out, const void* query, const void* k_cache, const void* v_cache,
    int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* query_start_loc, const int32_t* num_computed_tokens, int32_t num_reqs,
    int32_t num_q_tokens, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float softmax_scale, pkv_dtype q_dtype, pkv_dtype kv_dtype,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (num_reqs < 0 || num_q_tokens < 0 || num_blocks < 0 || max_blocks_per_seq < 0 ||
      max_seq_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  if (!(group == 1 || group == 2 || group == 4 || group == 8)) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 128 || q_dtype != PKV_BF16 || kv_dtype != PKV_BF16)
    return PKV_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.f)) return PKV_ERR_UNSUPPORTED;
  if (int64_t(max_blocks_per_seq) * kBlock < max_seq_len) return PKV_ERR_SHAPE;
  if (num_reqs == 0 || num_q_tokens == 0) return PKV_OK;
  if (num_blocks == 0) return PKV_ERR_SHAPE;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !query_start_loc ||
      !num_computed_tokens)
    return PKV_ERR_NULL;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_tables, 4) || !aligned(query_start_loc, 4) ||
      !aligned(num_computed_tokens, 4))
    return PKV_ERR_ALIGN;
  VarlenPlan p;
  if (!varlen_plan(num_reqs, num_q_tokens, num_kv_heads, head_dim, max_seq_len, p))
    return PKV_ERR_SHAPE;
  if (!workspace || workspace_bytes < p.total()) return PKV_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return PKV_ERR_ALIGN;
  // workgroups of eight 16-row units (a request of n tokens: ceil(n group / 16))
  const int64_t units = (int64_t(num_q_tokens) * group + pf::kUnitRows - 1) / pf::kUnitRows +
                        num_reqs;
  const int64_t wide = (units + pf::kUnits - 1) / pf::kUnits * num_kv_heads;
  const int64_t narrow = (int64_t(num_reqs) * p.runs_per_req * num_kv_heads + 3) / 4;
  // persistent: two workgroups per compute unit (the occupancy the LDS and
  // registers allow), never more than the longest queue needs
  int device = 0, cus = 0;
  if (hipGetDevice(&device) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus <= 0)
    return PKV_ERR_LAUNCH;
  const int64_t per_queue = std::min<int64_t>(
      (wide + kQueues - 1) / kQueues + (narrow + kQueues - 1) / kQueues,
      (2 * int64_t(cus) + kQueues - 1) / kQueues);
  const int64_t grid = per_queue * kQueues;
  if (grid > 0x7fffffff || int64_t(num_reqs) * num_kv_heads > 0x7fffffff) return PKV_ERR_SHAPE;
  if (p.wide_cap > 0x7fffffff || p.narrow_cap > 0x7fffffff ||
      (units + pf::kUnits - 1) / pf::kUnits * pf::kUnits > 0x7fffffff)
    return PKV_ERR_SHAPE;
  char* ws = static_cast<char*>(workspace);
  Plan plan;
  plan.tickets = reinterpret_cast<int32_t*>(ws);
  plan.cu_slots = reinterpret_cast<int32_t*>(ws + align256((kNarrowCount + 1) * sizeof(int32_t)));
  plan.wide_map = reinterpret_cast<int2*>(ws + p.ticket_bytes);
  plan.narrow_map = reinterpret_cast<int2*>(ws + p.ticket_bytes + p.wide_bytes);
  plan.wide_cap = int32_t(p.wide_cap);
  plan.narrow_cap = int32_t(p.narrow_cap);
  char* parts = ws + p.ticket_bytes + p.wide_bytes + p.narrow_bytes;
  float* part_o = reinterpret_cast<float*>(parts);
  float2* part_ml = reinterpret_cast<float2*>(parts + p.o_bytes);
  hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(kPlanThreads), 0, as_stream(stream),
                     query_start_loc, num_computed_tokens, num_reqs, group, max_blocks_per_seq,
                     p.runs_per_req, plan);
  hipLaunchKernelGGL(varlen_kernel, dim3(uint32_t(grid)), dim3(256), 0, as_stream(stream),
                     static_cast<uint16_t*>(out), static_cast<const uint16_t*>(query),
                     static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), num_blocks, block_tables,
                     max_blocks_per_seq, query_start_loc, num_computed_tokens, num_q_heads,
                     num_kv_heads, group, softmax_scale * pf::kLog2e, int32_t(wide),
                     int32_t(narrow), p.runs_per_req, plan, part_o, part_ml);
  if (p.runs_per_req > 1)
    hipLaunchKernelGGL(varlen_merge_kernel, dim3(uint32_t(num_reqs * num_kv_heads)), dim3(256),
                       0, as_stream(stream), static_cast<uint16_t*>(out), query_start_loc,
                       num_computed_tokens, max_blocks_per_seq, num_q_heads, num_kv_heads, group,
                       p.runs_per_req, part_o, part_ml);
  return launch_status();
}
