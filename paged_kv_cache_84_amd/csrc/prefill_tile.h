// Chunked-prefill tile on the gfx950 matrix cores (bf16, head_dim 128): the
// device code shared by the prefill kernel and the unified varlen kernel.
//
// A prompt chunk's rows attend causally to every earlier token of their
// request, read through its block table ("vLLM 引擎解剖", section
// "V1：统一调度预填充与解码", Fig. 3; "v1/v0 区别", §3.1 "Token 预算").  For a
// chunk, QK^T and PV are dense contractions, so both run on MFMA
// (v_mfma_f32_16x16x32_bf16), with fp32 accumulation.
//
// Work decomposition.  A workgroup (4 waves) owns 128 query rows and one kv
// head; rows are (token, q head) pairs of the kv head's group, so the
// group's heads share every K/V tile.  The rows are eight 16-row units taken
// in order from the requests' rows, so a workgroup may hold the end of one
// request and the start of the next (details above prefill_units).
// Workgroups are numbered kv-head-fastest, which puts one kv head on each of
// the eight XCDs (their L2 caches then each hold one head's shared prefix).
//
// Staging.  Keys are walked in tiles of 64 (four 16-token blocks gathered
// through the block table).  Each wave copies one block of K and of V
// straight from global memory into LDS (buffer loads with the LDS-destination
// bit: no register round trip), through a buffer resource that spans only
// the block's valid rows, so rows past the context and unusable block ids
// arrive as zeros (and the keys of an unusable id are then masked to -inf).  Two LDS stages alternate: the next tile is in flight
// while the current one is multiplied; one barrier per tile.  Rows are 256
// bytes; the sixteen 16-byte pieces of a row are stored XOR-swizzled by the
// row index so that both fragment reads below are free of bank conflicts
// (the swizzle is applied on the global side, by choosing which piece each
// lane fetches).
//
// Per wave (32 rows = two 16-row blocks) and 64-key tile:
//   S^T = K Q^T    A = K rows (ds_read_b128), B = the wave's Q in registers;
//                  each lane then holds one query and four keys per block;
//   softmax        online, base 2; the running max of a query is raised only
//                  when a score exceeds it by more than 8 (a factor 256 in the
//                  weights, harmless in fp32), so the cross-lane max and the
//                  rescale run only on the rare raise;
//   O^T += V^T P^T A = V^T read from row-major V by the transposing LDS read
//                  ds_read_b64_tr_b16, B = P^T straight from the S^T
//                  registers: the k order of the product is the permutation
//                  of the 32 keys that both layouts share, so no lane
//                  exchange is needed.
// P is fed to the second product as a pair of bf16 numbers (P = hi + lo, lo
// the bf16 rounding of the remainder), so P carries ~16 significant bits and
// the result keeps fp32-level accuracy.

#pragma once

#include <math.h>

#include "common.h"

namespace pkv {
namespace pf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t2 __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRows = kWaves * kRowsPerWave;   // query rows per workgroup
constexpr int kUnitRows = 16;                  // rows of a unit (one MFMA column block)
constexpr int kUnits = kRows / kUnitRows;      // units per workgroup, two per wave
constexpr int kKeys = 64;                      // keys per tile (four blocks)
constexpr int kRowBytes = kD * 2;              // one K or V row
constexpr int kTileBytes = kKeys * kRowBytes;  // 16 KiB
constexpr int kBlockBytes = kBlock * kRowBytes;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRaise = 8.0f;
constexpr float kNoMax = -1e30f;               // running max before any key

// s_waitcnt with vmcnt = 0 and the other counters left free.
constexpr int kWaitVm0 = 0x0F70;

PKV_DEVICE f32x4_t mfma(u32x4 a, u32x4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

PKV_DEVICE uint32_t pack_bf16(float a, float b) {
  bf16x2_t2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Physical 16-byte piece of logical piece c in row r.  K: c ^ (r mod 16);
// V: c ^ 2 (r mod 8), which keeps the two pieces of every 32-byte run
// together (the transposing read fetches 32 contiguous bytes per key).
PKV_DEVICE int k_piece(int r, int c) { return c ^ (r & 15); }
PKV_DEVICE int v_piece(int r, int c) { return c ^ ((r & 7) << 1); }

// Inclusive prefix sum over the wave.
PKV_DEVICE int wave_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// One LDS stage: the K and V rows of a 64-key tile (row-major, swizzled),
// and which of its four blocks have unusable ids.
struct Stage {
  u32x4 k[kTileBytes / 16];
  u32x4 v[kTileBytes / 16];
  uint32_t bad[kWaves];   // block w of the tile: inside the context, unusable id
};

}  // namespace pf


// One workgroup (4 waves) of the chunked prefill over kv head `kvh`.
//
// Its query rows are eight 16-row units taken in order from the requests'
// rows (a request's rows are its (token, q head) pairs of the kv head's
// group, token-major, so a unit holds 16 / group whole tokens).  Lane i < 8
// passes unit i as (request, index of the unit in that request's rows);
// request < 0 marks a unit past the last one.  Wave w owns units 2w and
// 2w + 1, one per 16-row block of its S^T columns.  So a request's rows are
// cut into workgroups without a partly empty workgroup at each request's
// end: a request of 100 tokens at group 4 is 25 units, not three full tiles
// and a fourth of 16 rows.
//
// Keys are walked in 64-key tiles in order.  At tile kt, the requests of the
// workgroup whose four block ids for the tile are the same (requests on a
// shared prefix, "PagedAttention：为 KV 缓存分页", the sharing of physical
// blocks) are served by one staged copy; a request whose ids differ gets a
// copy of its own, one after the other.  A wave multiplies only the copies
// of its units' requests.  Within such a copy, a row of another request has
// every score masked: its weights are 0, its rescale factor exactly 1 and
// its products add exact zeros, so its running max, sum and output are
// untouched.  Every row therefore sees exactly the tiles of its own request,
// in order, with the same arithmetic whatever else shares its workgroup, and
// a prompt's rows come out the same however its chunks are cut.
//
// stage0 and stage1 are the workgroup's two LDS stages, passed as separate
// objects so the compiler can tell the stage being read from the stage the
// copies are writing.
PKV_DEVICE void prefill_units(
    pf::Stage& stage0, pf::Stage& stage1, int unit_req, int unit_idx, int kvh,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    int32_t num_blocks, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ num_computed,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t group, float scale_log2) {
  using namespace pf;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tpu = kUnitRows / group;     // tokens per unit

  // ---- the units, lane i < 8 holding unit i
  const int ur = lane < kUnits ? unit_req : -1;
  const int uu = lane < kUnits ? unit_idx : 0;
  const bool uvalid = ur >= 0;
  int ubeg = 0, un = 0, ucomp = 0;
  if (uvalid) {
    ubeg = query_start_loc[ur];
    un = query_start_loc[ur + 1] - ubeg;
    ucomp = num_computed[ur];
  }
  const uint64_t valids = __ballot(uvalid);
  if (valids == 0) return;      // the same for every wave of the workgroup
  // keys the unit's rows see (through its last token)
  const int ukeys = uvalid ? ucomp + min(uu * tpu + tpu, un) : 0;
  // a request's first unit in the workgroup is its slot
  const int prev = __shfl_up(ur, 1, kWave);
  const bool ufirst = uvalid && (lane == 0 || prev != ur);
  const uint64_t firsts = __ballot(ufirst);
  const int uslot = uvalid ? 63 - __builtin_clzll(firsts & ((2ull << lane) - 1)) : 0;
  // keys a slot's request sees in this workgroup: those of its last unit
  int skeys;
  {
    const uint64_t above = lane < kWave - 1 ? firsts >> (lane + 1) : 0;
    const int last = above ? lane + __builtin_ctzll(above) : __popcll(valids) - 1;
    const int k = __shfl(ukeys, last, kWave);
    skeys = ufirst ? k : 0;
  }
  const int stiles = (skeys + kKeys - 1) / kKeys;

  // ---- this wave's units (2 wave + qb), their rows and Q fragments
  const int g = lane >> 4;          // lane group: keys 4g..4g+3 of a 16-key block
  const int n16 = lane & 15;
  int qreq[2], qslot[2], fpos[2], qbeg[2], qpos[2];
  bool qvalid[2];
  u32x4 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int s = 2 * wave + qb;
    qreq[qb] = __builtin_amdgcn_readlane(ur, s);
    qslot[qb] = __builtin_amdgcn_readlane(uslot, s);
    qbeg[qb] = __builtin_amdgcn_readlane(ubeg, s);
    const int u = __builtin_amdgcn_readlane(uu, s);
    const int n = __builtin_amdgcn_readlane(un, s);
    const int c = __builtin_amdgcn_readlane(ucomp, s);
    fpos[qb] = c + u * tpu;         // position of the unit's first token
    const int row = u * kUnitRows + n16;
    const int t = row / group;
    const int h = kvh * group + row % group;
    qvalid[qb] = qreq[qb] >= 0 && t < n;
    qpos[qb] = qvalid[qb] ? c + t : -1;
    const int tc = qvalid[qb] ? t : 0;      // keep the address inside the batch
    const uint16_t* qp = query + (int64_t(qbeg[qb] + tc) * num_q_heads + h) * kD + g * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[qb][ks] = qvalid[qb] ? load16(qp + ks * 32) : u32x4{0, 0, 0, 0};
  }

  // ---- block ids of a tile: lane 4i + b < 32 holds block b of unit i's
  // request.  The loads are unconditional buffer loads (a lane without a
  // request reads past the range and gets 0), so a load in flight is never
  // merged into a register before it is used; entries past a table row are
  // replaced by -1 when the ids are used.
  const int idreq = __shfl(ur, (lane >> 2) & (kUnits - 1), kWave);
  const bool idlane = lane < 4 * kUnits && idreq >= 0;
  const int last_req = __builtin_amdgcn_readlane(ur, __popcll(valids) - 1);
  const auto id_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(block_tables), 0,
      int32_t(min<int64_t>((int64_t(last_req) + 1) * max_blocks * 4, 0x7fffffff)),
      kRawBufferFlags);
  const uint32_t id_off =
      idlane ? uint32_t((int64_t(idreq) * max_blocks + (lane & 3)) * 4) : 0x80000000u;
  auto load_ids = [&](int kt) -> int32_t {
    return __builtin_amdgcn_raw_buffer_load_b32(id_rsrc, id_off + uint32_t(kt) * 16, 0, 0);
  };
  auto ids_at = [&](int32_t raw, int kt) -> int32_t {
    return idlane && kt * 4 + (lane & 3) < max_blocks ? raw : -1;
  };
  // slots whose request reaches tile kt
  auto active = [&](int kt) -> uint32_t { return uint32_t(__ballot(ufirst && kt < stiles)); };
  // the copy that serves `pend`'s first slot, and the pending slots it serves
  auto pick = [&](uint32_t pend, int32_t ids, int& lead, uint32_t& members) {
    lead = __builtin_ctz(pend);
    members = 1u << lead;
    if (pend != members) {
      const int32_t lid = __shfl(ids, 4 * lead + (lane & 3), kWave);
      const uint64_t eq = __ballot(lane < 4 * kUnits && ids == lid);
      const uint32_t e = uint32_t(eq);
      const uint32_t all4 = e & (e >> 1) & (e >> 2) & (e >> 3);
#pragma unroll
      for (int i = 1; i < kUnits; ++i) members |= ((all4 >> (4 * i)) & 1u) << i;
      members &= pend;
    }
  };
  // keys the members' requests see: the copy stages no row past them
  auto member_keys = [&](int lead, uint32_t members) -> int {
    if (members == (1u << lead)) return __builtin_amdgcn_readlane(skeys, lead);
    int k = (lane < kUnits && ((members >> (lane & 7)) & 1u)) ? skeys : 0;
    k = max(k, __shfl_xor(k, 1, kWave));
    k = max(k, __shfl_xor(k, 2, kWave));
    k = max(k, __shfl_xor(k, 4, kWave));
    return __builtin_amdgcn_readfirstlane(k);
  };

  // ---- staging: wave w copies block w of each tile (4 x 1 KiB per cache).
  // Copy i writes rows 4i..4i+3 of the block; lane L lands on row 4i + L/16,
  // physical piece L%16, so it fetches the logical piece that maps there.
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int p = lane & 15;
    koff[i] = uint32_t(r * kRowBytes + k_piece(r, p) * 16);   // k_piece is an involution
    voff[i] = uint32_t(r * kRowBytes + v_piece(r, p) * 16);
  }
  const int64_t head_bytes = int64_t(kBlockBytes);
  const int64_t block_bytes = int64_t(num_kv_heads) * head_bytes;
  const char* kbase = reinterpret_cast<const char*>(k_cache) + int64_t(kvh) * head_bytes;
  const char* vbase = reinterpret_cast<const char*>(v_cache) + int64_t(kvh) * head_bytes;
  // a copy to stage: tile kt, leading slot, member slots, and for this
  // wave's block the id and the rows inside the members' contexts
  struct Copy {
    int kt, lead, rows;
    uint32_t members;
    int32_t id;
  };
  // issue the copies of this wave's block of a copy into a stage
  auto copy_block = [&](pf::Stage& st, const Copy& c) {
    int rows = c.rows;
    const bool usable = c.id >= 0 && c.id < num_blocks;
    // flag for compute(): inside the context but unusable
    if (lane == 0) st.bad[wave] = (rows > 0 && !usable) ? 1u : 0u;
    if (!usable) rows = 0;
    const int32_t b = rows > 0 ? c.id : 0;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kbase + int64_t(b) * block_bytes), 0, rows * kRowBytes, kRawBufferFlags);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vbase + int64_t(b) * block_bytes), 0, rows * kRowBytes, kRawBufferFlags);
    lds_char_t* kd = (lds_char_t*)(&st.k[0]) + wave * kBlockBytes;
    lds_char_t* vd = (lds_char_t*)(&st.v[0]) + wave * kBlockBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, kd + i * 1024, 16, koff[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, vd + i * 1024, 16, voff[i], 0, 0, 0);
  };

  // ---- fragment addresses inside a stage
  // K (A of S^T): row kb*16 + n16, logical piece ks*4 + g
  uint32_t ka[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) ka[ks] = uint32_t(n16 * kRowBytes + k_piece(n16, ks * 4 + g) * 16);
  // V (A of O^T, transposing read): lane g*16 + 4e + q addresses key
  // kb*16 + 4g + e, dims db*16 + 4q .. +3
  const int e = (lane >> 2) & 3, q4 = lane & 3;
  const int vkey = 4 * g + e;
  uint32_t va[8];
#pragma unroll
  for (int db = 0; db < 8; ++db)
    va[db] = uint32_t(vkey * kRowBytes + v_piece(vkey, 2 * db + (q4 >> 1)) * 16 + (q4 & 1) * 8);

  // ---- running state: O^T fragments (8 d-blocks x 2 query blocks), max, sum
  f32x4_t o[8][2];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {kNoMax, kNoMax};
  float l[2] = {0.f, 0.f};

  // qp[qb]: positions the causal mask compares with (-1: every key masked);
  // first_pos: the smallest of them over the wave's rows that take part
  auto compute = [&](const pf::Stage& st, int kt, const int (&qp)[2], int first_pos) {
    lds_char_t* kl = (lds_char_t*)(&st.k[0]);
    lds_char_t* vl = (lds_char_t*)(&st.v[0]);
    // S^T for the 64 keys x 32 queries of this wave
    f32x4_t s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 a = *reinterpret_cast<lds_u32x4_t*>(kl + ka[ks] + kb * kBlockBytes);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mfma(a, qf[qb][ks], s[kb][qb]);
      }
    }
    // a block inside the context whose id is unusable contributes nothing:
    // the wave that staged it left a flag in the stage, and its keys get -inf
    {
      const u32x4 bad = *reinterpret_cast<lds_u32x4_t*>((lds_char_t*)(&st.bad[0]));
      if (__builtin_expect((bad[0] | bad[1] | bad[2] | bad[3]) != 0, 0)) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          if (bad[kb])
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              s[kb][qb] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
    }
    // causal mask on tiles that reach past the first query's position
    // (keys past the context are past every query, so this covers them too)
    if (kt * kKeys + kKeys - 1 > first_pos) {
      const int key0 = kt * kKeys + 4 * g;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + kb * 16 + r > qp[qb]) s[kb][qb][r] = -INFINITY;
    }
    // does any score exceed its query's running max by more than kRaise?
    // (the scale is positive, so the raw maximum decides)
    float lmax[2];
    bool raise = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = fmaxf(fmaxf(s[0][qb][0], s[0][qb][1]), s[0][qb][2]);
      mx = fmaxf(fmaxf(mx, s[0][qb][3]), s[1][qb][0]);
      mx = fmaxf(fmaxf(mx, s[1][qb][1]), s[1][qb][2]);
      mx = fmaxf(fmaxf(mx, s[1][qb][3]), s[2][qb][0]);
      mx = fmaxf(fmaxf(mx, s[2][qb][1]), s[2][qb][2]);
      mx = fmaxf(fmaxf(mx, s[2][qb][3]), s[3][qb][0]);
      mx = fmaxf(fmaxf(mx, s[3][qb][1]), s[3][qb][2]);
      mx = fmaxf(mx, s[3][qb][3]);
      lmax[qb] = mx * scale_log2;
      raise |= lmax[qb] > m[qb] + kRaise;
    }
    if (__builtin_expect(__ballot(raise) != 0, 0)) {
      // only the rows that need it are raised: a row's arithmetic then never
      // depends on the other rows of its wave, so the rows come out the same
      // however the chunks of a prompt are cut
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = lmax[qb];
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float mn = mx > m[qb] + kRaise ? mx : m[qb];
        const float alpha = fast_exp2(m[qb] - mn);
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][qb] *= alpha;
        m[qb] = mn;
      }
    }
    // P = 2^(s * scale - m), split into bf16 hi + lo, as the B operand of
    // O^T += V^T P^T; keys kb0*16 + 4g + 0..3, then kb1*16 + 4g + 0..3
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 phi[2], plo[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float nm = -m[qb];
        float p[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = fast_exp2(fmaf(s[2 * kk][qb][r], scale_log2, nm));
          p[4 + r] = fast_exp2(fmaf(s[2 * kk + 1][qb][r], scale_log2, nm));
        }
        l[qb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t ua = __float_as_uint(p[2 * w]), ub = __float_as_uint(p[2 * w + 1]);
          phi[qb][w] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
          plo[qb][w] = pack_bf16(p[2 * w] - __uint_as_float(ua & 0xffff0000u),
                                 p[2 * w + 1] - __uint_as_float(ub & 0xffff0000u));
        }
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const i16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_i16x4_t*>(vl + va[db] + (2 * kk) * kBlockBytes));
        const i16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<lds_i16x4_t*>(vl + va[db] + (2 * kk + 1) * kBlockBytes));
        const uint2 xu = __builtin_bit_cast(uint2, x), yu = __builtin_bit_cast(uint2, y);
        const u32x4 a = {xu.x, xu.y, yu.x, yu.y};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          o[db][qb] = mfma(a, phi[qb], o[db][qb]);
          o[db][qb] = mfma(a, plo[qb], o[db][qb]);
        }
      }
    }
  };
  // multiply the staged copy if it serves one of this wave's units
  auto take = [&](const pf::Stage& st, int kt, uint32_t members) {
    bool in[2];
    int qp[2], first_pos = 0x7fffffff;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      in[qb] = qreq[qb] >= 0 && ((members >> qslot[qb]) & 1u);
      qp[qb] = in[qb] ? qpos[qb] : -1;
      // a unit of another request: every key masked; a unit past the end:
      // rows that are never written, no constraint
      if (qreq[qb] >= 0) first_pos = min(first_pos, in[qb] ? fpos[qb] : -1);
    }
    if (in[0] || in[1]) compute(st, kt, qp, first_pos);
  };

  if (firsts == 1) {
    // ---- one request: one copy per tile, its block ids by scalar loads two
    // tiles ahead
    const int kv = __builtin_amdgcn_readlane(skeys, 0);
    const int ntiles = (kv + kKeys - 1) / kKeys;
    const int32_t* trow = block_tables + int64_t(__builtin_amdgcn_readlane(ur, 0)) * max_blocks;
    auto table_id = [&](int lb) -> int32_t {
      return lb < max_blocks ? load_scalar(trow, lb) : -1;
    };
    auto single = [&](int kt, int32_t id) {
      Copy c;
      c.kt = kt;
      c.lead = 0;
      c.members = 1;
      c.id = id;
      c.rows = min(max(kv - (kt * (kKeys / kBlock) + wave) * kBlock, 0), kBlock);
      return c;
    };
    int32_t id_next = table_id(wave);
    int32_t id_after = table_id(kKeys / kBlock + wave);
    copy_block(stage0, single(0, id_next));
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    for (int kt = 0; kt < ntiles; kt += 2) {
      {
        const bool more = kt + 1 < ntiles;
        if (more) {
          id_next = id_after;
          id_after = table_id((kt + 2) * (kKeys / kBlock) + wave);
          copy_block(stage1, single(kt + 1, id_next));
        }
        take(stage0, kt, 1u);
        if (!more) break;
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
      }
      {
        const bool more = kt + 2 < ntiles;
        if (more) {
          id_next = id_after;
          id_after = table_id((kt + 3) * (kKeys / kBlock) + wave);
          copy_block(stage0, single(kt + 2, id_next));
        }
        take(stage1, kt + 1, 1u);
        if (!more) break;
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
      }
    }
  } else {
  // ---- the walk over copies.  ids_c holds the ids of tile nkt (the tile of
  // the last copy decided); raw_n those of tile nkt + 1, reloaded before
  // each copy is issued.  A copy is decided one copy ahead, after the
  // products of the copy before it are issued, so that the walk's scalar
  // work overlaps the tail of those products and the barrier.
  int nkt = 0;
  uint32_t covered = 0;
  int32_t ids_c = ids_at(load_ids(0), 0);
  int32_t raw_n = load_ids(1);
  auto advance = [&](Copy& c) -> bool {
    uint32_t pend = active(nkt) & ~covered;
    if (pend == 0) {
      ++nkt;
      covered = 0;
      ids_c = ids_at(raw_n, nkt);
      pend = active(nkt);
      if (pend == 0) return false;
    }
    pick(pend, ids_c, c.lead, c.members);
    covered |= c.members;
    c.kt = nkt;
    const int lb = nkt * (kKeys / kBlock) + wave;
    c.id = __builtin_amdgcn_readlane(ids_c, 4 * c.lead + wave);
    c.rows = min(max(member_keys(c.lead, c.members) - lb * kBlock, 0), kBlock);
    return true;
  };

  // ---- the key loop: copy c is read from stage c % 2 while copy c + 1 is
  // staged into the other stage
  Copy cur, nxt, nn;
  advance(cur);                   // a valid unit sees at least one key
  copy_block(stage0, cur);
  bool more = advance(nxt);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  for (;;) {
    {
      raw_n = load_ids(nkt + 1);
      if (more) copy_block(stage1, nxt);
      take(stage0, cur.kt, cur.members);
      if (!more) break;
      const bool more2 = advance(nn);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      cur = nxt;
      nxt = nn;
      more = more2;
    }
    {
      raw_n = load_ids(nkt + 1);
      if (more) copy_block(stage0, nxt);
      take(stage1, cur.kt, cur.members);
      if (!more) break;
      const bool more2 = advance(nn);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      cur = nxt;
      nxt = nn;
      more = more2;
    }
  }
  }

  // ---- normalise and write: lane holds d = db*16 + 4g + 0..3 of its query
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l[qb];
    lt += shfl_xor(lt, 16);
    lt += shfl_xor(lt, 32);
    if (!qvalid[qb]) continue;
    const float inv = 1.0f / lt;
    const int row = __builtin_amdgcn_readlane(uu, 2 * wave + qb) * kUnitRows + n16;
    const int t = row / group;
    const int h = kvh * group + row % group;
    uint16_t* op = out + (int64_t(qbeg[qb] + t) * num_q_heads + h) * kD + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint32_t w0 = uint32_t(f32_to_bf16(o[db][qb][0] * inv)) |
                          (uint32_t(f32_to_bf16(o[db][qb][1] * inv)) << 16);
      const uint32_t w1 = uint32_t(f32_to_bf16(o[db][qb][2] * inv)) |
                          (uint32_t(f32_to_bf16(o[db][qb][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(op + db * 16) = make_uint2(w0, w1);
    }
  }
}

// The same, with the units found by a scan over the requests: units
// 8 * (wg / num_kv_heads) .. +7 of all requests' units in order, kv head
// wg % num_kv_heads.
PKV_DEVICE void prefill_tile(
    pf::Stage& stage0, pf::Stage& stage1, int wg,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    int32_t num_blocks, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ num_computed,
    int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t group,
    float scale_log2) {
  using namespace pf;
  const int lane = threadIdx.x & (kWave - 1);
  const int kvh = wg % num_kv_heads;
  const int first = (wg / num_kv_heads) * kUnits;    // the workgroup's first unit
  int ureq = -1, uidx = 0;
  int before = 0;
  for (int base = 0; base < num_reqs && before < first + kUnits; base += kWave) {
    const int r = base + lane;
    const int n = r < num_reqs ? query_start_loc[r + 1] - query_start_loc[r] : 0;
    const int units = n > 0 ? int((int64_t(n) * group + kUnitRows - 1) / kUnitRows) : 0;
    const int incl = wave_scan(units);
    // unit t lies in the first request whose inclusive count passes it
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      const uint64_t hit = __ballot(before + incl > first + i);
      if (hit != 0) {
        const int j = __builtin_ctzll(hit);
        const int start = before + __shfl(incl - units, j, kWave);
        if (lane == i && ureq < 0) {
          ureq = base + j;
          uidx = first + i - start;
        }
      }
    }
    before += __shfl(incl, kWave - 1, kWave);
  }
  prefill_units(stage0, stage1, ureq, uidx, kvh, out, query, k_cache, v_cache, num_blocks,
                block_tables, max_blocks, query_start_loc, num_computed, num_q_heads,
                num_kv_heads, group, scale_log2);
}

}  // namespace pkv
