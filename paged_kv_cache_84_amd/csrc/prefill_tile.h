// Chunked-prefill tile on the gfx950 matrix cores (bf16, head_dim 128): the
// device code shared by the prefill kernel and the unified varlen kernel.
//
// A prompt chunk's rows attend causally to every earlier token of their
// request, read through its block table ("vLLM 引擎解剖", section
// "V1：统一调度预填充与解码", Fig. 3; "v1/v0 区别", §3.1 "Token 预算").  For a
// chunk, QK^T and PV are dense contractions, so both run on MFMA
// (v_mfma_f32_16x16x32_bf16), with fp32 accumulation.
//
// Work decomposition.  A workgroup (4 waves) owns 128 query rows of one
// request and one kv head; rows are (token, q head) pairs of the kv head's
// group, so the group's heads share every K/V tile.  Workgroups are numbered
// kv-head-fastest, which puts one kv head on each of the eight XCDs (their L2
// caches then each hold one head's shared prefix).
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


// One workgroup (4 waves) of the chunked prefill: token tile `tile_in_req` of
// request `req`, kv head `kvh`.  stage0 and stage1 are the workgroup's two
// LDS stages, passed as separate objects so the compiler can tell the stage
// being read from the stage the copies are writing.
PKV_DEVICE void prefill_tile_at(
    pf::Stage& stage0, pf::Stage& stage1, int req, int tile_in_req, int kvh,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    int32_t num_blocks, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ num_computed,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t group, float scale_log2) {
  using namespace pf;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tokens_per_wg = kRows / group;
  const int q_begin = load_scalar(query_start_loc, req);
  const int n_req = load_scalar(query_start_loc, req + 1) - q_begin;
  const int computed = load_scalar(num_computed, req);
  const int tok0 = tile_in_req * tokens_per_wg;
  const int ntok = min(tokens_per_wg, n_req - tok0);
  const int first_pos = computed + tok0;           // position of the tile's first query
  const int kv_len = first_pos + ntok;             // keys 0 .. kv_len-1 are visible
  const int ntiles = (kv_len + kKeys - 1) / kKeys;
  const int32_t* trow = block_tables + int64_t(req) * max_blocks;

  // ---- this lane's queries (one per 16-row block) and their Q fragments
  const int g = lane >> 4;          // lane group: keys 4g..4g+3 of a 16-key block
  const int n16 = lane & 15;
  const bool wave_active = wave * kRowsPerWave < ntok * group;
  int qpos[2];
  bool qvalid[2];
  u32x4 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = wave * kRowsPerWave + qb * 16 + n16;
    const int t = row / group;
    const int h = kvh * group + row % group;
    qvalid[qb] = t < ntok;
    qpos[qb] = qvalid[qb] ? first_pos + t : -1;
    const int tc = qvalid[qb] ? t : 0;      // keep the address inside the chunk
    const uint16_t* qp = query + (int64_t(q_begin + tok0 + tc) * num_q_heads + h) * kD + g * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[qb][ks] = qvalid[qb] ? load16(qp + ks * 32) : u32x4{0, 0, 0, 0};
  }

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
  auto table_id = [&](int lb) -> int32_t {
    return lb < max_blocks ? load_scalar(trow, lb) : -1;
  };
  // issue the copies of logical block lb (id already read) into a stage
  auto copy_block = [&](pf::Stage& st, int lb, int32_t id) {
    int rows = min(max(kv_len - lb * kBlock, 0), kBlock);
    const bool usable = id >= 0 && id < num_blocks;
    // flag for compute(): inside the context but unusable
    if (lane == 0) st.bad[wave] = (rows > 0 && !usable) ? 1u : 0u;
    if (!usable) rows = 0;
    const int32_t b = rows > 0 ? id : 0;
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

  auto compute = [&](const pf::Stage& st, int kt) {
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
            if (key0 + kb * 16 + r > qpos[qb]) s[kb][qb][r] = -INFINITY;
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

  // ---- the key loop: tile kt is read from stage kt % 2 while tile kt + 1
  // is copied into the other stage; block ids come one tile ahead of that.
  int32_t id_next = table_id(wave);               // tile 0
  int32_t id_after = table_id(kKeys / kBlock + wave);   // tile 1
  copy_block(stage0, wave, id_next);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; kt += 2) {
    // even tile from stage 0, its successor copied into stage 1
    {
      const bool more = kt + 1 < ntiles;
      if (more) {
        id_next = id_after;
        id_after = table_id((kt + 2) * (kKeys / kBlock) + wave);
        copy_block(stage1, (kt + 1) * (kKeys / kBlock) + wave, id_next);
      }
      if (wave_active) compute(stage0, kt);
      if (!more) break;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
    }
    // odd tile from stage 1
    {
      const bool more = kt + 2 < ntiles;
      if (more) {
        id_next = id_after;
        id_after = table_id((kt + 3) * (kKeys / kBlock) + wave);
        copy_block(stage0, (kt + 2) * (kKeys / kBlock) + wave, id_next);
      }
      if (wave_active) compute(stage1, kt + 1);
      if (!more) break;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
    }
  }

  if (!wave_active) return;
  // ---- normalise and write: lane holds d = db*16 + 4g + 0..3 of its query
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l[qb];
    lt += shfl_xor(lt, 16);
    lt += shfl_xor(lt, 32);
    if (!qvalid[qb]) continue;
    const float inv = 1.0f / lt;
    const int row = wave * kRowsPerWave + qb * 16 + n16;
    const int t = row / group;
    const int h = kvh * group + row % group;
    uint16_t* op = out + (int64_t(q_begin + tok0 + t) * num_q_heads + h) * kD + 4 * g;
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

// The same, with the piece found by a scan over the requests: token tile
// `wg / num_kv_heads` of the requests' tiles, kv head `wg % num_kv_heads`.
// Requests with at most `narrow_rows` query rows (tokens x group) get no
// tiles (another path serves them; 0 = every request).
PKV_DEVICE void prefill_tile(
    pf::Stage& stage0, pf::Stage& stage1, int wg, int narrow_rows,
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    int32_t num_blocks, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ num_computed,
    int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t group,
    float scale_log2) {
  using namespace pf;
  const int lane = threadIdx.x & (kWave - 1);
  const int tokens_per_wg = kRows / group;

  // ---- which (request, token tile, kv head) this workgroup owns
  const int kvh = wg % num_kv_heads;
  const int tile = wg / num_kv_heads;
  int req = -1, tile_in_req = 0;
  {
    int before = 0;
    for (int base = 0; base < num_reqs; base += kWave) {
      const int r = base + lane;
      const int n = r < num_reqs ? query_start_loc[r + 1] - query_start_loc[r] : 0;
      const int tiles = (n > 0 && n * group > narrow_rows) ? (n + tokens_per_wg - 1) / tokens_per_wg : 0;
      const int incl = wave_scan(tiles);
      const uint64_t hit = __ballot(before + incl > tile);
      if (hit) {
        const int first = __builtin_ctzll(hit);
        const int incl_first = __shfl(incl, first, kWave);
        const int tiles_first = __shfl(tiles, first, kWave);
        req = base + first;
        tile_in_req = tile - (before + incl_first - tiles_first);
        break;
      }
      before += __shfl(incl, kWave - 1, kWave);
    }
  }
  req = __builtin_amdgcn_readfirstlane(req);
  tile_in_req = __builtin_amdgcn_readfirstlane(tile_in_req);
  if (req < 0) return;
  prefill_tile_at(stage0, stage1, req, tile_in_req, kvh, out, query, k_cache, v_cache,
                  num_blocks, block_tables, max_blocks, query_start_loc, num_computed,
                  num_q_heads, num_kv_heads, group, scale_log2);
}

}  // namespace pkv
