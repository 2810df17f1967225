// Chunked-prefill attention on the gfx950 matrix cores (bf16, head_dim 128).
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
// caches then each hold one head's shared prefix).  The keys are walked in
// tiles of 64 (four 16-token blocks gathered through the block table),
// staged in LDS and double-buffered: the next tile's global loads are in
// flight while the current tile is multiplied.
//
// Per wave (32 rows, two 16-row blocks) and 64-key tile:
//   S^T = K Q^T   A = K rows from LDS, B = the wave's Q (registers), so the
//                 result holds, in each lane, one query and four keys;
//   softmax       online, base 2, running max per query raised only when a
//                 score exceeds it by more than 8, so rescaling is rare; the
//                 statistics of a query live in the lanes that hold it;
//   O^T += V^T P^T  A = V^T from LDS (V is written transposed into LDS),
//                 B = P^T straight from the S^T registers: the k order of the
//                 product is a permutation of the 32 keys chosen so that no
//                 lane exchange is needed.
// P is fed to the second product as a pair of bf16 numbers (P = hi + lo, lo
// the bf16 rounding of the remainder), so P carries ~16 significant bits and
// the result keeps fp32-level accuracy.

#include <math.h>

#include "abi_util.h"
#include "common.h"
#include "prefill_args.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t2 __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRows = kWaves * kRowsPerWave;   // query rows per workgroup
constexpr int kKeys = 64;                      // keys per tile
constexpr int kKStride = kD * 2 + 16;          // LDS bytes per K row
constexpr int kVtStride = 152;                 // LDS bytes per V^T row (64 keys + pad)
constexpr int kKBytes = kKeys * kKStride;      // 17408
constexpr int kVBytes = kD * kVtStride;        // 19456
constexpr int kStage = kKBytes + kVBytes;      // one buffered tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRaise = 8.0f;
constexpr float kNoMax = -1e30f;               // running max before any key

PKV_DEVICE f32x4_t mfma(u32x4 a, u32x4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

PKV_DEVICE uint32_t pack_bf16(float a, float b) {
  bf16x2_t2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

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

struct TileRegs {
  u32x4 k[4];      // four 16-byte pieces of K rows
  u32x4 v[4];      // two key pairs x (key 2p, key 2p+1) 16-byte pieces
};

}  // namespace

__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    int32_t num_blocks, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ query_start_loc, const int32_t* __restrict__ num_computed,
    int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t group,
    float scale_log2) {
  extern __shared__ __align__(16) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int tokens_per_wg = kRows / group;

  // ---- which (request, token tile, kv head) this workgroup owns
  const int kvh = blockIdx.x % num_kv_heads;
  const int tile = blockIdx.x / num_kv_heads;
  int req = -1, tile_in_req = 0;
  {
    int before = 0;
    for (int base = 0; base < num_reqs; base += kWave) {
      const int r = base + lane;
      const int n = r < num_reqs ? query_start_loc[r + 1] - query_start_loc[r] : 0;
      const int tiles = n > 0 ? (n + tokens_per_wg - 1) / tokens_per_wg : 0;
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
  if (req < 0) return;
  const int q_begin = query_start_loc[req];
  const int n_req = query_start_loc[req + 1] - q_begin;
  const int computed = num_computed[req];
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

  // ---- staging of one 64-key tile: global -> registers -> LDS
  const int64_t head_stride = int64_t(kBlock) * kD;
  const int64_t block_stride = int64_t(num_kv_heads) * head_stride;
  auto block_of = [&](int kt, int j) -> int32_t {
    const int lb = kt * 4 + j;
    const int32_t b = lb < max_blocks ? trow[lb] : -1;
    return (b >= 0 && b < num_blocks) ? b : -1;
  };
  auto fetch = [&](TileRegs& tr, int kt) {
    int32_t ids[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ids[j] = block_of(kt, j);
    // K: piece p = tid + 256 i -> key p / 16, 16-byte chunk p % 16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i;
      const int key = p >> 4, chunk = p & 15;
      const int32_t b = ids[key >> 4];
      const bool ok = b >= 0 && kt * kKeys + key < kv_len;
      const uint16_t* src = k_cache + int64_t(ok ? b : 0) * block_stride + kvh * head_stride +
                            (key & 15) * kD + chunk * 8;
      tr.k[i] = ok ? load16(src) : u32x4{0, 0, 0, 0};
    }
    // V: key pair kp = (p / 4) % 32 ... two pairs per thread, 4 x 16 bytes
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      const int c = (p & 3) + 4 * (p >> 7);      // 16-byte chunk 0..15
      const int kp = (p >> 2) & 31;              // key pair 0..31
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = 2 * kp + h;
        const int32_t b = ids[key >> 4];
        const bool ok = b >= 0 && kt * kKeys + key < kv_len;
        const uint16_t* src = v_cache + int64_t(ok ? b : 0) * block_stride +
                              kvh * head_stride + (key & 15) * kD + c * 8;
        tr.v[2 * i + h] = ok ? load16(src) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store = [&](const TileRegs& tr, int stage) {
    char* kl = lds + stage * kStage;
    char* vl = kl + kKBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i;
      *reinterpret_cast<u32x4*>(kl + (p >> 4) * kKStride + (p & 15) * 16) = tr.k[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      const int c = (p & 3) + 4 * (p >> 7);
      const int kp = (p >> 2) & 31;
      const u32x4 v0 = tr.v[2 * i], v1 = tr.v[2 * i + 1];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int d = c * 8 + 2 * w;
        // (key 2kp, key 2kp+1) at column d, then at column d+1
        *reinterpret_cast<uint32_t*>(vl + d * kVtStride + kp * 4) =
            __builtin_amdgcn_perm(v1[w], v0[w], 0x05040100u);
        *reinterpret_cast<uint32_t*>(vl + (d + 1) * kVtStride + kp * 4) =
            __builtin_amdgcn_perm(v1[w], v0[w], 0x07060302u);
      }
    }
  };

  // ---- running state: O^T fragments (8 d-blocks x 2 query blocks), max, sum
  f32x4_t o[8][2];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {kNoMax, kNoMax};
  float l[2] = {0.f, 0.f};

  TileRegs tr;
  fetch(tr, 0);
  store(tr, 0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const bool more = kt + 1 < ntiles;
    if (more) fetch(tr, kt + 1);
    const char* kl = lds + (kt & 1) * kStage;
    const char* vl = kl + kKBytes;
    if (wave_active) {
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
          const u32x4 a = *reinterpret_cast<const u32x4*>(
              kl + (kb * 16 + n16) * kKStride + ks * 64 + g * 16);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mfma(a, qf[qb][ks], s[kb][qb]);
        }
      }
      // scale, causal / length mask, tile max per query
      const int key0 = kt * kKeys + 4 * g;
      const bool edge = kt * kKeys + kKeys - 1 > first_pos;   // tile crosses the diagonal
      float tmax[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float t = s[kb][qb][r] * scale_log2;
            if (edge) t = (key0 + kb * 16 + r <= qpos[qb]) ? t : -INFINITY;
            s[kb][qb][r] = t;
            mx = fmaxf(mx, t);
          }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        tmax[qb] = mx;
      }
      const bool raise = tmax[0] > m[0] + kRaise || tmax[1] > m[1] + kRaise;
      if (__builtin_expect(__ballot(raise) != 0, 0)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float mn = fmaxf(m[qb], tmax[qb]);
          const float alpha = fast_exp2(m[qb] - mn);
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) o[db][qb] *= alpha;
          m[qb] = mn;
        }
      }
      // P = 2^(s - m), split into bf16 hi + lo, as the B operand of O^T += V^T P^T
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 phi[2], plo[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          float p[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] = fast_exp2(s[2 * kk][qb][r] - m[qb]);
            p[4 + r] = fast_exp2(s[2 * kk + 1][qb][r] - m[qb]);
          }
          float sum = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) sum += p[e];
          l[qb] += sum;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float a = p[2 * w], b = p[2 * w + 1];
            const uint32_t hi = (__float_as_uint(b) & 0xffff0000u) | (__float_as_uint(a) >> 16);
            const float ra = a - __uint_as_float(__float_as_uint(a) & 0xffff0000u);
            const float rb = b - __uint_as_float(__float_as_uint(b) & 0xffff0000u);
            phi[qb][w] = hi;
            plo[qb][w] = pack_bf16(ra, rb);
          }
        }
        // V^T fragment rows d, keys {kb0*16 + 4g + 0..3} then {kb1*16 + 4g + 0..3}
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const char* row = vl + (db * 16 + n16) * kVtStride;
          const uint2 x = *reinterpret_cast<const uint2*>(row + (2 * kk * 16 + 4 * g) * 2);
          const uint2 y = *reinterpret_cast<const uint2*>(row + ((2 * kk + 1) * 16 + 4 * g) * 2);
          const u32x4 a = {x.x, x.y, y.x, y.y};
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            o[db][qb] = mfma(a, phi[qb], o[db][qb]);
            o[db][qb] = mfma(a, plo[qb], o[db][qb]);
          }
        }
      }
    }
    if (more) {
      __syncthreads();                 // everyone is done reading the other buffer
      store(tr, (kt + 1) & 1);
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

// Host launch: grid = (token tiles upper bound) x kv heads, kv head fastest.
pkv_status launch_prefill_mfma(const PrefillArgs& a) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int tokens_per_wg = kRows / group;
  const int64_t tiles = (int64_t(a.num_q_tokens) + tokens_per_wg - 1) / tokens_per_wg +
                        a.num_reqs;
  const int64_t grid = tiles * a.num_kv_heads;
  if (grid > 0x7fffffff) return PKV_ERR_SHAPE;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_mfma_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStage) != hipSuccess)
    return PKV_ERR_LAUNCH;
  hipLaunchKernelGGL(prefill_mfma_kernel, dim3(uint32_t(grid)), dim3(256), 2 * kStage,
                     as_stream(a.stream), static_cast<uint16_t*>(a.out),
                     static_cast<const uint16_t*>(a.query),
                     static_cast<const uint16_t*>(a.k_cache),
                     static_cast<const uint16_t*>(a.v_cache), a.num_blocks, a.block_tables,
                     a.max_blocks_per_seq, a.query_start_loc, a.num_computed_tokens,
                     a.num_reqs, a.num_q_heads, a.num_kv_heads, group,
                     a.softmax_scale * kLog2e);
  return launch_status();
}

}  // namespace pkv
