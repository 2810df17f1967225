// Shared device helpers for the gfx950 kernels of the paged KV cache library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

#define PKV_DEVICE __device__ __forceinline__

namespace pkv {

constexpr int kBlock = PKV_BLOCK_SIZE;   // tokens per physical block
constexpr int kWave = 64;                // CDNA wavefront width

// Storage tags: the element types a cache or tensor can hold.
struct F32 { using storage = float;    static constexpr int bytes = 4; };
struct BF16 { using storage = uint16_t; static constexpr int bytes = 2; };
struct FP8 { using storage = uint8_t;  static constexpr int bytes = 1; };

// ---------------------------------------------------------------- bf16

// Exact: a bf16 is the upper half of a binary32.
PKV_DEVICE float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
PKV_DEVICE float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
PKV_DEVICE float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// binary32 -> bf16, round to nearest even; NaN stays a quiet NaN.
PKV_DEVICE uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Dot product of two bf16 pairs accumulated into fp32 (v_dot2_f32_bf16).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
PKV_DEVICE float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------- fp8 E4M3

// Two fp8 codes (bytes 0,1 or 2,3 of `packed`) -> two binary32 values, by the
// gfx950 converter (OCP E4M3).
template <bool kHigh>
PKV_DEVICE void fp8x2_to_f32(uint32_t packed, float& a, float& b) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8(packed, kHigh);
  a = v[0];
  b = v[1];
}

// Two fp8 codes -> one packed bf16 pair (exact: E4M3 values fit in bf16).
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
template <bool kHigh>
PKV_DEVICE uint32_t fp8x2_to_bf16x2(uint32_t packed) {
  auto v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, kHigh);
  return __builtin_bit_cast(uint32_t, v);
}

// binary32 -> E4M3 code: round to nearest even, saturate finite values to
// +-448, NaN -> 0x7F with the sign kept.  Written from the format definition
// with integer arithmetic so the result does not depend on a hardware mode.
PKV_DEVICE uint8_t f32_to_e4m3(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return uint8_t(sign | 0x7fu);       // NaN
  if (a > 0x43e00000u) return uint8_t(sign | 0x7eu);       // |f| > 448
  const int e = int(a >> 23) - 127;
  if (e >= -6) {                                           // normal E4M3
    uint32_t m = a & 0x7fffffu;
    uint32_t q = m >> 20;                                  // 3 kept bits
    const uint32_t rest = m & 0xfffffu;
    if (rest > 0x80000u || (rest == 0x80000u && (q & 1u))) q += 1;
    uint32_t ef = uint32_t(e + 7);
    if (q == 8) { q = 0; ef += 1; }
    return uint8_t(sign | (ef << 3) | q);                  // <= 448 by the test above
  }
  // subnormal range: units of 2^-9, scaling by 2^9 is exact
  const float t = __uint_as_float(a) * 512.0f;
  const uint32_t q = uint32_t(__builtin_rintf(t));         // nearest even
  return uint8_t(sign | q);                                // q == 8 is 2^-6 exactly
}

// ---------------------------------------------------------------- lanes

PKV_DEVICE int lane_id() { return __lane_id(); }

// DPP lane exchange inside groups of four lanes.
template <int kPerm>
PKV_DEVICE float quad_perm(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kPerm, 0xf, 0xf, true));
}
constexpr int kQuadSwap1 = 0xB1;  // [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // [2,3,0,1]

// Value of lane 7-i inside each group of eight lanes (DPP row_half_mirror).
PKV_DEVICE float half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, true));
}

// Sum over the four lanes of each quad; every lane of the quad gets it.
PKV_DEVICE float quad_sum(float v) {
  v += quad_perm<kQuadSwap1>(v);
  v += quad_perm<kQuadSwap2>(v);
  return v;
}

PKV_DEVICE float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

PKV_DEVICE float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

PKV_DEVICE float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += shfl_xor(v, m);
  return v;
}

// A wave-uniform read of read-only memory through the constant address
// space, which keeps it on the scalar unit (s_load) wherever it appears.
typedef __attribute__((address_space(4))) const int32_t const_i32_t;
PKV_DEVICE int32_t load_scalar(const int32_t* p, int64_t i) {
  return ((const_i32_t*)p)[i];
}

// Sum of v over the lanes below this one.  An inclusive scan by DPP moves
// (no LDS round trips): within each row of 16 lanes, shifts by 1, 2, 4 and 8
// (lanes shifted in from outside the row add 0); then the last lane of row 0
// is added to row 1 and that of row 2 to row 3 (row_bcast:15), and lane 31
// to rows 2 and 3 (row_bcast:31).
PKV_DEVICE int wave_exclusive_sum(int v) {
  int x = v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x - v;
}

PKV_DEVICE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global accesses.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
PKV_DEVICE u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
PKV_DEVICE void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Buffer resource over `bytes` bytes at `base` (raw buffer, 32-bit format
// field as the gfx9 family expects); loads past `bytes` return zeros.
constexpr int kRawBufferFlags = 0x00020000;
PKV_DEVICE __amdgpu_buffer_rsrc_t tile_resource(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRawBufferFlags);
}
// K/V tiles are read once per step: non-temporal loads (cache policy "nt")
// keep them from displacing reused data and stream measurably faster.
#ifndef PKV_TILE_LOAD_AUX
#define PKV_TILE_LOAD_AUX 2
#endif
PKV_DEVICE u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  return __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, PKV_TILE_LOAD_AUX));
}
// The same with a constant part of the offset in the scalar offset field, so
// that one per-lane offset register serves every piece of a tile.
PKV_DEVICE u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t offset, int scalar_offset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       r, offset, scalar_offset, PKV_TILE_LOAD_AUX));
}
// The same with the default cache policy, for data that other workgroups reuse.
PKV_DEVICE u32x4 buffer_load16_cached(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0));
}

}  // namespace pkv
