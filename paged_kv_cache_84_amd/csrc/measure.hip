// Hardware ceilings for reading the hot path's rates: a streaming HBM read
// with the decode's 16-byte non-temporal loads, a register-only loop of the
// prefill's bf16 MFMA, and the same loop with the softmax's vector work
// issued by the same waves.  Each leaves a result the caller can check, so
// that the compiler cannot have dropped the work being timed.

#include "abi_util.h"
#include "common.h"
#include "pagedkv_measure.h"

namespace pkv {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;          // 16-byte loads in flight per thread
constexpr int kReadWgsPerCu = 4;
constexpr int kNumCus = 256;            // MI355X compute units

__global__ void clear_word_kernel(uint32_t* w) { *w = 0u; }

// Workgroup g reads the contiguous range of 16-byte pieces
// [g * per, (g + 1) * per), its threads striding by the workgroup size,
// kReadUnroll loads at a time (contiguous ranges per workgroup keep DRAM
// pages open: measured ~7.1-7.25 TB/s on MI355X against 5.8-7.2 TB/s for a
// grid-wide stride).  The workgroup folds its lanes and adds its word to
// the checksum with one atomic XOR.
__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(
    const u32x4* __restrict__ buf, int64_t pieces, uint32_t* __restrict__ checksum) {
  __shared__ uint32_t part[kReadThreads / kWave];
  const int64_t per = (pieces + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = int64_t(blockIdx.x) * per;
  const int64_t b1 = b0 + per < pieces ? b0 + per : pieces;
  int64_t i = b0 + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (kReadUnroll - 1) * kReadThreads < b1; i += kReadUnroll * kReadThreads) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * kReadThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < b1; i += kReadThreads) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) acc ^= uint32_t(__shfl_xor(int(acc), o, kWave));
  if (lane_id() == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = 0u;
#pragma unroll
    for (int k = 0; k < kReadThreads / kWave; ++k) w ^= part[k];
    __hip_atomic_fetch_xor(checksum, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaWavesPerWg = 8;
constexpr int kMfmaChains = 8;          // independent accumulators per wave
constexpr int kVecChains = 5;           // vector chains beside them

__global__ __launch_bounds__(kMfmaWavesPerWg * kWave) void mfma_bf16_kernel(
    int32_t iterations, float* __restrict__ result) {
  const int lane = lane_id();
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)float(lane % 16 + 1);
    b[e] = (__bf16)1.0f;
  }
  f32x4_t c[kMfmaChains];
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < iterations; ++r) {
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
  }
  // every chain feeds the stored value's condition, so none can be dropped
  float others = 0.f;
#pragma unroll
  for (int j = 1; j < kMfmaChains; ++j) others += c[j][0] + c[j][3];
  const int wave = int(blockIdx.x) * kMfmaWavesPerWg + int(threadIdx.x) / kWave;
  if (lane == 0) result[wave] = others >= 0.f ? c[0][0] : -1.f;
}

// The prefill's mix of work: bf16 MFMAs and the softmax's vector
// instructions (fp32 fma and add, a transcendental 2^x, integer ops of the
// bf16 split), both from the same waves.  Mode 0 issues only the MFMAs, 1
// only the vector work, 2 both, interleaved in one loop: per iteration 8
// MFMAs and 5 chains x (fma, and, sub, add) plus 2 x (sub, exp2), i.e. 3
// vector instructions and 0.25 exp2 per MFMA (the prefill tile issues 2.8
// and 0.33).  Lane 0 of each wave stores
// result[2w] = element (0, 0) of its first accumulator (32 * iterations when
// the MFMAs ran, else 0) and result[2w + 1] = its vector chains' sum (equal
// in every wave, 0 when the vector work did not run).
template <int MODE>
__global__ __launch_bounds__(kMfmaWavesPerWg * kWave) void mfma_valu_kernel(
    int32_t iterations, float* __restrict__ result) {
  const int lane = lane_id();
  constexpr bool do_m = MODE != 1, do_v = MODE != 0;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)float(lane % 16 + 1);
    b[e] = (__bf16)1.0f;
  }
  f32x4_t c[kMfmaChains];
  float x[kVecChains], y[kVecChains];
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kVecChains; ++j) {
    x[j] = 0.125f * float(j);
    y[j] = 0.f;
  }
  for (int r = 0; r < iterations; ++r) {
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) {
      if constexpr (do_m) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
      if constexpr (do_v) if (j < kVecChains) {
        // x contracts toward 0.5 and stays in [0, 1); p = 2^(x - 1) on some
        x[j] = __builtin_fmaf(x[j], 0.5f, 0.25f);
        float p = x[j];
        if (j % 3 == 0) p = __builtin_amdgcn_exp2f(x[j] - 1.0f);
        const float hi = __uint_as_float(__float_as_uint(p) & 0xffff0000u);
        y[j] += p - hi;
      }
    }
  }
  float others = 0.f, v = 0.f;
#pragma unroll
  for (int j = 1; j < kMfmaChains; ++j) others += c[j][0] + c[j][3];
#pragma unroll
  for (int j = 0; j < kVecChains; ++j) v += y[j];
  const int wave = int(blockIdx.x) * kMfmaWavesPerWg + int(threadIdx.x) / kWave;
  if (lane == 0) {
    result[2 * wave] = others >= 0.f ? c[0][0] : -1.f;
    result[2 * wave + 1] = v;
  }
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_measure_hbm_read(const void* buf, int64_t bytes, uint32_t* checksum,
                                           void* stream) {
  if (bytes <= 0 || bytes % 16 != 0 || bytes >= (int64_t(1) << 40)) return PKV_ERR_SHAPE;
  if (!buf || !checksum) return PKV_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(checksum, 4)) return PKV_ERR_ALIGN;
  hipStream_t st = as_stream(stream);
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, st, checksum);
  if (launch_status() != PKV_OK) return PKV_ERR_LAUNCH;
  const int64_t pieces = bytes / 16;
  const int64_t wgs_needed = (pieces + kReadThreads - 1) / kReadThreads;
  const int wgs = int(std::min<int64_t>(int64_t(kNumCus) * kReadWgsPerCu, wgs_needed));
  hipLaunchKernelGGL(hbm_read_kernel, dim3(wgs), dim3(kReadThreads), 0, st,
                     static_cast<const u32x4*>(buf), pieces, checksum);
  return launch_status();
}

extern "C" pkv_status pkv_measure_mfma_bf16(int32_t iterations, int32_t waves, float* result,
                                            void* stream) {
  if (iterations < 1 || iterations > 524288 || waves < kMfmaWavesPerWg ||
      waves % kMfmaWavesPerWg != 0)
    return PKV_ERR_SHAPE;
  if (!result) return PKV_ERR_NULL;
  if (!aligned(result, 4)) return PKV_ERR_ALIGN;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(waves / kMfmaWavesPerWg),
                     dim3(kMfmaWavesPerWg * kWave), 0, as_stream(stream), iterations, result);
  return launch_status();
}

extern "C" pkv_status pkv_measure_mfma_valu(int32_t iterations, int32_t waves, int32_t mode,
                                            float* result, void* stream) {
  if (iterations < 1 || iterations > 524288 || waves < kMfmaWavesPerWg ||
      waves % kMfmaWavesPerWg != 0 || mode < 0 || mode > 2)
    return PKV_ERR_SHAPE;
  if (!result) return PKV_ERR_NULL;
  if (!aligned(result, 4)) return PKV_ERR_ALIGN;
  auto kernel = mode == 0 ? mfma_valu_kernel<0> : mode == 1 ? mfma_valu_kernel<1>
                                                            : mfma_valu_kernel<2>;
  hipLaunchKernelGGL(kernel, dim3(waves / kMfmaWavesPerWg), dim3(kMfmaWavesPerWg * kWave), 0,
                     as_stream(stream), iterations, result);
  return launch_status();
}
