// Host-side helpers shared by the C ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Status of the launch just issued on this thread.
inline pkv_status launch_status() {
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

inline int32_t dtype_bytes(pkv_dtype t) {
  switch (t) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

}  // namespace pkv
