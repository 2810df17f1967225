// Library-wide entry points: block size, status strings, KV sizing.

#include "abi_util.h"

extern "C" int32_t pkv_block_size(void) { return PKV_BLOCK_SIZE; }

extern "C" const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case PKV_ERR_SHAPE: return "inconsistent or negative sizes";
    case PKV_ERR_UNSUPPORTED: return "unsupported head_dim, dtype or group size";
    case PKV_ERR_WORKSPACE: return "decode workspace missing or too small";
    case PKV_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case PKV_ERR_NO_BLOCKS: return "too few free blocks";
    case PKV_ERR_REQUEST: return "unknown or duplicate request";
    default: return "unknown status";
  }
}

// Per-token KV bytes: key and value, per layer, per kv head, per element.
extern "C" int64_t kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t bytes_per_elem) {
  if (num_layers < 0 || num_kv_heads < 0 || head_dim < 0 || bytes_per_elem < 0)
    return -1;
  int64_t r = 2;
  for (const int32_t f : {bytes_per_elem, num_layers, num_kv_heads, head_dim})
    if (__builtin_mul_overflow(r, int64_t(f), &r)) return -1;
  return r;
}
