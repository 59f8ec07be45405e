// Status strings, the thread-local last-error message and shared argument checks.
#include <stdarg.h>
#include <stdio.h>

#include "ra_host.h"

namespace ra {

static thread_local char g_last_error[512] = "";

ra_status fail(ra_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

ra_status ok() {
  g_last_error[0] = '\0';
  return RA_OK;
}

ra_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

ra_status validate_step(const ra_shape* s, const int32_t* seg_ids, int64_t seg_len) {
  if (s == nullptr) return fail(RA_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->batch < 1 || s->q_len < 1 || s->kv_len < 1)
    return fail(RA_ERR_INVALID_ARGUMENT, "batch, q_len and kv_len must be >= 1 (got %d, %d, %d)",
                s->batch, s->q_len, s->kv_len);
  // Tile arithmetic inside the kernels is 32-bit, and per-lane byte offsets within
  // a tile of rows are 32-bit.
  if (s->q_len > (1 << 30) || s->kv_len > (1 << 30))
    return fail(RA_ERR_INVALID_ARGUMENT, "q_len and kv_len must be <= 2^30 (got %d, %d)", s->q_len, s->kv_len);
  if (s->heads_q > 4096) return fail(RA_ERR_INVALID_ARGUMENT, "heads_q must be <= 4096 (got %d)", s->heads_q);
  if (s->heads_q < 1 || s->heads_kv < 1 || s->heads_q % s->heads_kv != 0)
    return fail(RA_ERR_INVALID_ARGUMENT, "heads_q (%d) must be a positive multiple of heads_kv (%d)",
                s->heads_q, s->heads_kv);
  if (s->q_offset < 0 || s->kv_offset < 0)
    return fail(RA_ERR_INVALID_ARGUMENT, "q_offset and kv_offset must be >= 0");
  if (s->causal != 0 && s->causal != 1) return fail(RA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (!(s->softmax_scale > 0.0f) || s->softmax_scale > 1e30f)
    return fail(RA_ERR_INVALID_ARGUMENT, "softmax_scale must be a positive finite number");
  if (s->dtype != RA_DTYPE_F32 && s->dtype != RA_DTYPE_BF16)
    return fail(RA_ERR_UNSUPPORTED, "dtype %d is not supported (f32=0, bf16=1)", s->dtype);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", s->head_dim);
  // Index arithmetic inside the kernels is 64-bit for element offsets; row counts stay 32-bit.
  if ((int64_t)s->batch * s->q_len * s->heads_q > INT32_MAX ||
      (int64_t)s->batch * s->kv_len * s->heads_kv > INT32_MAX)
    return fail(RA_ERR_INVALID_ARGUMENT, "batch*len*heads exceeds 2^31-1 rows");
  if (seg_ids != nullptr) {
    if (seg_len < 1) return fail(RA_ERR_INVALID_ARGUMENT, "seg_len must be >= 1 when seg_ids is given");
    if (s->q_offset + s->q_len > seg_len || s->kv_offset + s->kv_len > seg_len)
      return fail(RA_ERR_INVALID_ARGUMENT,
                  "segment range past seg_len (q_offset+q_len=%lld, kv_offset+kv_len=%lld, seg_len=%lld)",
                  (long long)(s->q_offset + s->q_len), (long long)(s->kv_offset + s->kv_len),
                  (long long)seg_len);
    if (!aligned16(seg_ids)) return fail(RA_ERR_INVALID_ARGUMENT, "seg_ids must be 16-byte aligned");
  }
  return RA_OK;
}

}  // namespace ra

extern "C" const char* ra_status_string(ra_status st) {
  switch (st) {
    case RA_OK: return "RA_OK";
    case RA_ERR_INVALID_ARGUMENT: return "RA_ERR_INVALID_ARGUMENT";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_HIP: return "RA_ERR_HIP";
  }
  return "RA_UNKNOWN_STATUS";
}

extern "C" const char* ra_last_error(void) { return ra::g_last_error; }

extern "C" int32_t ra_abi_version(void) { return 3; }
