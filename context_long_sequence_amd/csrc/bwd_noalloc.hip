// ring_attn_bwd_step_noalloc: the backward ring step for callers that cannot
// allocate device memory -- code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc.  Same kernels and the same results as
// ring_attn_bwd_step.  The scratch of the split dK/dV kernel is this file's static
// device array (kDkdvScratchBytes per GPU, held until the process ends) instead of
// library-allocated memory, and both kernels of a step run on the caller's stream
// (no side stream is created).
#include <mutex>

#include "bwd_d128.h"

namespace ra {
namespace {

// Arrival counters, then partial sums (layout of kDkdvScratchBytes in bwd_d128.h).
// Host code never uses this name as an address: the device copy's address comes
// from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kDkdvScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

ra_status scratch_address(void*& out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(RA_ERR_HIP, "ring_attn_bwd_step_noalloc: no current device");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(RA_ERR_HIP, "ring_attn_bwd_step_noalloc: hipGetSymbolAddress of the scratch failed: %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  out = g_scratch_ptr[dev];
  return RA_OK;
}

}  // namespace
}  // namespace ra

extern "C" ra_status ring_attn_bwd_step_noalloc(const ra_shape* s, const void* q, const void* k, const void* v,
                                                const void* d_o, const float* lse, const float* delta,
                                                const int32_t* seg_ids, int64_t seg_len, float* dq_acc,
                                                float* dk_acc, float* dv_acc, void* stream) {
  void* p = nullptr;
  const ra_status st = ra::scratch_address(p);
  if (st != RA_OK) return st;
  return ra::bwd_step_entry(s, q, k, v, d_o, lse, delta, seg_ids, seg_len, dq_acc, dk_acc, dv_acc, stream, p,
                            /*allocate=*/false, /*side=*/false);
}
