// ring_recv_copy: the one-GPU stand-in for the transfer of a ring step (K/V, or a
// travelling dK/dV partial, arriving from the peer), issued on the DMA engines so
// that it does not compete for compute units with the step kernels on another
// stream (aicassindra, "Transformer math: SP math", section on context
// parallelism: K/V blocks rotate around the ring).
#include "ra_host.h"

extern "C" ra_status ring_recv_copy(void* dst, const void* src, size_t bytes, void* stream) {
  using namespace ra;
  if (bytes == 0) return ok();
  if (dst == nullptr || src == nullptr) return fail(RA_ERR_INVALID_ARGUMENT, "dst and src must be non-NULL");
  const hipError_t e =
      hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDeviceNoCU, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_HIP, "ring_recv_copy: %s", hipGetErrorString(e));
  return ok();
}
