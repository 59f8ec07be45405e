// lse_merge: fold one ring step's partial attention result into the running one.
//
// The ring delivers one partial (O_s, LSE_s) per KV chunk; the partials of
// disjoint key sets combine exactly by rescaling with their log-sum-exps
// (axolotl docs "Sequence Parallelism", introduction: per-chunk results are
// aggregated as they travel around the ring):
//   M = max(L, L_s), L' = M + ln(e^(L-M) + e^(L_s-M)), O' = e^(L-L') O + e^(L_s-L') O_s.
// The kernel is a single coalesced pass over O (HBM-bound): one workgroup per
// token row (b, i), whose Hq*d fp32 values are contiguous; each thread handles
// 16-byte vectors and finds its head's LSE pair in [B, Hq, Sq].
#include "ra_device.h"
#include "ra_host.h"

namespace ra {
namespace {

constexpr int kThreads = 256;

template <bool kMerge, int kOut>  // kOut: 0 = no output, 1 = f32 copy, 2 = bf16
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(int Sq, int Hq, int d4, float* __restrict__ o_acc,
                                                             float* __restrict__ lse_acc,
                                                             const float* __restrict__ o_step,
                                                             const float* __restrict__ lse_step,
                                                             void* __restrict__ o_out) {
  const int64_t row = blockIdx.x;  // b * Sq + i
  const int b = (int)(row / Sq);
  const int i = (int)(row - (int64_t)b * Sq);
  const int n4 = Hq * d4;
  const int64_t base4 = row * n4;
  f32x4* acc4 = reinterpret_cast<f32x4*>(o_acc) + base4;
  for (int t = threadIdx.x; t < n4; t += kThreads) {
    const int h = t / d4;
    f32x4 o = acc4[t];
    if constexpr (kMerge) {
      const int64_t li = ((int64_t)b * Hq + h) * Sq + i;
      const MergeWeights mw = merge_weights(lse_acc[li], lse_step[li]);
      if (mw.live) {
        o = merge_o(o, reinterpret_cast<const f32x4*>(o_step)[base4 + t], mw);
        acc4[t] = o;
      }
    }
    if constexpr (kOut == 1) {
      reinterpret_cast<f32x4*>(o_out)[base4 + t] = o;
    } else if constexpr (kOut == 2) {
      reinterpret_cast<bf16x4*>(o_out)[base4 + t] = to_bf16x4(o);
    }
  }
  if constexpr (kMerge) {
    // The merged LSE is written only after every thread of the row has read the
    // running one: a head's d/4 vectors may span two waves or two passes of the loop
    // above.
    __syncthreads();
    for (int h = threadIdx.x; h < Hq; h += kThreads) {
      const int64_t li = ((int64_t)b * Hq + h) * Sq + i;
      const MergeWeights mw = merge_weights(lse_acc[li], lse_step[li]);
      if (mw.live) lse_acc[li] = mw.lse;
    }
  }
}

template <bool kMerge>
void launch(int B, int Sq, int Hq, int d, float* o_acc, float* lse_acc, const float* o_step,
            const float* lse_step, void* o_out, int out_dtype, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)B * Sq));
  const int d4 = d / 4;
  if (o_out == nullptr)
    hipLaunchKernelGGL((lse_merge_kernel<kMerge, 0>), grid, dim3(kThreads), 0, stream, Sq, Hq, d4, o_acc,
                       lse_acc, o_step, lse_step, o_out);
  else if (out_dtype == RA_DTYPE_F32)
    hipLaunchKernelGGL((lse_merge_kernel<kMerge, 1>), grid, dim3(kThreads), 0, stream, Sq, Hq, d4, o_acc,
                       lse_acc, o_step, lse_step, o_out);
  else
    hipLaunchKernelGGL((lse_merge_kernel<kMerge, 2>), grid, dim3(kThreads), 0, stream, Sq, Hq, d4, o_acc,
                       lse_acc, o_step, lse_step, o_out);
}

}  // namespace
}  // namespace ra

extern "C" ra_status lse_merge(int32_t B, int32_t Sq, int32_t Hq, int32_t d, float* o_acc, float* lse_acc,
                               const float* o_step, const float* lse_step, void* o_out, int32_t out_dtype,
                               void* stream) {
  using namespace ra;
  if (B < 1 || Sq < 1 || Hq < 1 || d < 1)
    return fail(RA_ERR_INVALID_ARGUMENT, "batch, q_len, heads_q and head_dim must be >= 1");
  if (d % 4 != 0) return fail(RA_ERR_UNSUPPORTED, "head_dim %d is not a multiple of 4", d);
  if ((int64_t)B * Sq > INT32_MAX || (int64_t)Hq * d > INT32_MAX)
    return fail(RA_ERR_INVALID_ARGUMENT, "sizes exceed 2^31-1");
  if (!o_acc || !lse_acc) return fail(RA_ERR_INVALID_ARGUMENT, "o_acc and lse_acc must be non-NULL");
  if ((o_step == nullptr) != (lse_step == nullptr))
    return fail(RA_ERR_INVALID_ARGUMENT, "o_step and lse_step must both be NULL or both non-NULL");
  const bool merge = o_step != nullptr;
  if (!merge && o_out == nullptr)
    return fail(RA_ERR_INVALID_ARGUMENT, "nothing to do: no step to merge and no o_out");
  if (o_out && out_dtype != RA_DTYPE_F32 && out_dtype != RA_DTYPE_BF16)
    return fail(RA_ERR_UNSUPPORTED, "out_dtype %d is not supported", out_dtype);
  if (!aligned16(o_acc) || !aligned16(lse_acc) || (o_step && !aligned16(o_step)) ||
      (lse_step && !aligned16(lse_step)) || (o_out && ((uintptr_t)o_out & 7u)))
    return fail(RA_ERR_INVALID_ARGUMENT, "misaligned pointer (16 bytes; o_out 8 bytes)");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (merge)
    launch<true>(B, Sq, Hq, d, o_acc, lse_acc, o_step, lse_step, o_out, out_dtype, hs);
  else
    launch<false>(B, Sq, Hq, d, o_acc, lse_acc, o_step, lse_step, o_out, out_dtype, hs);
  return check_launch("lse_merge");
}
