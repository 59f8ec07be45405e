// segment_mask_from_pos: sample id of every token of a packed row.
//
// With packing, several samples share one row and each sample's position ids
// restart at 0; under context parallelism a chunk may begin in the middle of a
// sample, so the sample index is taken from a cumulative sum over the GLOBAL row
// (axolotl docs "Sequence Parallelism", section Mamba/SSM Hybrid Models, item on
// seq_idx; section Sample Packing with Sequence Parallelism):
//   seg[b, t] = #{t' <= t : pos[b, t'] == 0} - 1.
// One workgroup scans one row in blocks of 4096 tokens with a running carry.
#include "ra_device.h"
#include "ra_host.h"

namespace ra {
namespace {

constexpr int kThreads = 1024;
constexpr int kPer = 4;

__global__ __launch_bounds__(kThreads) void segment_kernel(int S, const int32_t* __restrict__ pos,
                                                           int32_t* __restrict__ seg) {
  __shared__ int wave_tot[kThreads / 64];
  __shared__ int wave_pre[kThreads / 64];
  const int b = blockIdx.x;
  const int32_t* prow = pos + (int64_t)b * S;
  int32_t* srow = seg + (int64_t)b * S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  // 64-bit token indices: base + kThreads * kPer may pass 2^31 - 1 near the S limit.
  for (int64_t base = 0; base < S; base += kThreads * kPer) {
    int c[kPer];
    int run = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int64_t t = base + tid * kPer + e;
      run += (t < S && prow[t] == 0) ? 1 : 0;
      c[e] = run;
    }
    // inclusive scan of `run` over the wave
    int x = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int w = lane < kThreads / 64 ? wave_tot[lane] : 0;
      int incl = w;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (lane < kThreads / 64) wave_pre[lane] = incl - w;
    }
    __syncthreads();
    const int before = carry + wave_pre[wave] + (x - run);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int64_t t = base + tid * kPer + e;
      if (t < S) srow[t] = before + c[e] - 1;
    }
    carry += wave_pre[kThreads / 64 - 1] + wave_tot[kThreads / 64 - 1];
    __syncthreads();
  }
}

}  // namespace
}  // namespace ra

extern "C" ra_status segment_mask_from_pos(int32_t B, int64_t S, const int32_t* position_ids, int32_t* seg_ids,
                                           void* stream) {
  using namespace ra;
  if (B < 1 || S < 1) return fail(RA_ERR_INVALID_ARGUMENT, "batch and seq_len must be >= 1");
  if (S > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "seq_len exceeds 2^31-1");
  if (!position_ids || !seg_ids) return fail(RA_ERR_INVALID_ARGUMENT, "position_ids and seg_ids must be non-NULL");
  if (((uintptr_t)position_ids & 3u) || ((uintptr_t)seg_ids & 3u))
    return fail(RA_ERR_INVALID_ARGUMENT, "position_ids and seg_ids must be 4-byte aligned");
  hipLaunchKernelGGL(segment_kernel, dim3((unsigned)B), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     (int)S, position_ids, seg_ids);
  return check_launch("segment_mask_from_pos");
}
