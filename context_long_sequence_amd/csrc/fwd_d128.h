// Shared by the forward-step kernels: the launch arguments, the per-row epilogue
// (store, or merge into the running result) and the wide bf16 head_dim-128 kernel's
// entry points.
#pragma once

#include "ra_device.h"
#include "ra_host.h"

namespace ra {

constexpr float kFwdSlack = 8.0f;  // lazy-rescale threshold (log2 units)

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seg;  // [B, seg_len] or null
  int64_t seg_len;
  float* o;
  float* lse;
  int B, Sq, Sk, Hq, Hkv;
  int64_t q_offset, kv_offset;
  int causal;
  float scale_log2;  // softmax_scale * log2(e)
  int n_qtiles;
  // Fused merge (ring_attn_fwd_step_merge): o and lse hold the running result and
  // receive the merged one; o_out (optional) the merged O converted to out_kind
  // (1 = fp32, 2 = bf16).
  int merge;
  void* o_out;
  int out_kind;
};

// Epilogue of one query row held by this lane (both half-waves of the row call it):
// the step's O = acc * inv in the vectors at columns 32*db + 8*r4 + 4*half, and its
// LSE ls.  Stored as is, or merged into the running (o, lse) with the merge rule of
// lse_merge (same functions, same bits) and optionally converted into o_out.  All
// loads of the running row precede the stores (the pointers are restrict).
template <int DB>
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& a, const f32x16 (&oacc)[DB], float inv, float ls,
                                             int b, int hq, int qi, int half) {
  constexpr int D = 32 * DB;
  const int64_t row = ((int64_t)b * a.Sq + qi) * ((int64_t)a.Hq * D) + (int64_t)hq * D;
  const int64_t li = ((int64_t)b * a.Hq + hq) * a.Sq + qi;
  float* __restrict__ orow = a.o + row;
  f32x4 os[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      os[db][r4] = f32x4{oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv, oacc[db][4 * r4 + 2] * inv,
                         oacc[db][4 * r4 + 3] * inv};
  if (!a.merge) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * r4 + 4 * half) = os[db][r4];
    if (half == 0) a.lse[li] = ls;
    return;
  }
  const MergeWeights mw = merge_weights(a.lse[li], ls);
  // A row this step adds nothing to (weight 0: merge_o returns the running O and the
  // merged LSE equals the running one, bit for bit) is left as it is: only read, and
  // only when it is also converted.
  const bool changed = mw.live && mw.ws != 0.0f;
  if (!changed && a.out_kind == 0) return;
  f32x4 o[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) o[db][r4] = *reinterpret_cast<const f32x4*>(orow + 32 * db + 8 * r4 + 4 * half);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int c = 32 * db + 8 * r4 + 4 * half;
      if (changed) {
        o[db][r4] = merge_o(o[db][r4], os[db][r4], mw);
        *reinterpret_cast<f32x4*>(orow + c) = o[db][r4];
      }
      if (a.out_kind == 1)
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.o_out) + row + c) = o[db][r4];
      else if (a.out_kind == 2)
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.o_out) + row + c) = to_bf16x4(o[db][r4]);
    }
  if (half == 0 && changed) a.lse[li] = mw.lse;
}

// bf16, head_dim 128, 64 queries per wave (fwd64_d128.hip): grid size and launch.
int64_t fwd64_d128_workgroups(const FwdArgs& args);
ra_status launch_fwd64_d128(FwdArgs args, hipStream_t stream);

}  // namespace ra
