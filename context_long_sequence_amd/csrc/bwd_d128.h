// Shared declarations of the backward ring-step kernels.
#pragma once

#include "ra_device.h"
#include "ra_host.h"

namespace ra {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  const float* lse;
  const float* delta;
  const int32_t* seg;
  int64_t seg_len;
  float* dq;
  float* dk;
  float* dv;
  int B, Sq, Sk, Hq, Hkv;
  int64_t q_offset, kv_offset;
  int causal;
  float scale;
  float scale_log2;
  int n_tiles;  // key tiles per (b, kv head) for dkdv; query tiles per (b, q head) for dq
  // Split dK/dV (32-key kernel): up to n_split workgroups share one key block's query
  // tiles; their fp32 partial sums go to `part` and the last of them to finish (by
  // the per-block arrival counter in `count`, zero at launch) adds them up in split
  // order.  n_split = 1: no scratch, each workgroup updates dK/dV itself.
  float* part;
  int* count;
  int n_split;
};

// Scratch of the split dK/dV kernel: kDkdvCounters arrival counters, then
// kDkdvPartBytes of partial sums (128 keys x 128 columns x dK and dV, fp32, per
// workgroup: kDkdvPartPerWg bytes).
constexpr int kDkdvCounters = 65536;
constexpr size_t kDkdvCountBytes = sizeof(int) * (size_t)kDkdvCounters;
constexpr size_t kDkdvPartPerWg = 2 * 128 * 128 * sizeof(float);
constexpr size_t kDkdvPartBytes = (size_t)64 << 20;
constexpr size_t kDkdvScratchBytes = kDkdvCountBytes + kDkdvPartBytes;

constexpr int kD128 = 128;
constexpr int kD128Tile = 32;  // keys per staged tile of the dQ kernel

// bf16, head_dim 128: dK/dV kernel (bwd_dkdv_d128.hip) on `stream` and dQ kernel
// (bwd_dq_d128.hip) on the device's side stream (`side`), or both on `stream`.
// `scratch` (kDkdvScratchBytes, device memory) is used when the 32-key dK/dV kernel
// splits its key blocks; bwd_d128_needs_scratch tells whether this step does.
ra_status launch_bwd_d128(BwdArgs args, hipStream_t stream, void* scratch, bool side);
bool bwd_d128_needs_scratch(const BwdArgs& args);
ra_status launch_dkdv_d128(BwdArgs args, hipStream_t stream, void* scratch);
int dkdv_d128_split(const BwdArgs& args);

// The backward step behind the C entry points (bwd_step.hip): checks, then the
// kernels.  scratch: device memory of kDkdvScratchBytes or null; when a split step
// needs scratch and none is given, `allocate` lets it take the device's
// library-allocated scratch (else the step fails).  side: run dQ on the side stream.
ra_status bwd_step_entry(const ra_shape* s, const void* q, const void* k, const void* v, const void* d_o,
                         const float* lse, const float* delta, const int32_t* seg_ids, int64_t seg_len,
                         float* dq_acc, float* dk_acc, float* dv_acc, void* stream, void* scratch, bool allocate,
                         bool side);
// dK/dV with 64 keys per wave (bwd_dkdv64_d128.hip) and its grid size.
ra_status launch_dkdv64_d128(BwdArgs args, hipStream_t stream);
int64_t dkdv64_d128_workgroups(const BwdArgs& args);
// dQ with 64 queries per wave (bwd_dq64_d128.hip) and its grid size.
ra_status launch_dq64_d128(BwdArgs args, hipStream_t stream);
int64_t dq64_d128_workgroups(const BwdArgs& args);
ra_status launch_dq_d128(BwdArgs args, hipStream_t stream);

}  // namespace ra
