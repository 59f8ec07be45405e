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
};

constexpr int kD128 = 128;
constexpr int kD128Tile = 32;  // keys per staged tile of the dQ kernel

// bf16, head_dim 128: dK/dV kernel (bwd_dkdv_d128.hip) then dQ kernel
// (bwd_dq_d128.hip) on `stream`.
ra_status launch_bwd_d128(BwdArgs args, hipStream_t stream);
ra_status launch_dkdv_d128(BwdArgs args, hipStream_t stream);
// dK/dV with 64 keys per wave (bwd_dkdv64_d128.hip) and its grid size.
ra_status launch_dkdv64_d128(BwdArgs args, hipStream_t stream);
int64_t dkdv64_d128_workgroups(const BwdArgs& args);
// dQ with 64 queries per wave (bwd_dq64_d128.hip) and its grid size.
ra_status launch_dq64_d128(BwdArgs args, hipStream_t stream);
int64_t dq64_d128_workgroups(const BwdArgs& args);
ra_status launch_dq_d128(BwdArgs args, hipStream_t stream);

}  // namespace ra
