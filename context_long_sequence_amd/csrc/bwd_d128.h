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

// Contiguous range [begin, end) of tiles (of `tile` items over `n` items of the
// row starting at `row`) whose segment-id range meets [lo, hi].  Segment ids are
// nondecreasing along the row, so the live tiles are contiguous.  Wave-uniform.
__device__ __forceinline__ void seg_tile_range(const int32_t* row, int n, int tile, int t_begin, int t_end,
                                               int lo, int hi, int& out_begin, int& out_end) {
  const int lane = threadIdx.x & 63;
  int first = t_end, last = -1;
  for (int base = t_begin; base < t_end; base += 64) {
    const int t = base + lane;
    bool live = false;
    if (t < t_end) {
      const int a = t * tile;
      const int z = min((t + 1) * tile, n) - 1;
      live = row[z] >= lo && row[a] <= hi;
    }
    const uint64_t mask = __ballot(live);
    if (mask) {
      first = min(first, base + (int)__builtin_ctzll(mask));
      last = max(last, base + 63 - (int)__builtin_clzll(mask));
    }
  }
  out_begin = first;
  out_end = last + 1;
}

// Token span [lo, hi) of segment `s` in a row of `n` nondecreasing segment ids:
// lo = first index with id >= s, hi = first index with id > s (binary searches).
// With ids that decrease somewhere the span is some range inside [0, n] (never an
// access outside the row).
__device__ __forceinline__ void seg_span(const int32_t* row, int64_t n, int s, int64_t& lo, int64_t& hi) {
  int64_t a = 0, b = n;
  while (a < b) {
    const int64_t m = (a + b) >> 1;
    if (row[m] < s)
      a = m + 1;
    else
      b = m;
  }
  lo = a;
  b = n;
  while (a < b) {
    const int64_t m = (a + b) >> 1;
    if (row[m] <= s)
      a = m + 1;
    else
      b = m;
  }
  hi = a;
}

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
