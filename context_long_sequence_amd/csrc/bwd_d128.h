// Shared declarations of the backward ring-step kernels.
#pragma once

#include "ra_device.h"
#include "ra_host.h"

#ifndef RA_DKDV_QBLOCKS
#define RA_DKDV_QBLOCKS 2  // 32-query blocks per staged query tile of the bf16 d=128 dK/dV kernel
#endif
#ifndef RA_DKDV_WAVES
#define RA_DKDV_WAVES 4  // waves (x 32 keys) per dK/dV workgroup of the bf16 d=128 path
#endif

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

constexpr int kD128 = 128;
constexpr int kD128Tile = 32;  // rows per staged tile (keys for dQ, queries for dK/dV)

// Register prefetch of one ROWS-row x 128-column bf16 tile by NT threads.
template <int NT, int ROWS = 32>
struct TileStage {
  static constexpr int kPer = ROWS * 16 / NT;  // 16-byte chunks per thread
  static_assert(kPer * NT == ROWS * 16, "tile must split evenly over the threads");
  u32x4 reg[kPer];
  // rows [row0, row0 + ROWS) of a [rows, stride] matrix, rows clamped to nrows-1
  __device__ __forceinline__ void fetch(const __bf16* base, int64_t stride, int row0, int nrows, int tid) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int u = tid + r * NT;
      const int row = min(row0 + (u >> 4), nrows - 1);
      reg[r] = *reinterpret_cast<const u32x4*>(base + (int64_t)row * stride + (u & 15) * 8);
    }
  }
  __device__ __forceinline__ void put(__bf16* tile, int tid) const {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int u = tid + r * NT;
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(tile) + tile_off(u >> 4, u & 15)) = reg[r];
    }
  }
};

// bf16, head_dim 128: dK/dV kernel (bwd_dkdv_d128.hip) then dQ kernel
// (bwd_dq_d128.hip) on `stream`.
ra_status launch_bwd_d128(BwdArgs args, hipStream_t stream);
ra_status launch_dkdv_d128(BwdArgs args, hipStream_t stream);
ra_status launch_dq_d128(BwdArgs args, hipStream_t stream);

}  // namespace ra
