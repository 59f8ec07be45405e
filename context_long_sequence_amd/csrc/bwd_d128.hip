// Backward ring step for the hot shape (bf16, head_dim 128).  Same arithmetic as
// the generic kernels in bwd_step.hip (probabilities recomputed from the final
// log-sum-exp; archcrux, "sequence-parallel long-context attention OOM"), laid
// out for gfx950:
//  * Q, dO, K, V tiles live in LDS row-major with the 16-byte-chunk XOR swizzle
//    of ra_device.h, filled from registers prefetched one tile ahead, double
//    buffered (one barrier per tile).
//  * Operands that need the other orientation (K^T for dQ, Q^T and dO^T for
//    dK/dV) come from transposing LDS reads of the same tiles, so nothing is
//    stored twice.
#include "bwd_d128.h"

namespace ra {
namespace {

constexpr int kD = 128;
constexpr int kTile = 32;  // rows per staged tile (keys for dQ, queries for dK/dV)

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

// ------------------------------------------------------------------------------------
// dQ: 4 waves x 32 queries of one query head; walks the key tiles of the chunk.
// ------------------------------------------------------------------------------------
constexpr int kDqWaves = 4;
constexpr int kDqThreads = 64 * kDqWaves;

template <bool kSeg>
__global__ __launch_bounds__(kDqThreads) void dq_d128_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) __bf16 kbuf[2][kTile * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 vbuf[2][kTile * kD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int group = a.Hq / a.Hkv;
  int rem = logical;
  const int qt_rev = rem % a.n_tiles;
  rem /= a.n_tiles;
  const int hg = rem % group;
  rem /= group;
  const int g = rem % a.Hkv;
  const int b = rem / a.Hkv;
  const int qt = a.n_tiles - 1 - qt_rev;
  const int hq = g * group + hg;

  constexpr int BM = 32 * kDqWaves;
  const int q0 = qt * BM;
  const int q_last = min(q0 + BM, a.Sq) - 1;
  const int qw = q0 + 32 * wave;
  const int qi = qw + col;
  const bool q_valid = qi < a.Sq;
  const int64_t qg = a.q_offset + qi;

  const int64_t q_rs = (int64_t)a.Hq * kD, kv_rs = (int64_t)a.Hkv * kD;
  const __bf16* kbase = static_cast<const __bf16*>(a.k) + (int64_t)b * a.Sk * kv_rs + (int64_t)g * kD;
  const __bf16* vbase = static_cast<const __bf16*>(a.v) + (int64_t)b * a.Sk * kv_rs + (int64_t)g * kD;

  int n_keys = a.Sk;
  if (a.causal) {
    const int64_t last_visible = a.q_offset + q_last - a.kv_offset;
    n_keys = (int)max<int64_t>(0, min<int64_t>((int64_t)a.Sk, last_visible + 1));
  }
  int kt_begin = 0, kt_end = (n_keys + kTile - 1) / kTile;
  int seg_q = 0;
  const int32_t* seg_row = nullptr;
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    const int lo = seg_row[a.q_offset + q0], hi = seg_row[a.q_offset + q_last];
    seg_q = q_valid ? seg_row[a.q_offset + qi] : lo;
    int sb, se;
    seg_tile_range(seg_row + a.kv_offset, a.Sk, kTile, 0, kt_end, lo, hi, sb, se);
    kt_begin = sb;
    kt_end = max(sb, se);
  }

  bf16x8 qf[8], dof[8];
  {
    const int64_t off = ((int64_t)b * a.Sq + (q_valid ? qi : 0)) * q_rs + (int64_t)hq * kD + 8 * half;
    const __bf16* qp = static_cast<const __bf16*>(a.q) + off;
    const __bf16* dp = static_cast<const __bf16*>(a.d_o) + off;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qf[s] = q_valid ? load_bf16x8(qp + 16 * s) : bf16x8{};
      dof[s] = q_valid ? load_bf16x8(dp + 16 * s) : bf16x8{};
    }
  }
  const int64_t li = ((int64_t)b * a.Hq + hq) * a.Sq + (q_valid ? qi : 0);
  const float lse_q = q_valid ? a.lse[li] : -INFINITY;
  const float neg_lse2 = lse_q == -INFINITY ? -INFINITY : -lse_q * kLog2e;
  const float dl = q_valid ? a.delta[li] : 0.0f;

  f32x16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dq[db] = f32x16{};

  TileStage<kDqThreads> ks, vs;
  if (kt_begin < kt_end) {
    ks.fetch(kbase, kv_rs, kt_begin * kTile, a.Sk, tid);
    vs.fetch(vbase, kv_rs, kt_begin * kTile, a.Sk, tid);
    ks.put(kbuf[0], tid);
    vs.put(vbuf[0], tid);
  }
  for (int t = kt_begin; t < kt_end; ++t) {
    const int cur = (t - kt_begin) & 1;
    __syncthreads();  // tile t visible; every wave is done with tile t-1
    const bool more = t + 1 < kt_end;
    if (more) {
      ks.fetch(kbase, kv_rs, (t + 1) * kTile, a.Sk, tid);
      vs.fetch(vbase, kv_rs, (t + 1) * kTile, a.Sk, tid);
    }
    const __bf16* kt_ = kbuf[cur];
    const __bf16* vt_ = vbuf[cur];
    const int k0 = t * kTile;
    bool partial = (k0 + kTile > a.Sk) || (qw + 32 > a.Sq);  // wave-uniform
    if (a.causal) partial |= (a.kv_offset + k0 + kTile - 1 > a.q_offset + qw);
    if constexpr (kSeg) partial = true;

    // S^T = K Q^T and dP^T = V dO^T; register i of half h = key k0 + 16h + i.
    f32x16 st = f32x16{}, dpt = f32x16{};
    {
      const int row = key_of_row(col);
      bf16x8 f[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) f[s] = read_chunk(kt_, row, 2 * s + half);
#pragma unroll
      for (int s = 0; s < 8; ++s) st = mfma_bf16(f[s], qf[s], st);
#pragma unroll
      for (int s = 0; s < 8; ++s) f[s] = read_chunk(vt_, row, 2 * s + half);
#pragma unroll
      for (int s = 0; s < 8; ++s) dpt = mfma_bf16(f[s], dof[s], dpt);
    }
    float p[16], ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = exp2_fast(__builtin_fmaf(st[i], a.scale_log2, neg_lse2));
    if (partial) {  // one wave-uniform branch around the element mask
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = k0 + 16 * half + i;
        bool vis = q_valid && kj < a.Sk;
        if (a.causal) vis = vis && (a.kv_offset + kj <= qg);
        if constexpr (kSeg) vis = vis && (kj < a.Sk ? seg_row[a.kv_offset + kj] == seg_q : false);
        p[i] = vis ? p[i] : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) ds[i] = p[i] * (dpt[i] - dl);
    // dQ^T += K^T dS^T: K^T rows (keys 16h + 8m + j) by transposing reads of the K tile.
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const bf16x8 sf = to_bf16x8(ds[8 * m], ds[8 * m + 1], ds[8 * m + 2], ds[8 * m + 3], ds[8 * m + 4],
                                  ds[8 * m + 5], ds[8 * m + 6], ds[8 * m + 7]);
      bf16x8 kt[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) kt[db] = read_transposed(kt_, 16 * half + 8 * m, 32 * db, lane);
#pragma unroll
      for (int db = 0; db < 4; ++db) dq[db] = mfma_bf16(kt[db], sf, dq[db]);
    }
    if (more) {
      ks.put(kbuf[cur ^ 1], tid);  // slot of tile t-1, released by this step's barrier
      vs.put(vbuf[cur ^ 1], tid);
    }
  }

  if (q_valid) {
    float* row = a.dq + ((int64_t)b * a.Sq + qi) * q_rs + (int64_t)hq * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4* p = reinterpret_cast<f32x4*>(row + 32 * db + 8 * r4 + 4 * half);
        f32x4 cur = *p;
#pragma unroll
        for (int j = 0; j < 4; ++j) cur[j] += a.scale * dq[db][4 * r4 + j];
        *p = cur;
      }
  }
}

// ------------------------------------------------------------------------------------
// dK, dV: NW waves x 32 keys of one KV head; walks the 32-query tiles of every
// query head of the GQA group (the group reduction happens in registers).
// ------------------------------------------------------------------------------------
template <bool kSeg, int NW>
__global__ __launch_bounds__(64 * NW) void dkdv_d128_kernel(BwdArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int QBQ = RA_DKDV_QBLOCKS;   // 32-query blocks per staged query tile
  constexpr int QT = kTile * QBQ;        // queries per staged tile
  __shared__ __attribute__((aligned(1024))) __bf16 qbuf[2][QT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 dobuf[2][QT * kD];
  __shared__ float lse_s[2][QT];
  __shared__ float dl_s[2][QT];
  __shared__ int segq_s[2][QT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int kt = logical % a.n_tiles;
  const int g = (logical / a.n_tiles) % a.Hkv;
  const int b = logical / a.n_tiles / a.Hkv;
  const int group = a.Hq / a.Hkv;

  const int k0 = kt * 32 * NW;
  const int k_last = min(k0 + 32 * NW, a.Sk) - 1;
  const int kw = k0 + 32 * wave;
  const int kj = kw + col;
  const bool k_valid = kj < a.Sk;
  const int64_t kgl = a.kv_offset + kj;

  const int64_t q_rs = (int64_t)a.Hq * kD, kv_rs = (int64_t)a.Hkv * kD;

  // K and V of this lane's key as B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kf[8], vf[8];
  {
    const int64_t off = ((int64_t)b * a.Sk + (k_valid ? kj : 0)) * kv_rs + (int64_t)g * kD + 8 * half;
    const __bf16* kp = static_cast<const __bf16*>(a.k) + off;
    const __bf16* vp = static_cast<const __bf16*>(a.v) + off;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[s] = k_valid ? load_bf16x8(kp + 16 * s) : bf16x8{};
      vf[s] = k_valid ? load_bf16x8(vp + 16 * s) : bf16x8{};
    }
  }

  const int n_qt = (a.Sq + QT - 1) / QT;
  int qt_begin = 0, qt_end = n_qt;
  if (a.causal) {
    const int64_t first_q = a.kv_offset + k0 - a.q_offset;
    qt_begin = (int)min<int64_t>((int64_t)n_qt, max<int64_t>(0, first_q) / QT);
  }
  int seg_k = 0;
  const int32_t* seg_row = nullptr;
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    seg_k = k_valid ? seg_row[kgl] : INT32_MIN;
    const int lo = seg_row[a.kv_offset + k0], hi = seg_row[a.kv_offset + k_last];
    int sb, se;
    seg_tile_range(seg_row + a.q_offset, a.Sq, QT, qt_begin, qt_end, lo, hi, sb, se);
    qt_begin = sb;
    qt_end = max(sb, se);
  }
  const int n_q = qt_end - qt_begin;
  const int n_iter = n_q * group;

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  TileStage<NT, QT> qs, ds_;
  float lse_r = 0.0f, dl_r = 0.0f;
  int segq_r = 0;
  auto fetch = [&](int it) {
    const int hq = g * group + it / n_q;
    const int q0 = (qt_begin + it % n_q) * QT;
    const int64_t off = (int64_t)b * a.Sq * q_rs + (int64_t)hq * kD;
    qs.fetch(static_cast<const __bf16*>(a.q) + off, q_rs, q0, a.Sq, tid);
    ds_.fetch(static_cast<const __bf16*>(a.d_o) + off, q_rs, q0, a.Sq, tid);
    if (tid < QT) {
      const int qi = q0 + tid;
      const bool ok = qi < a.Sq;
      const int64_t li = ((int64_t)b * a.Hq + hq) * a.Sq + qi;
      const float l = ok ? a.lse[li] : -INFINITY;
      lse_r = l == -INFINITY ? INFINITY : l * kLog2e;  // rows with no visible key contribute nothing
      dl_r = ok ? a.delta[li] : 0.0f;
      if constexpr (kSeg) segq_r = ok ? seg_row[a.q_offset + qi] : INT32_MAX;
    }
  };
  auto put = [&](int slot) {
    qs.put(qbuf[slot], tid);
    ds_.put(dobuf[slot], tid);
    if (tid < QT) {
      lse_s[slot][tid] = lse_r;
      dl_s[slot][tid] = dl_r;
      if constexpr (kSeg) segq_s[slot][tid] = segq_r;
    }
  };

  if (n_iter > 0) {
    fetch(0);
    put(0);
  }
  for (int it = 0; it < n_iter; ++it) {
    const int cur = it & 1;
    __syncthreads();  // tile `it` visible; every wave is done with tile it-1
    const bool more = it + 1 < n_iter;
    if (more) fetch(it + 1);
    const int qtile0 = (qt_begin + it % n_q) * QT;
    const __bf16* qt_ = qbuf[cur];
    const __bf16* dt_ = dobuf[cur];
#pragma unroll
    for (int qb = 0; qb < QBQ; ++qb) {
      const int q0 = qtile0 + 32 * qb;
      bool partial = (q0 + 32 > a.Sq) || (kw + 32 > a.Sk);  // wave-uniform
      if (a.causal) partial |= (a.kv_offset + kw + 31 > a.q_offset + q0);
      if constexpr (kSeg) partial = true;
      if (a.causal && a.kv_offset + kw > a.q_offset + q0 + 31) continue;  // block entirely before these keys

      // S = Q K^T and dP = dO V^T: lane = key, register i of half h = query q0 + 16h + i.
      f32x16 s = f32x16{}, dp = f32x16{};
      {
        const int row = 32 * qb + key_of_row(col);
        bf16x8 f[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) f[c] = read_chunk(qt_, row, 2 * c + half);
#pragma unroll
        for (int c = 0; c < 8; ++c) s = mfma_bf16(f[c], kf[c], s);
#pragma unroll
        for (int c = 0; c < 8; ++c) f[c] = read_chunk(dt_, row, 2 * c + half);
#pragma unroll
        for (int c = 0; c < 8; ++c) dp = mfma_bf16(f[c], vf[c], dp);
      }
      float p[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        p[i] = exp2_fast(__builtin_fmaf(s[i], a.scale_log2, -lse_s[cur][32 * qb + 16 * half + i]));
      if (partial) {  // one wave-uniform branch around the element mask
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = 32 * qb + 16 * half + i;
          const int qi = qtile0 + ql;
          bool vis = qi < a.Sq && k_valid;
          if (a.causal) vis = vis && (kgl <= a.q_offset + qi);
          if constexpr (kSeg) vis = vis && (segq_s[cur][ql] == seg_k);
          p[i] = vis ? p[i] : 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) dsv[i] = p[i] * (dp[i] - dl_s[cur][32 * qb + 16 * half + i]);
      // dV += P^T dO and dK += dS^T Q; dO^T / Q^T operands by transposing reads.
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 pf = to_bf16x8(p[8 * m], p[8 * m + 1], p[8 * m + 2], p[8 * m + 3], p[8 * m + 4], p[8 * m + 5],
                                    p[8 * m + 6], p[8 * m + 7]);
        const bf16x8 sf = to_bf16x8(dsv[8 * m], dsv[8 * m + 1], dsv[8 * m + 2], dsv[8 * m + 3], dsv[8 * m + 4],
                                    dsv[8 * m + 5], dsv[8 * m + 6], dsv[8 * m + 7]);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 dot = read_transposed(dt_, 32 * qb + 16 * half + 8 * m, 32 * db, lane);
          const bf16x8 qtf = read_transposed(qt_, 32 * qb + 16 * half + 8 * m, 32 * db, lane);
          dv[db] = mfma_bf16(pf, dot, dv[db]);
          dk[db] = mfma_bf16(sf, qtf, dk[db]);
        }
      }
    }
    if (more) put(cur ^ 1);  // slot of tile it-1, released by this step's barrier
  }

  // lane = d column, register i of half h = key kw + mfma32_row(i, h).
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw + mfma32_row(i, half);
      if (key < a.Sk) {
        const int64_t off = ((int64_t)b * a.Sk + key) * kv_rs + (int64_t)g * kD + 32 * db + col;
        a.dk[off] += a.scale * dk[db][i];
        a.dv[off] += dv[db][i];
      }
    }
}

}  // namespace

ra_status launch_bwd_d128(BwdArgs args, hipStream_t stream) {
  constexpr int NW = RA_DKDV_WAVES;
  args.n_tiles = (args.Sk + 32 * NW - 1) / (32 * NW);
  int64_t n_wg = (int64_t)args.B * args.Hkv * args.n_tiles;
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  if (args.seg)
    hipLaunchKernelGGL((dkdv_d128_kernel<true, NW>), dim3((unsigned)n_wg), dim3(64 * NW), 0, stream, args);
  else
    hipLaunchKernelGGL((dkdv_d128_kernel<false, NW>), dim3((unsigned)n_wg), dim3(64 * NW), 0, stream, args);
  ra_status st = check_launch("ring_attn_bwd_step (dK/dV)");
  if (st != RA_OK) return st;
  args.n_tiles = (args.Sq + 32 * kDqWaves - 1) / (32 * kDqWaves);
  n_wg = (int64_t)args.B * args.Hq * args.n_tiles;
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  if (args.seg)
    hipLaunchKernelGGL((dq_d128_kernel<true>), dim3((unsigned)n_wg), dim3(kDqThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((dq_d128_kernel<false>), dim3((unsigned)n_wg), dim3(kDqThreads), 0, stream, args);
  return check_launch("ring_attn_bwd_step (dQ)");
}

}  // namespace ra
