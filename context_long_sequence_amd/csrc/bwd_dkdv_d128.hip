// dK, dV of one backward ring step for the hot shape (bf16, head_dim 128):
//   dV_j += sum_i P_ij dO_i,  dK_j += scale * sum_i P_ij (dP_ij - delta_i) q_i,
// summed over the query heads of the KV head's GQA group, P recomputed from the
// final log-sum-exp (archcrux, "sequence-parallel long-context attention OOM").
// Each wave keeps 32 keys' K and V operands and dK/dV accumulators in registers
// and walks the 64-query tiles of every query head of the group.  Q and dO tiles
// are copied global -> LDS (swizzled, row-major) two steps ahead into a ring of
// three slots without passing through registers; their transposes are read with
// transposing LDS reads.
#include "bwd_d128.h"

#ifndef RA_DKDV_BATCH
#define RA_DKDV_BATCH 1  // issue each MFMA chain's operand reads before its first MFMA
#endif

namespace ra {
namespace {

constexpr int kD = kD128;
constexpr int kTile = kD128Tile;

// ------------------------------------------------------------------------------------
// dK, dV: NW waves x 32 keys of one KV head; walks the 32-query tiles of every
// query head of the GQA group (the group reduction happens in registers).
// ------------------------------------------------------------------------------------
template <bool kSeg, int NW>
__global__ __launch_bounds__(64 * NW) void dkdv_d128_kernel(BwdArgs a) {
  static_assert(NW == 4, "the tile copy below splits each tile over exactly 4 waves");
  constexpr int QT = 64;  // queries per staged tile (two 32-query MFMA blocks)
  // Three tile slots per tensor, each its own array so that the compiler can tell
  // the slot being read from the slots still being filled.
  __shared__ __attribute__((aligned(1024))) __bf16 qs0[QT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 qs1[QT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 qs2[QT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ds0[QT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ds1[QT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ds2[QT * kD];
  // per slot: lse[QT], delta[QT], segment id bits[QT], and a landing zone for the
  // 4th wave's copy (every wave issues the same number of copies per tile)
  __shared__ __attribute__((aligned(1024))) float xs0[4 * QT];
  __shared__ __attribute__((aligned(1024))) float xs1[4 * QT];
  __shared__ __attribute__((aligned(1024))) float xs2[4 * QT];

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
  int seg_w_lo = 0, seg_w_hi = 0;  // segment ids of the wave's first and last key
  const int32_t* seg_row = nullptr;
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    seg_k = k_valid ? seg_row[kgl] : INT32_MIN;
    seg_w_lo = seg_row[a.kv_offset + min(kw, a.Sk - 1)];
    seg_w_hi = seg_row[a.kv_offset + min(kw + 32, a.Sk) - 1];
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

  const __bf16* qg_base = static_cast<const __bf16*>(a.q) + (int64_t)b * a.Sq * q_rs;
  const __bf16* dg_base = static_cast<const __bf16*>(a.d_o) + (int64_t)b * a.Sq * q_rs;

  // Copies tile t (query head, 64 queries) global -> LDS slot without registers:
  // 4 + 4 sixteen-byte copies of Q/dO rows and one 4-byte-per-lane copy of
  // lse (wave 0), delta (wave 1), segment ids (wave 2) or a dummy (wave 3).
  auto issue = [&](int t, __bf16* qs, __bf16* ds, float* xs) {
    const int hq = g * group + t / n_q;
    const int q0 = (qt_begin + t % n_q) * QT;
    const int64_t hoff = (int64_t)hq * kD + (int64_t)q0 * q_rs;
    load_rows_lds<QT, 4>(qs, qg_base + hoff, q_rs, a.Sq - q0, wave, lane);
    load_rows_lds<QT, 4>(ds, dg_base + hoff, q_rs, a.Sq - q0, wave, lane);
    const int qi = min(q0 + lane, a.Sq - 1);
    const int64_t li = ((int64_t)b * a.Hq + hq) * a.Sq + qi;
    const void* src = a.lse + li;
    if (wave == 1) src = a.delta + li;
    if constexpr (kSeg) {
      if (wave == 2) src = seg_row + a.q_offset + qi;
    }
    __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)(xs + wave * QT), 4, 0, 0);
  };
  constexpr int kCopiesPerTile = 9;
  static_assert(kCopiesPerTile == 2 * (QT / 4 / 4) + 1, "copy count per wave and tile");

  auto compute = [&](int it, const __bf16* qt_, const __bf16* dt_, const float* xs) {
    const int qtile0 = (qt_begin + it % n_q) * QT;
#pragma unroll
    for (int qb = 0; qb < QT / 32; ++qb) {
      const int q0 = qtile0 + 32 * qb;
      bool partial = (q0 + 32 > a.Sq) || (kw + 32 > a.Sk);  // wave-uniform
      if (a.causal) partial |= (a.kv_offset + kw + 31 > a.q_offset + q0);
      if constexpr (kSeg) {
        // Segment ids are nondecreasing: only blocks that straddle a segment
        // boundary need the per-element segment test.
        const int sq_lo = __builtin_bit_cast(int, xs[2 * QT + 32 * qb]);
        const int sq_hi = __builtin_bit_cast(int, xs[2 * QT + 32 * qb + 31]);
        partial |= !(sq_lo == sq_hi && sq_lo == seg_w_lo && seg_w_lo == seg_w_hi);
      }
      if (a.causal && a.kv_offset + kw > a.q_offset + q0 + 31) continue;  // block entirely before these keys

      // S = Q K^T and dP = dO V^T: lane = key, register i of half h = query q0 + 16h + i.
      f32x16 s = f32x16{}, dp = f32x16{};
      {
        const int row = 32 * qb + key_of_row(col);
        bf16x8 fq[8], fd[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) fq[c] = read_chunk(qt_, row, 2 * c + half);
#pragma unroll
        for (int c = 0; c < 8; ++c) fd[c] = read_chunk(dt_, row, 2 * c + half);
        if constexpr (RA_DKDV_BATCH) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          s = mfma_bf16(fq[c], kf[c], s);
          dp = mfma_bf16(fd[c], vf[c], dp);
        }
      }
      float p[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float l = xs[32 * qb + 16 * half + i];
        // a row with no visible key at all (LSE = -inf) contributes nothing
        const float neg_lse2 = l == -INFINITY ? -INFINITY : -l * kLog2e;
        p[i] = exp2_fast(__builtin_fmaf(s[i], a.scale_log2, neg_lse2));
      }
      if (partial) {  // one wave-uniform branch around the element mask
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = 32 * qb + 16 * half + i;
          const int qi = qtile0 + ql;
          bool vis = qi < a.Sq && k_valid;
          if (a.causal) vis = vis && (kgl <= a.q_offset + qi);
          if constexpr (kSeg) vis = vis && (__builtin_bit_cast(int, xs[2 * QT + ql]) == seg_k);
          p[i] = vis ? p[i] : 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) dsv[i] = p[i] * (dp[i] - xs[QT + 32 * qb + 16 * half + i]);
      // dV += P^T dO and dK += dS^T Q; dO^T / Q^T operands by transposing reads.
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 pf = to_bf16x8(p[8 * m], p[8 * m + 1], p[8 * m + 2], p[8 * m + 3], p[8 * m + 4], p[8 * m + 5],
                                    p[8 * m + 6], p[8 * m + 7]);
        const bf16x8 sf = to_bf16x8(dsv[8 * m], dsv[8 * m + 1], dsv[8 * m + 2], dsv[8 * m + 3], dsv[8 * m + 4],
                                    dsv[8 * m + 5], dsv[8 * m + 6], dsv[8 * m + 7]);
        bf16x8 dot[4], qtf[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          dot[db] = read_transposed(dt_, 32 * qb + 16 * half + 8 * m, 32 * db, lane);
          qtf[db] = read_transposed(qt_, 32 * qb + 16 * half + 8 * m, 32 * db, lane);
        }
        if constexpr (RA_DKDV_BATCH) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          dv[db] = mfma_bf16(pf, dot[db], dv[db]);
          dk[db] = mfma_bf16(sf, qtf[db], dk[db]);
        }
      }
    }
  };

  // One step: wait for tile `it` (copies issued two steps ago), publish it to the
  // workgroup, start copying tile it+2 into the slot tile it-1 used, compute.
  // The barrier is a bare s_barrier: a workgroup fence would also wait for the
  // copies still in flight.  The empty asm statements keep the compiler from
  // moving LDS accesses across it; the copies of this wave are waited for
  // explicitly (vmcnt counts them in issue order).
  auto step = [&](int it, const __bf16* qc, const __bf16* dc, const float* xc, __bf16* qn, __bf16* dn, float* xn) {
    if (it + 1 < n_iter)
      __builtin_amdgcn_s_waitcnt(0x0F70 | kCopiesPerTile);  // vmcnt(9): tile it+1 may stay in flight
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (it + 2 < n_iter) issue(it + 2, qn, dn, xn);
    compute(it, qc, dc, xc);
  };

  if (n_iter > 0) issue(0, qs0, ds0, xs0);
  if (n_iter > 1) issue(1, qs1, ds1, xs1);
  for (int it = 0; it < n_iter; it += 3) {
    step(it, qs0, ds0, xs0, qs2, ds2, xs2);
    if (it + 1 < n_iter) step(it + 1, qs1, ds1, xs1, qs0, ds0, xs0);
    if (it + 2 < n_iter) step(it + 2, qs2, ds2, xs2, qs1, ds1, xs1);
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

ra_status launch_dkdv_d128(BwdArgs args, hipStream_t stream) {
  constexpr int NW = RA_DKDV_WAVES;
  args.n_tiles = (args.Sk + 32 * NW - 1) / (32 * NW);
  const int64_t n_wg = (int64_t)args.B * args.Hkv * args.n_tiles;
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  if (args.seg)
    hipLaunchKernelGGL((dkdv_d128_kernel<true, NW>), dim3((unsigned)n_wg), dim3(64 * NW), 0, stream, args);
  else
    hipLaunchKernelGGL((dkdv_d128_kernel<false, NW>), dim3((unsigned)n_wg), dim3(64 * NW), 0, stream, args);
  return check_launch("ring_attn_bwd_step (dK/dV)");
}

}  // namespace ra
