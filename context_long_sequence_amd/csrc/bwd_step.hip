// ring_attn_bwd_step: one ring step of the attention backward pass for one KV
// chunk, on gfx950 MFMA.
//
// The forward kept only O and the merged log-sum-exp; the probabilities are
// recomputed here (archcrux, "sequence-parallel long-context attention OOM":
// FlashAttention-style kernels never store the score matrix but still have to
// backpropagate over the whole context; recomputation trades memory for work):
//   P_ij = exp(s_ij - LSE_i)   (s = scale q.k, LSE = final merged log-sum-exp)
//   dV_j += sum_i P_ij dO_i,   dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - delta_i)
//   dK_j += scale sum_i dS_ij q_i,   dQ_i += scale sum_j dS_ij k_j.
//
// Two kernels, no atomics, deterministic:
//  * dkdv_kernel: a workgroup owns 128 keys of one KV head (32 per wave) and
//    walks the query tiles of every query head of its GQA group, so the group
//    reduction of dK/dV happens in registers.  Scores are computed as S = Q K^T
//    with the KEY in the lane, which lets P^T and dS^T feed the dV/dK MFMAs
//    directly from registers; Q and dO are staged in LDS both row-major and
//    transposed.
//  * dq_kernel: a workgroup owns 128 queries of one query head (32 per wave)
//    and walks the key tiles like the forward (query in the lane); K is staged
//    row-major and transposed, V row-major.
// dK/dV and dQ are read-modify-written (+=) by exactly one workgroup each.
#include <mutex>
#include <type_traits>

#include "bwd_d128.h"

namespace ra {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Stores a pair of 16-byte rows (items 2p and 2p+1, columns ch*E .. ch*E+E-1) into a
// transposed LDS tile: dst[(ch*E + j) * pitch + 2p + {0,1}].
template <typename T>
__device__ __forceinline__ void store_pair_transposed(T* dst, int pitch, int p, int ch, u32x4 x0, u32x4 x1) {
  constexpr int E = 16 / sizeof(T);
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = (x0[j] & 0xFFFFu) | (x1[j] << 16);
      const uint32_t hi = (x0[j] >> 16) | (x1[j] & 0xFFFF0000u);
      *reinterpret_cast<uint32_t*>(&dst[(ch * E + 2 * j) * pitch + 2 * p]) = lo;
      *reinterpret_cast<uint32_t*>(&dst[(ch * E + 2 * j + 1) * pitch + 2 * p]) = hi;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x2 pr = {u32_as_f32(x0[j]), u32_as_f32(x1[j])};
      *reinterpret_cast<f32x2*>(&dst[(ch * E + j) * pitch + 2 * p]) = pr;
    }
  }
}

// ------------------------------------------------------------------------------------
// dK, dV
// ------------------------------------------------------------------------------------
template <typename T, int D, bool kSeg>
__global__ __launch_bounds__(kThreads) void dkdv_kernel(BwdArgs a) {
  using M = Mfma<T>;
  constexpr int KPL = M::KPL;
  constexpr int E = 16 / sizeof(T);
  constexpr int PAD = 16 / sizeof(T);
  constexpr int BMQ = 64;                 // queries per tile (two 32-query MFMA blocks)
  constexpr int QP = D + PAD;             // row-major Q/dO pitch
  constexpr int TP = BMQ + PAD;           // transposed Q/dO pitch
  constexpr int QSTEPS = D / (2 * KPL);
  constexpr int PSTEPS = 16 / KPL;
  constexpr int DB = D / 32;
  constexpr int UNITS = (BMQ / 2) * (D / E);  // (query pair, 16-byte chunk)
  constexpr int UL = (UNITS + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) T q_lds[BMQ * QP];
  __shared__ __attribute__((aligned(16))) T do_lds[BMQ * QP];
  __shared__ __attribute__((aligned(16))) T qt_lds[D * TP];
  __shared__ __attribute__((aligned(16))) T dot_lds[D * TP];
  __shared__ float lse_lds[BMQ];
  __shared__ float dl_lds[BMQ];
  __shared__ int segq_lds[BMQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int kt = logical % a.n_tiles;
  const int g = (logical / a.n_tiles) % a.Hkv;
  const int b = logical / a.n_tiles / a.Hkv;
  const int group = a.Hq / a.Hkv;

  const int k0 = kt * 32 * kWaves;          // first key of the workgroup
  const int k_last = min(k0 + 32 * kWaves, a.Sk) - 1;
  const int kw = k0 + 32 * wave;            // first key of this wave
  const int kj = kw + col;                  // this lane's key (column of S)
  const bool k_valid = kj < a.Sk;
  const int64_t kgl = a.kv_offset + kj;     // global key index

  const T* qb = static_cast<const T*>(a.q);
  const T* kb = static_cast<const T*>(a.k);
  const T* vb = static_cast<const T*>(a.v);
  const T* dob = static_cast<const T*>(a.d_o);
  const int64_t q_rs = (int64_t)a.Hq * D;
  const int64_t kv_rs = (int64_t)a.Hkv * D;

  // K and V of this lane's key as B operands of S = Q K^T and dP = dO V^T.
  typename M::frag kf[QSTEPS], vf[QSTEPS];
  {
    const int64_t off = ((int64_t)b * a.Sk + (k_valid ? kj : 0)) * kv_rs + (int64_t)g * D + KPL * half;
#pragma unroll
    for (int s = 0; s < QSTEPS; ++s) {
      kf[s] = k_valid ? M::load(kb + off + s * 2 * KPL) : typename M::frag{};
      vf[s] = k_valid ? M::load(vb + off + s * 2 * KPL) : typename M::frag{};
    }
  }

  // Query tiles that can see any key of this workgroup.
  const int n_qt = (a.Sq + BMQ - 1) / BMQ;
  int qt_begin = 0, qt_end = n_qt;
  if (a.causal) {
    const int64_t first_q = a.kv_offset + k0 - a.q_offset;  // first local query that sees key k0
    qt_begin = (int)min<int64_t>((int64_t)n_qt, max<int64_t>(0, first_q) / BMQ);
  }
  int seg_k = 0;
  const int32_t* seg_row = nullptr;
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    seg_k = k_valid ? seg_row[kgl] : INT32_MIN;
    const int lo = seg_row[a.kv_offset + k0], hi = seg_row[a.kv_offset + k_last];
    int sb, se;
    seg_tile_range(seg_row + a.q_offset, a.Sq, BMQ, qt_begin, qt_end, lo, hi, sb, se);
    qt_begin = sb;
    qt_end = max(sb, se);
  }
  const int n_iter = (qt_end - qt_begin) * group;

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  u32x4 qreg[UL][2], dreg[UL][2];
  float lse_r = 0.f, dl_r = 0.f;
  int segq_r = 0;
  auto load_tile = [&](int it) {
    const int hq = g * group + it / (qt_end - qt_begin);
    const int q0 = (qt_begin + it % (qt_end - qt_begin)) * BMQ;
#pragma unroll
    for (int r = 0; r < UL; ++r) {
      const int u = tid + r * kThreads;
      const int p = u % (BMQ / 2), ch = u / (BMQ / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int qi = q0 + 2 * p + e;
        if (u < UNITS && qi < a.Sq) {
          const int64_t off = ((int64_t)b * a.Sq + qi) * q_rs + (int64_t)hq * D + ch * E;
          qreg[r][e] = *reinterpret_cast<const u32x4*>(qb + off);
          dreg[r][e] = *reinterpret_cast<const u32x4*>(dob + off);
        } else {
          qreg[r][e] = u32x4{0, 0, 0, 0};
          dreg[r][e] = u32x4{0, 0, 0, 0};
        }
      }
    }
    if (tid < BMQ) {
      const int qi = q0 + tid;
      const bool ok = qi < a.Sq;
      const int64_t li = ((int64_t)b * a.Hq + hq) * a.Sq + qi;
      // A row with no visible key anywhere (LSE = -inf) contributes nothing.
      const float l = ok ? a.lse[li] : -INFINITY;
      lse_r = l == -INFINITY ? INFINITY : l * kLog2e;
      dl_r = ok ? a.delta[li] : 0.f;
      if constexpr (kSeg) segq_r = ok ? seg_row[a.q_offset + qi] : INT32_MAX;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < UL; ++r) {
      const int u = tid + r * kThreads;
      if (u < UNITS) {
        const int p = u % (BMQ / 2), ch = u / (BMQ / 2);
        *reinterpret_cast<u32x4*>(&q_lds[(2 * p) * QP + ch * E]) = qreg[r][0];
        *reinterpret_cast<u32x4*>(&q_lds[(2 * p + 1) * QP + ch * E]) = qreg[r][1];
        *reinterpret_cast<u32x4*>(&do_lds[(2 * p) * QP + ch * E]) = dreg[r][0];
        *reinterpret_cast<u32x4*>(&do_lds[(2 * p + 1) * QP + ch * E]) = dreg[r][1];
        store_pair_transposed<T>(qt_lds, TP, p, ch, qreg[r][0], qreg[r][1]);
        store_pair_transposed<T>(dot_lds, TP, p, ch, dreg[r][0], dreg[r][1]);
      }
    }
    if (tid < BMQ) {
      lse_lds[tid] = lse_r;
      dl_lds[tid] = dl_r;
      if constexpr (kSeg) segq_lds[tid] = segq_r;
    }
  };

  if (n_iter > 0) load_tile(0);
  for (int it = 0; it < n_iter; ++it) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < n_iter) load_tile(it + 1);
    const int q0 = (qt_begin + it % (qt_end - qt_begin)) * BMQ;

    bool partial = (q0 + BMQ > a.Sq) || (kw + 32 > a.Sk);
    if (a.causal) partial |= (a.kv_offset + kw + 31 > a.q_offset + q0);
    if constexpr (kSeg) partial = true;

    auto tile = [&](auto mask_tag) {
      constexpr bool kMask = decltype(mask_tag)::value;
#pragma unroll
      for (int qb = 0; qb < BMQ / 32; ++qb) {
        // S = Q K^T and dP = dO V^T: lane = key, register i of half h = query 32qb + 16h + i.
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
        {
          const T* qrow = &q_lds[(32 * qb + key_of_row(col)) * QP + KPL * half];
          typename M::frag f[QSTEPS];
#pragma unroll
          for (int s = 0; s < QSTEPS; ++s) f[s] = M::load(qrow + s * 2 * KPL);
#pragma unroll
          for (int s = 0; s < QSTEPS; ++s) sacc = M::mma(f[s], kf[s], sacc);
        }
        {
          const T* drow = &do_lds[(32 * qb + key_of_row(col)) * QP + KPL * half];
          typename M::frag f[QSTEPS];
#pragma unroll
          for (int s = 0; s < QSTEPS; ++s) f[s] = M::load(drow + s * 2 * KPL);
#pragma unroll
          for (int s = 0; s < QSTEPS; ++s) dpacc = M::mma(f[s], vf[s], dpacc);
        }
        float p[16], ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = 32 * qb + 16 * half + i;
          float pi = exp2_fast(__builtin_fmaf(sacc[i], a.scale_log2, -lse_lds[ql]));
          if constexpr (kMask) {
            const int qi = q0 + ql;
            bool vis = qi < a.Sq && k_valid;
            if (a.causal) vis = vis && (kgl <= a.q_offset + qi);
            if constexpr (kSeg) vis = vis && (segq_lds[ql] == seg_k);
            pi = vis ? pi : 0.0f;
          }
          p[i] = pi;
          ds[i] = pi * (dpacc[i] - dl_lds[ql]);
        }
        // dV += P^T dO, dK += dS^T Q (scale applied at the end).
#pragma unroll
        for (int m = 0; m < PSTEPS; ++m) {
          typename M::frag dof_t[DB], qf_t[DB];
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int off = (32 * db + col) * TP + 32 * qb + 16 * half + KPL * m;
            dof_t[db] = M::load(&dot_lds[off]);
            qf_t[db] = M::load(&qt_lds[off]);
          }
          const typename M::frag pf = M::pack(&p[m * KPL]);
          const typename M::frag sf = M::pack(&ds[m * KPL]);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            dvacc[db] = M::mma(pf, dof_t[db], dvacc[db]);
            dkacc[db] = M::mma(sf, qf_t[db], dkacc[db]);
          }
        }
      }
    };
    if (partial)
      tile(BoolTag<true>{});
    else
      tile(BoolTag<false>{});
  }

  // dK/dV accumulators: lane = d column, register i of half h = key row mfma32_row(i, h).
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw + mfma32_row(i, half);
      if (key < a.Sk) {
        const int64_t off = ((int64_t)b * a.Sk + key) * kv_rs + (int64_t)g * D + 32 * db + col;
        a.dk[off] += a.scale * dkacc[db][i];
        a.dv[off] += dvacc[db][i];
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// dQ
// ------------------------------------------------------------------------------------
template <typename T, int D, bool kSeg>
__global__ __launch_bounds__(kThreads) void dq_kernel(BwdArgs a) {
  using M = Mfma<T>;
  constexpr int KPL = M::KPL;
  constexpr int E = 16 / sizeof(T);
  constexpr int PAD = 16 / sizeof(T);
  constexpr int BN = 64;
  constexpr int BM = 32 * kWaves;
  constexpr int KP = D + PAD;        // row-major K/V pitch
  constexpr int TP = BN + PAD;       // transposed K pitch
  constexpr int QSTEPS = D / (2 * KPL);
  constexpr int PSTEPS = 16 / KPL;
  constexpr int DB = D / 32;
  constexpr int KUNITS = (BN / 2) * (D / E);   // (key pair, chunk) units of K
  constexpr int VCH = BN * D / E;               // 16-byte chunks of V
  static_assert(KUNITS % kThreads == 0 && VCH % kThreads == 0, "tile/threads mismatch");
  constexpr int KL = KUNITS / kThreads;
  constexpr int VL = VCH / kThreads;

  __shared__ __attribute__((aligned(16))) T k_lds[BN * KP];
  __shared__ __attribute__((aligned(16))) T v_lds[BN * KP];
  __shared__ __attribute__((aligned(16))) T kt_lds[D * TP];
  __shared__ int segk_lds[BN];

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

  const int q0 = qt * BM;
  const int q_last = min(q0 + BM, a.Sq) - 1;
  const int qw = q0 + wave * 32;
  const int qi = qw + col;
  const bool q_valid = qi < a.Sq;
  const int64_t qg = a.q_offset + qi;

  const T* qb = static_cast<const T*>(a.q);
  const T* kb = static_cast<const T*>(a.k);
  const T* vb = static_cast<const T*>(a.v);
  const T* dob = static_cast<const T*>(a.d_o);
  const int64_t q_rs = (int64_t)a.Hq * D;
  const int64_t kv_rs = (int64_t)a.Hkv * D;

  int n_keys = a.Sk;
  if (a.causal) {
    const int64_t last_visible = a.q_offset + q_last - a.kv_offset;
    n_keys = (int)max<int64_t>(0, min<int64_t>((int64_t)a.Sk, last_visible + 1));
  }
  int kt_begin = 0, kt_end = (n_keys + BN - 1) / BN;
  int seg_q = 0;
  const int32_t* seg_row = nullptr;
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    const int lo = seg_row[a.q_offset + q0], hi = seg_row[a.q_offset + q_last];
    seg_q = q_valid ? seg_row[a.q_offset + qi] : lo;
    int sb, se;
    seg_tile_range(seg_row + a.kv_offset, a.Sk, BN, 0, kt_end, lo, hi, sb, se);
    kt_begin = sb;
    kt_end = max(sb, se);
  }

  typename M::frag qf[QSTEPS], dof[QSTEPS];
  {
    const int64_t off = ((int64_t)b * a.Sq + (q_valid ? qi : 0)) * q_rs + (int64_t)hq * D + KPL * half;
#pragma unroll
    for (int s = 0; s < QSTEPS; ++s) {
      qf[s] = q_valid ? M::load(qb + off + s * 2 * KPL) : typename M::frag{};
      dof[s] = q_valid ? M::load(dob + off + s * 2 * KPL) : typename M::frag{};
    }
  }
  const int64_t li = ((int64_t)b * a.Hq + hq) * a.Sq + (q_valid ? qi : 0);
  const float lse_q = q_valid ? a.lse[li] : -INFINITY;
  const float lse2 = lse_q == -INFINITY ? INFINITY : lse_q * kLog2e;
  const float dl = q_valid ? a.delta[li] : 0.0f;

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

  u32x4 kreg[KL][2], vreg[VL];
  int sreg = 0;
  auto load_tile = [&](int t) {
    const int k0 = t * BN;
#pragma unroll
    for (int r = 0; r < KL; ++r) {
      const int u = tid + r * kThreads;
      const int p = u % (BN / 2), ch = u / (BN / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int kj = k0 + 2 * p + e;
        kreg[r][e] = kj < a.Sk ? *reinterpret_cast<const u32x4*>(kb + ((int64_t)b * a.Sk + kj) * kv_rs +
                                                                 (int64_t)g * D + ch * E)
                               : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int c = tid + r * kThreads;
      const int key = c / (D / E), ch = c % (D / E);
      const int kj = k0 + key;
      vreg[r] = kj < a.Sk ? *reinterpret_cast<const u32x4*>(vb + ((int64_t)b * a.Sk + kj) * kv_rs +
                                                            (int64_t)g * D + ch * E)
                          : u32x4{0, 0, 0, 0};
    }
    if constexpr (kSeg) {
      if (tid < BN) sreg = (k0 + tid < a.Sk) ? seg_row[a.kv_offset + k0 + tid] : INT32_MIN;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < KL; ++r) {
      const int u = tid + r * kThreads;
      const int p = u % (BN / 2), ch = u / (BN / 2);
      *reinterpret_cast<u32x4*>(&k_lds[(2 * p) * KP + ch * E]) = kreg[r][0];
      *reinterpret_cast<u32x4*>(&k_lds[(2 * p + 1) * KP + ch * E]) = kreg[r][1];
      store_pair_transposed<T>(kt_lds, TP, p, ch, kreg[r][0], kreg[r][1]);
    }
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int c = tid + r * kThreads;
      const int key = c / (D / E), ch = c % (D / E);
      *reinterpret_cast<u32x4*>(&v_lds[key * KP + ch * E]) = vreg[r];
    }
    if constexpr (kSeg) {
      if (tid < BN) segk_lds[tid] = sreg;
    }
  };

  if (kt_begin < kt_end) load_tile(kt_begin);
  for (int t = kt_begin; t < kt_end; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < kt_end) load_tile(t + 1);
    const int k0 = t * BN;
    // Wave-uniform (the two tile bodies contain MFMAs, which must not diverge).
    bool partial = (k0 + BN > a.Sk) || (qw + 32 > a.Sq);
    if (a.causal) partial |= (a.kv_offset + k0 + BN - 1 > a.q_offset + qw);
    if constexpr (kSeg) partial = true;

    auto tile = [&](auto mask_tag) {
      constexpr bool kMask = decltype(mask_tag)::value;
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk) {
        const T* krow = &k_lds[(32 * kbk + key_of_row(col)) * KP + KPL * half];
        const T* vrow = &v_lds[(32 * kbk + key_of_row(col)) * KP + KPL * half];
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
        {
          typename M::frag kf[QSTEPS];
#pragma unroll
          for (int s = 0; s < QSTEPS; ++s) kf[s] = M::load(krow + s * 2 * KPL);
#pragma unroll
          for (int s = 0; s < QSTEPS; ++s) sacc = M::mma(kf[s], qf[s], sacc);
        }
        {
          typename M::frag vf[QSTEPS];
#pragma unroll
          for (int s = 0; s < QSTEPS; ++s) vf[s] = M::load(vrow + s * 2 * KPL);
#pragma unroll
          for (int s = 0; s < QSTEPS; ++s) dpacc = M::mma(vf[s], dof[s], dpacc);
        }
        typename M::frag ktf[PSTEPS][DB];
#pragma unroll
        for (int m = 0; m < PSTEPS; ++m)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            ktf[m][db] = M::load(&kt_lds[(32 * db + col) * TP + 32 * kbk + 16 * half + KPL * m]);
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pi = exp2_fast(__builtin_fmaf(sacc[i], a.scale_log2, -lse2));
          if constexpr (kMask) {
            const int kl = 32 * kbk + 16 * half + i;
            const int kj = k0 + kl;
            bool vis = q_valid && kj < a.Sk;
            if (a.causal) vis = vis && (a.kv_offset + kj <= qg);
            if constexpr (kSeg) vis = vis && (segk_lds[kl] == seg_q);
            pi = vis ? pi : 0.0f;
          }
          ds[i] = pi * (dpacc[i] - dl);
        }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int m = 0; m < PSTEPS; ++m) {
          const typename M::frag sf = M::pack(&ds[m * KPL]);
#pragma unroll
          for (int db = 0; db < DB; ++db) dqacc[db] = M::mma(ktf[m][db], sf, dqacc[db]);
        }
      }
    };
    if (partial)
      tile(BoolTag<true>{});
    else
      tile(BoolTag<false>{});
  }

  if (q_valid) {
    float* row = a.dq + ((int64_t)b * a.Sq + qi) * q_rs + (int64_t)hq * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4* p = reinterpret_cast<f32x4*>(row + 32 * db + 8 * r4 + 4 * half);
        f32x4 cur = *p;
        cur[0] += a.scale * dqacc[db][4 * r4];
        cur[1] += a.scale * dqacc[db][4 * r4 + 1];
        cur[2] += a.scale * dqacc[db][4 * r4 + 2];
        cur[3] += a.scale * dqacc[db][4 * r4 + 3];
        *p = cur;
      }
    }
  }
}

// Scratch of the split dK/dV kernel: kDkdvScratchBytes of device memory per device,
// allocated by the first step that splits and kept until the process ends.  Steps
// on one device share it, so steps that overlap on one device (different streams)
// must not both split; the ring runs its steps in stream order.
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

ra_status device_scratch(void*& out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(RA_ERR_HIP, "ring_attn_bwd_step: no current device");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipMalloc(&p, kDkdvScratchBytes) != hipSuccess)
      return fail(RA_ERR_HIP, "ring_attn_bwd_step: scratch allocation (%zu bytes) failed", kDkdvScratchBytes);
    g_scratch[dev] = p;
  }
  out = g_scratch[dev];
  return RA_OK;
}

template <typename T, int D>
ra_status launch_bwd(BwdArgs args, hipStream_t stream, void* scratch, bool allocate, bool side) {
  if constexpr (std::is_same<T, __bf16>::value && D == 128) {
    if (!scratch && bwd_d128_needs_scratch(args)) {
      if (!allocate) return fail(RA_ERR_INVALID_ARGUMENT, "ring_attn_bwd_step: this step needs scratch");
      const ra_status st = device_scratch(scratch);
      if (st != RA_OK) return st;
    }
    return launch_bwd_d128(args, stream, scratch, side);
  }
  // dK/dV: one workgroup per (b, kv head, 128-key tile).
  args.n_tiles = (args.Sk + 32 * kWaves - 1) / (32 * kWaves);
  int64_t n_wg = (int64_t)args.B * args.Hkv * args.n_tiles;
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  if (args.seg)
    hipLaunchKernelGGL((dkdv_kernel<T, D, true>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((dkdv_kernel<T, D, false>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, args);
  ra_status st = check_launch("ring_attn_bwd_step (dK/dV)");
  if (st != RA_OK) return st;
  // dQ: one workgroup per (b, q head, 128-query tile).
  args.n_tiles = (args.Sq + 32 * kWaves - 1) / (32 * kWaves);
  n_wg = (int64_t)args.B * args.Hq * args.n_tiles;
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  if (args.seg)
    hipLaunchKernelGGL((dq_kernel<T, D, true>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((dq_kernel<T, D, false>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, args);
  return check_launch("ring_attn_bwd_step (dQ)");
}

}  // namespace
}  // namespace ra

namespace ra {

ra_status bwd_step_entry(const ra_shape* s, const void* q, const void* k, const void* v, const void* d_o,
                         const float* lse, const float* delta, const int32_t* seg_ids, int64_t seg_len,
                         float* dq_acc, float* dk_acc, float* dv_acc, void* stream, void* scratch, bool allocate,
                         bool side) {
  ra_status st = validate_step(s, seg_ids, seg_len);
  if (st != RA_OK) return st;
  if (!q || !k || !v || !d_o || !lse || !delta || !dq_acc || !dk_acc || !dv_acc)
    return fail(RA_ERR_INVALID_ARGUMENT, "q, k, v, d_o, lse, delta, dq_acc, dk_acc and dv_acc must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o) || !aligned16(lse) ||
      !aligned16(delta) || !aligned16(dq_acc) || !aligned16(dk_acc) || !aligned16(dv_acc))
    return fail(RA_ERR_INVALID_ARGUMENT, "all tensor pointers must be 16-byte aligned");
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.d_o = d_o;
  a.lse = lse;
  a.delta = delta;
  a.seg = seg_ids;
  a.seg_len = seg_len;
  a.dq = dq_acc;
  a.dk = dk_acc;
  a.dv = dv_acc;
  a.B = s->batch;
  a.Sq = s->q_len;
  a.Sk = s->kv_len;
  a.Hq = s->heads_q;
  a.Hkv = s->heads_kv;
  a.q_offset = s->q_offset;
  a.kv_offset = s->kv_offset;
  a.causal = s->causal;
  a.scale = s->softmax_scale;
  a.scale_log2 = s->softmax_scale * kLog2e;
  a.n_tiles = 0;
  a.part = nullptr;
  a.count = nullptr;
  a.n_split = 1;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (s->dtype == RA_DTYPE_BF16) {
    if (s->head_dim == 128) return launch_bwd<__bf16, 128>(a, hs, scratch, allocate, side);
    return launch_bwd<__bf16, 64>(a, hs, scratch, allocate, side);
  }
  if (s->head_dim == 128) return launch_bwd<float, 128>(a, hs, scratch, allocate, side);
  return launch_bwd<float, 64>(a, hs, scratch, allocate, side);
}

}  // namespace ra

extern "C" ra_status ring_attn_bwd_step(const ra_shape* s, const void* q, const void* k, const void* v,
                                        const void* d_o, const float* lse, const float* delta,
                                        const int32_t* seg_ids, int64_t seg_len, float* dq_acc, float* dk_acc,
                                        float* dv_acc, void* stream) {
  return ra::bwd_step_entry(s, q, k, v, d_o, lse, delta, seg_ids, seg_len, dq_acc, dk_acc, dv_acc, stream, nullptr,
                            true, true);
}
