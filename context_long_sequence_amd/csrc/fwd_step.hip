// ring_attn_fwd_step: one ring step of attention — the local query shard against
// one KV chunk — on gfx950 MFMA.
//
// What is computed (per batch row b, query head h, local query i):
//   s_ij = scale * q_i . k_j over the visible keys j of this chunk,
//   O_i = sum_j softmax_j(s_ij) v_j,  LSE_i = ln sum_j exp(s_ij)
// with O = 0, LSE = -inf for a row that sees no key of this chunk.  This is the
// per-chunk partial result that the ring merges step by step (axolotl docs
// "Sequence Parallelism", introduction and Implementation Details; aicassindra
// "Transformer math: SP math", section on context parallelism).  The score
// matrix only ever exists one 32x64 register tile at a time (archcrux,
// "sequence-parallel long-context attention OOM").
//
// Work decomposition: one workgroup = 4 waves = 128 queries of one (b, h); each
// wave owns 32 queries.  The workgroup walks the chunk in tiles of 64 keys that
// are staged in LDS (K row-major, V transposed) and shared by the 4 waves.
//
// Register layout: scores are computed transposed, S^T = K Q^T, so that the
// accumulator column — the lane — is the query: lane l and lane l+32 hold the
// 32 keys of one query row between them, and the row max / row sum are
// in-register reductions plus one exchange between the two half-waves.  K rows
// are loaded in a permuted order so that register i of half h holds key 16h+i;
// P then feeds the P.V MFMA (O^T = V^T P^T) straight from registers as its B
// operand, and V^T is read from LDS as 16-byte rows.
#include <type_traits>

#include "fwd_d128.h"

namespace ra {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // queries per workgroup
constexpr int kBN = 64;           // keys per tile

template <typename T, int D, bool kSeg>
__global__ __launch_bounds__(kThreads) void fwd_step_kernel(FwdArgs a) {
  using M = Mfma<T>;
  constexpr int KPL = M::KPL;
  constexpr int E = 16 / sizeof(T);              // elements per 16-byte chunk
  constexpr int KPAD = 16 / sizeof(T);           // K row padding (16 bytes)
  constexpr int VPAD = 16 / sizeof(T);           // V^T row padding (16 bytes)
  constexpr int KP = D + KPAD;                   // K tile row pitch (elements)
  constexpr int VP = kBN + VPAD;                 // V^T tile row pitch (elements)
  constexpr int QSTEPS = D / (2 * KPL);          // MFMAs per 32x32 score block
  constexpr int PSTEPS = 16 / KPL;               // MFMAs per 32-key block of P.V
  constexpr int DB = D / 32;                     // 32-row blocks of O^T
  constexpr int KCH = kBN * D / E;               // 16-byte chunks of a K tile
  constexpr int VUNITS = (kBN / 2) * (D / E);    // (key pair, chunk) units of a V tile
  static_assert(KCH % kThreads == 0 && VUNITS % kThreads == 0, "tile/threads mismatch");
  constexpr int KLD = KCH / kThreads;
  constexpr int VLD = VUNITS / kThreads;

  __shared__ __attribute__((aligned(16))) T k_lds[kBN * KP];
  __shared__ __attribute__((aligned(16))) T vt_lds[D * VP];
  __shared__ int seg_lds[kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // Workgroup -> (b, kv head, q head within group, q tile).  Tiles of one KV head
  // are kept together on one XCD; the heaviest (latest) query tiles go first.
  const int n_wg = gridDim.x;
  const int logical = xcd_logical_id(blockIdx.x, n_wg);
  const int group = a.Hq / a.Hkv;
  int rem = logical;
  const int qt_rev = rem % a.n_qtiles;
  rem /= a.n_qtiles;
  const int hg = rem % group;
  rem /= group;
  const int g = rem % a.Hkv;
  const int b = rem / a.Hkv;
  const int qt = a.n_qtiles - 1 - qt_rev;
  const int hq = g * group + hg;

  const int q0 = qt * kBM;                        // first query of the workgroup
  const int q_last = min(q0 + kBM, a.Sq) - 1;     // last valid query of the workgroup
  const int qw = q0 + wave * 32;                  // first query of this wave
  const int qi = qw + col;                        // this lane's query
  const bool q_valid = qi < a.Sq;
  const int64_t qg = a.q_offset + qi;             // global index of this lane's query

  const T* qbase = static_cast<const T*>(a.q);
  const T* kbase = static_cast<const T*>(a.k);
  const T* vbase = static_cast<const T*>(a.v);
  const int64_t q_row_stride = (int64_t)a.Hq * D;
  const int64_t kv_row_stride = (int64_t)a.Hkv * D;

  // ---- key range of this workgroup -------------------------------------------------
  int n_keys = a.Sk;
  if (a.causal) {
    const int64_t last_visible = a.q_offset + q_last - a.kv_offset;  // local key index
    n_keys = (int)max<int64_t>(0, min<int64_t>((int64_t)a.Sk, last_visible + 1));
  }
  int kt_begin = 0;
  int kt_end = (n_keys + kBN - 1) / kBN;
  int seg_q = 0, seg_q_lo = 0, seg_q_hi = 0;
  const int32_t* seg_row = nullptr;
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    seg_q_lo = seg_row[a.q_offset + q0];
    seg_q_hi = seg_row[a.q_offset + q_last];
    seg_q = q_valid ? seg_row[a.q_offset + qi] : seg_q_lo;
    // Segment ids are nondecreasing along the row, so the tiles that share a
    // segment with this query tile form one contiguous range.
    const int32_t* seg_k = seg_row + a.kv_offset;
    int first_live = kt_end, last_live = -1;
    for (int base = 0; base < kt_end; base += 64) {
      const int t = base + lane;
      bool live = false;
      if (t < kt_end) {
        const int k_first = t * kBN;
        const int k_last = min((t + 1) * kBN, a.Sk) - 1;
        live = seg_k[k_last] >= seg_q_lo && seg_k[k_first] <= seg_q_hi;
      }
      const uint64_t mask = __ballot(live);
      if (mask) {
        first_live = min(first_live, base + (int)__builtin_ctzll(mask));
        last_live = max(last_live, base + 63 - (int)__builtin_clzll(mask));
      }
    }
    kt_begin = first_live;
    kt_end = last_live + 1;
  }

  // ---- Q fragments in registers (B operand of S^T = K Q^T) -----------------------------
  typename M::frag qf[QSTEPS];
  {
    const T* qrow = qbase + ((int64_t)b * a.Sq + (q_valid ? qi : 0)) * q_row_stride + (int64_t)hq * D;
#pragma unroll
    for (int s = 0; s < QSTEPS; ++s) {
      qf[s] = M::load(qrow + s * 2 * KPL + KPL * half);
      if (!q_valid) qf[s] = typename M::frag{};
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // running max of log2-scaled scores (shared by both halves)
  float l_run = 0.0f;       // running sum of this half's 16 keys per block

  // ---- global -> register staging of one K/V tile ----------------------------------
  u32x4 kreg[KLD];
  u32x4 vreg[VLD][2];
  int sreg = 0;
  auto load_tile = [&](int kt) {
    const int k0 = kt * kBN;
#pragma unroll
    for (int r = 0; r < KLD; ++r) {
      const int c = tid + r * kThreads;
      const int key = c / (D / E), ch = c % (D / E);
      const int kj = k0 + key;
      if (kj < a.Sk)
        kreg[r] = *reinterpret_cast<const u32x4*>(kbase + ((int64_t)b * a.Sk + kj) * kv_row_stride +
                                                  (int64_t)g * D + ch * E);
      else
        kreg[r] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < VLD; ++r) {
      const int u = tid + r * kThreads;
      const int kp = u % (kBN / 2), ch = u / (kBN / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int kj = k0 + 2 * kp + e;
        if (kj < a.Sk)
          vreg[r][e] = *reinterpret_cast<const u32x4*>(vbase + ((int64_t)b * a.Sk + kj) * kv_row_stride +
                                                       (int64_t)g * D + ch * E);
        else
          vreg[r][e] = u32x4{0, 0, 0, 0};
      }
    }
    if constexpr (kSeg) {
      if (tid < kBN) {
        const int kj = k0 + tid;
        sreg = kj < a.Sk ? seg_row[a.kv_offset + kj] : INT32_MIN;
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < KLD; ++r) {
      const int c = tid + r * kThreads;
      const int key = c / (D / E), ch = c % (D / E);
      *reinterpret_cast<u32x4*>(&k_lds[key * KP + ch * E]) = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < VLD; ++r) {
      const int u = tid + r * kThreads;
      const int kp = u % (kBN / 2), ch = u / (kBN / 2);
      if constexpr (sizeof(T) == 2) {
        // 8 d-values of keys 2kp and 2kp+1 -> 8 rows of V^T, one dword (key pair) each.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t x0 = vreg[r][0][j], x1 = vreg[r][1][j];
          const uint32_t lo = (x0 & 0xFFFFu) | (x1 << 16);          // d = 2j
          const uint32_t hi = (x0 >> 16) | (x1 & 0xFFFF0000u);      // d = 2j+1
          *reinterpret_cast<uint32_t*>(&vt_lds[(ch * E + 2 * j) * VP + 2 * kp]) = lo;
          *reinterpret_cast<uint32_t*>(&vt_lds[(ch * E + 2 * j + 1) * VP + 2 * kp]) = hi;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x2 pr = {u32_as_f32(vreg[r][0][j]), u32_as_f32(vreg[r][1][j])};
          *reinterpret_cast<f32x2*>(&vt_lds[(ch * E + j) * VP + 2 * kp]) = pr;
        }
      }
    }
    if constexpr (kSeg) {
      if (tid < kBN) seg_lds[tid] = sreg;
    }
  };

  if (kt_begin < kt_end) load_tile(kt_begin);

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (kt + 1 < kt_end) load_tile(kt + 1);  // overlaps with the math below

    const int k0 = kt * kBN;
    // Does this wave need per-element masking on this tile?  (wave-uniform)
    bool partial = (k0 + kBN > a.Sk);
    if (a.causal) partial |= (a.kv_offset + k0 + kBN - 1 > a.q_offset + qw);
    if constexpr (kSeg) partial = true;  // element test is cheap next to the tile's MFMAs

    auto tile = [&](auto mask_tag) {
      constexpr bool kMask = decltype(mask_tag)::value;
      // S^T for two 32-key blocks; the 16-byte K operands are fetched as a batch.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const T* krow = &k_lds[(32 * kb + key_of_row(col)) * KP + KPL * half];
        typename M::frag kf[QSTEPS];
#pragma unroll
        for (int s = 0; s < QSTEPS; ++s) kf[s] = M::load(krow + s * 2 * KPL);
        sacc[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < QSTEPS; ++s) sacc[kb] = M::mma(kf[s], qf[s], sacc[kb]);
      }

      // Row max of the raw scores (the scale is positive, so it commutes with max).
      float rmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float sv = sacc[kb][i];
          if constexpr (kMask) {
            const int kl = 32 * kb + 16 * half + i;  // key within the tile
            const int kj = k0 + kl;
            bool vis = kj < a.Sk;
            if (a.causal) vis = vis && (a.kv_offset + kj <= qg);
            if constexpr (kSeg) vis = vis && (seg_lds[kl] == seg_q);
            sv = vis ? sv : -INFINITY;
            sacc[kb][i] = sv;
          }
          rmax = fmaxf(rmax, sv);
        }
      }
      rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
      const float tmax = rmax * a.scale_log2;
      // Lazy rescaling: the running max only moves when a row's max grows by more
      // than kFwdSlack (log2 units), so P stays <= 2^kFwdSlack and most tiles skip the
      // rescale of O entirely.  Both halves of a row see the same tmax and m_run.
      const bool grow = tmax > m_run + kFwdSlack;
      if (__ballot(grow)) {
        const float m_new = grow ? tmax : m_run;
        const float alpha = grow ? exp2_fast(m_run - m_new) : 1.0f;  // 0 when m_run = -inf
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        m_run = m_new;
      }
      const float neg_m = (m_run == -INFINITY) ? 0.0f : -m_run;

      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2_fast(__builtin_fmaf(sacc[kb][i], a.scale_log2, neg_m));
          sacc[kb][i] = p;
          psum += p;
        }
      }
      l_run += psum;

      // O^T += V^T P^T.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[i] = sacc[kb][i];
        typename M::frag vf[PSTEPS][DB];
#pragma unroll
        for (int m = 0; m < PSTEPS; ++m)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            vf[m][db] = M::load(&vt_lds[(32 * db + col) * VP + 32 * kb + 16 * half + KPL * m]);
#pragma unroll
        for (int m = 0; m < PSTEPS; ++m) {
          const typename M::frag pf = M::pack(&pv[m * KPL]);
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] = M::mma(vf[m][db], pf, oacc[db]);
        }
      }
    };
    if (partial)
      tile(BoolTag<true>{});
    else
      tile(BoolTag<false>{});
  }

  // ---- epilogue ---------------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool live = l_tot != 0.0f;  // l_tot >= 0; NaN (from NaN inputs) stays live and propagates
  const float inv = live ? 1.0f / l_tot : 0.0f;
  if (q_valid) fwd_epilogue<DB>(a, oacc, inv, live ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY, b, hq, qi, half);
}


// ------------------------------------------------------------------------------------
// bf16, head_dim 128: the hot shape.  One workgroup = 4 or 8 waves x 32 queries of
// one query head.  K and V tiles of 32
// keys are copied global -> LDS (swizzled, row-major) without staging registers
// into two rings of three slots, K three
// tiles and V two tiles ahead of their use, so a copy has two steps to land.  V^T
// operands come from transposing LDS reads.  The scores of tile t+1 are issued
// before the softmax of tile t, so the matrix cores work while the vector ALUs do
// the softmax.
// ------------------------------------------------------------------------------------

// NW = 4 or 8 waves (x 32 queries) per workgroup: with 8, two waves per SIMD share
// each K/V tile copy (half the tile traffic per query); 4 keeps more workgroups for
// small grids.
template <bool kSeg, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_step_d128_kernel(FwdArgs a) {
  static_assert(NW == 4 || NW == 8, "tile blocks of 1 KiB split evenly over the waves");
  // 8-wave workgroups take 64-key tiles (two 32-key blocks): half the barriers,
  // copies and per-tile reductions per key.
  constexpr int KB = NW == 8 ? 2 : 1;  // 32-key blocks per tile
  constexpr int D = 128, BN = 32 * KB, BM = 32 * NW;
  static_assert(!(kSeg && KB > 1), "packed rows use 32-key tiles");
  constexpr int kD128Blocks = BN / 4 / NW;  // 1 KiB blocks (4 rows) of a tile copied by each wave
  // Each slot its own array, so the compiler can tell the copies in flight from
  // the tiles being read.
  __shared__ __attribute__((aligned(1024))) __bf16 ks0[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 ks1[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 ks2[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 vs0[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 vs1[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 vs2[BN * D];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int group = a.Hq / a.Hkv;
  int rem = logical;
  const int qt_rev = rem % a.n_qtiles;
  rem /= a.n_qtiles;
  const int hg = rem % group;
  rem /= group;
  const int g = rem % a.Hkv;
  const int b = rem / a.Hkv;
  const int qt = a.n_qtiles - 1 - qt_rev;
  const int hq = g * group + hg;

  const int q0 = qt * BM;
  const int q_last = min(q0 + BM, a.Sq) - 1;
  const int qw = q0 + 32 * wave;
  const int qi = qw + col;
  const bool qv = qi < a.Sq;

  const int64_t q_rs = (int64_t)a.Hq * D;
  const int kv_rb = a.Hkv * D * 2;  // bytes between consecutive keys
  const char* kbase = static_cast<const char*>(a.k) + ((int64_t)b * a.Sk * a.Hkv + g) * (D * 2);
  const char* vbase = static_cast<const char*>(a.v) + ((int64_t)b * a.Sk * a.Hkv + g) * (D * 2);

  // Key tiles this workgroup visits.
  int n_keys = a.Sk;
  if (a.causal) {
    const int64_t last_visible = a.q_offset + q_last - a.kv_offset;
    n_keys = (int)max<int64_t>(0, min<int64_t>((int64_t)a.Sk, last_visible + 1));
  }
  int kt_begin = 0, kt_end = (n_keys + BN - 1) / BN;
  const int32_t* seg_row = nullptr;
  int seg_q = 0;
  int seg_w_lo = 0, seg_w_hi = 0;  // segment ids of the wave's first and last query
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    const int lo = seg_row[a.q_offset + q0], hi = seg_row[a.q_offset + q_last];
    seg_q = qv ? seg_row[a.q_offset + qi] : lo;
    seg_w_lo = seg_row[a.q_offset + min(qw, a.Sq - 1)];
    seg_w_hi = seg_row[a.q_offset + min(qw + 32, a.Sq) - 1];
    const int32_t* seg_k = seg_row + a.kv_offset;
    int first_live = kt_end, last_live = -1;
    for (int base = 0; base < kt_end; base += 64) {
      const int t = base + lane;
      bool live = false;
      if (t < kt_end) {
        const int k_first = t * BN;
        const int k_last = min((t + 1) * BN, a.Sk) - 1;
        live = seg_k[k_last] >= lo && seg_k[k_first] <= hi;
      }
      const uint64_t mask = __ballot(live);
      if (mask) {
        first_live = min(first_live, base + (int)__builtin_ctzll(mask));
        last_live = max(last_live, base + 63 - (int)__builtin_clzll(mask));
      }
    }
    kt_begin = first_live;
    kt_end = max(first_live, last_live + 1);
  }
  // Merging a step without a live tile into the running result changes nothing:
  // unless the merged output is also converted, the workgroup is done.
  if (kt_begin >= kt_end && a.merge && a.out_kind == 0) return;

  // Q operands (B of S^T = K Q^T).
  bf16x8 qf[8];
  {
    const __bf16* qrow = static_cast<const __bf16*>(a.q) + ((int64_t)b * a.Sq + (qv ? qi : 0)) * q_rs +
                         (int64_t)hq * D + 8 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = qv ? load_bf16x8(qrow + 16 * s) : bf16x8{};
  }

  // Causal limit: key k0 + 16*half + i is visible iff i <= causal_lim - k0.  Clamped
  // to +-2^30 (k0 <= 2^30), which keeps the test exact without 64-bit arithmetic.
  // wave_last_visible: the last chunk key the wave's first query sees (same clamp).
  const int wave_last_visible =
      (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, a.q_offset + qw - a.kv_offset));
  int causal_lim = 1 << 30;
  if (a.causal) {
    const int64_t c = a.q_offset + qi - a.kv_offset - 16 * half;
    causal_lim = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, c));
  }

  // Copies: 32 rows x 256 bytes per tile = 8 blocks of 1 KiB, 8 / waves per wave; lane
  // l of a block writes 16 bytes at 16*l, so it fetches the global chunk that the
  // swizzle puts there.  Raw buffer loads with a per-tile descriptor whose range
  // ends at the chunk's last key: rows past it read as zeros (and are masked).
  uint32_t coff[kD128Blocks];
#pragma unroll
  for (int r = 0; r < kD128Blocks; ++r) {
    const int row = (kD128Blocks * wave + r) * 4 + (lane >> 4);
    coff[r] = (uint32_t)(row * kv_rb + ((lane & 15) ^ swz(row)) * 16);
  }
  auto copy_tile = [&](const char* base, int t, __bf16* dst) {
    const int k0 = t * BN;
    // Through the tile's last valid key row; < 2^31 since kv_rb <= 4096 * 256.
    const int bytes = (min(a.Sk - k0, BN) - 1) * kv_rb + D * 2;
    const buffer_rsrc rs = make_rsrc32(base + (int64_t)k0 * kv_rb, bytes);
    char* d = reinterpret_cast<char*>(dst) + kD128Blocks * wave * 1024;
#pragma unroll
    for (int r = 0; r < kD128Blocks; ++r) buffer_load_lds16(rs, d + r * 1024, coff[r]);
  };
  constexpr int kCopiesPerTile = kD128Blocks;  // per wave and tensor

  // LDS operand offsets.  K (A of S^T): row key_of_row(col), 16-byte chunk 2s+half,
  // i.e. kA ^ (s << 5).  V^T (A of O^T += V^T P^T) via transposing reads of rows
  // 16*half + 8m + k (+4) at columns 32*db + ...: per-lane bases B0 (rows +k) and B1
  // (rows +4+k); column block db selects bits 6-7 by XOR, m adds 2048 bytes.
  const int kA = row_read_base(lane);
  const TrBases trb = tr_bases(lane);
  const int vB0 = trb.b0, vB1 = trb.b1;
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  auto tr_read = [](const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  struct Scores {
    f32x16 s[KB];
  };
  auto qk = [&](const __bf16* kt) {
    const char* base = reinterpret_cast<const char*>(kt);
    bf16x8 kf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = load_bf16x8(base + (kA ^ (s << 5)));
    __builtin_amdgcn_sched_barrier(0);  // all eight reads in flight before the first MFMA
    Scores acc;
    acc.s[0] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc.s[0] = mfma_bf16(kf[s], qf[s], acc.s[0]);
    if constexpr (KB > 1) {
      // Block 1 (keys 32..63, 8 KiB further): its operands reuse the registers as
      // block 0's MFMAs release them.
#pragma unroll
      for (int s = 0; s < 8; ++s) kf[s] = load_bf16x8(base + 8192 + (kA ^ (s << 5)));
      acc.s[1] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) acc.s[1] = mfma_bf16(kf[s], qf[s], acc.s[1]);
    }
    return acc;
  };

  // Softmax of tile t's scores and O^T += V^T P^T.
  auto consume = [&](Scores sc, const __bf16* vt, int t) {
    const int k0 = t * BN;
    bool partial = (k0 + BN > a.Sk);
    if (a.causal) partial |= (k0 + BN - 1 > wave_last_visible);
    if constexpr (kSeg) {
      // Segment ids are nondecreasing: the block needs the segment test only if the
      // wave's queries and the tile's keys are not all in one and the same segment.
      const int sk_lo = seg_row[a.kv_offset + k0];
      const int sk_hi = seg_row[a.kv_offset + min(k0 + BN, a.Sk) - 1];
      partial |= !(sk_lo == sk_hi && sk_lo == seg_w_lo && seg_w_lo == seg_w_hi);
    }
    if (partial) {  // one wave-uniform branch around the element mask
      // Register i of half h of block kb holds key k0 + 32kb + 16h + i.
      const int lim = min(a.causal ? causal_lim - k0 : (1 << 30), a.Sk - 1 - k0 - 16 * half);
      if constexpr (kSeg) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // Wave-uniform addresses (scalar loads), clamped into the chunk.
          const int s_lo = seg_row[a.kv_offset + min(k0 + i, a.Sk - 1)];
          const int s_hi = seg_row[a.kv_offset + min(k0 + 16 + i, a.Sk - 1)];
          const bool vis = (i <= lim) & ((half ? s_hi : s_lo) == seg_q);
          sc.s[0][i] = vis ? sc.s[0][i] : -INFINITY;
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sc.s[kb][i] = (i + 32 * kb <= lim) ? sc.s[kb][i] : -INFINITY;
      }
    }

    // Row max and (below) row sum as trees of independent operations, so that the
    // vector instructions between two MFMAs do not wait on one another.
    auto max3 = [](float x, float y, float z) { return fmaxf(fmaxf(x, y), z); };
    float r = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const f32x16& c = sc.s[kb];
      r = fmaxf(r, fmaxf(max3(max3(c[0], c[1], c[2]), max3(c[3], c[4], c[5]), max3(c[6], c[7], c[8])),
                         max3(max3(c[9], c[10], c[11]), max3(c[12], c[13], c[14]), c[15])));
    }
    const float tmax = half_max(r) * a.scale_log2;
    // Lazy rescaling: the running max only moves when a row's max grows by more
    // than kFwdSlack (log2 units), so P stays <= 2^kFwdSlack and most tiles skip the
    // rescale of O entirely.  Both halves of a row see the same tmax and m_run.
    const bool grow = tmax > m_run + kFwdSlack;
    if (__ballot(grow)) {
      const float al = grow ? exp2_fast(m_run - tmax) : 1.0f;  // 0 when m_run = -inf
      if (grow) m_run = tmax;
      l_run *= al;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= al;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.0f : -m_run;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = exp2_fast(__builtin_fmaf(sc.s[kb][i], a.scale_log2, neg_m));
      float ps4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ps4[j] = (p[4 * j] + p[4 * j + 1]) + (p[4 * j + 2] + p[4 * j + 3]);
      l_run += (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
      const bf16x8 pf0 = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      const bf16x8 pf1 = to_bf16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);

      // O^T += V^T P^T: register 8m+j of half h holds key 32kb + 16h + 8m + j.
      const char* vb = reinterpret_cast<const char*>(vt) + 8192 * kb;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8 vf[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x4_t x0 = tr_read(vb + (vB0 ^ (db << 6)) + 2048 * m);
          const bf16x4_t x1 = tr_read(vb + (vB1 ^ (db << 6)) + 2048 * m);
          vf[db] = bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        }
        // Two waves share each SIMD.  With 4-wave workgroups (two per CU) the products
        // go out at raised priority, ahead of the other wave's softmax instructions
        // (8K chunk step -2 to -7 %); with 8-wave workgroups each group of four stays
        // together in the schedule (64K chunk step -1 %), where the priority gained
        // nothing.
        if constexpr (NW == 4)
          __builtin_amdgcn_s_setprio(1);
        else
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] = mfma_bf16(vf[db], m ? pf1 : pf0, oacc[db]);
        if constexpr (NW == 4)
          __builtin_amdgcn_s_setprio(0);
        else
          __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // One step: K(t+1) and V(t) must have landed (copied two steps ago; this wave's
  // copies from the previous step may stay in flight), then every wave's copies are
  // published with a bare s_barrier (a workgroup fence would also drain the copies
  // in flight; the empty asm statements keep LDS accesses on their side of it).
  // The slots freed by that barrier receive K(t+3) and V(t+2).
  // `steady`: the caller guarantees t + 3 < kt_end, so the waits and copies need no
  // tests (the bulk of the loop); the last steps go through the general form.
  Scores s_next{};
  auto step = [&](auto steady_tag, int t, const __bf16* kq, const __bf16* vc, __bf16* kn, __bf16* vn) {
    constexpr bool kSteady = decltype(steady_tag)::value;
    if (kSteady || t + 2 < kt_end)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCopiesPerTile));  // both tensors of the last step in flight
    else if (t + 1 < kt_end)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCopiesPerTile));  // its V copies in flight
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kSteady || t + 3 < kt_end) copy_tile(kbase, t + 3, kn);
    if (kSteady || t + 2 < kt_end) copy_tile(vbase, t + 2, vn);
    // Scores of tile t+1 (on the last step the slot is stale and the result unused).
    const Scores sc = s_next;
    s_next = qk(kq);
    consume(sc, vc, t);
  };

  if (kt_begin < kt_end) {
    const int t = kt_begin;
    copy_tile(kbase, t, ks0);
    copy_tile(vbase, t, vs0);
    if (t + 1 < kt_end) {
      copy_tile(kbase, t + 1, ks1);
      copy_tile(vbase, t + 1, vs1);
    }
    if (t + 2 < kt_end) copy_tile(kbase, t + 2, ks2);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    s_next = qk(ks0);
  }
  // Slots: K(j) in ks[(j - kt_begin) % 3], V(j) in vs[(j - kt_begin) % 3].  Six
  // steps per iteration, so the two score register sets alternate without copies;
  // every exit leaves through a break, so only O, m and l are live there.
  // The steady loop runs while all six of its steps have t + 3 < kt_end; the rest
  // (at most 8 steps) runs through the general steps, which continue the same slot
  // rotation (both loops advance t by 6).
  if (kt_begin < kt_end) {
    const BoolTag<true> st;
    const BoolTag<false> gen;
    int t = kt_begin;
    for (; t + 8 < kt_end; t += 6) {
      step(st, t, ks1, vs0, ks0, vs2);
      step(st, t + 1, ks2, vs1, ks1, vs0);
      step(st, t + 2, ks0, vs2, ks2, vs1);
      step(st, t + 3, ks1, vs0, ks0, vs2);
      step(st, t + 4, ks2, vs1, ks1, vs0);
      step(st, t + 5, ks0, vs2, ks2, vs1);
    }
    for (;; t += 6) {
      step(gen, t, ks1, vs0, ks0, vs2);
      if (t + 1 >= kt_end) break;
      step(gen, t + 1, ks2, vs1, ks1, vs0);
      if (t + 2 >= kt_end) break;
      step(gen, t + 2, ks0, vs2, ks2, vs1);
      if (t + 3 >= kt_end) break;
      step(gen, t + 3, ks1, vs0, ks0, vs2);
      if (t + 4 >= kt_end) break;
      step(gen, t + 4, ks2, vs1, ks1, vs0);
      if (t + 5 >= kt_end) break;
      step(gen, t + 5, ks0, vs2, ks2, vs1);
      if (t + 6 >= kt_end) break;
    }
  }

  const float l_tot = half_sum(l_run);
  const bool live = l_tot != 0.0f;  // l_tot >= 0; NaN (from NaN inputs) stays live and propagates
  const float inv = live ? 1.0f / l_tot : 0.0f;
  if (qv) fwd_epilogue<4>(a, oacc, inv, live ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY, b, hq, qi, half);
}

template <typename T, int D>
ra_status launch_fwd(const FwdArgs& args, hipStream_t stream) {
  const int64_t n_wg = (int64_t)args.B * args.Hq * args.n_qtiles;
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  if constexpr (std::is_same<T, __bf16>::value && D == 128) {
    // Packed rows: 64 queries per wave (four query heads of a GQA group per
    // workgroup) when that grid gives every CU (256 on MI355X) two workgroups: each
    // K/V operand read feeds two MFMAs.  On unpacked rows the 8-wave kernel below,
    // with two waves per SIMD to hide the softmax, is as fast or faster.
    if (args.seg != nullptr && fwd64_d128_workgroups(args) >= 2 * 256) return launch_fwd64_d128(args, stream);
    // 8-wave workgroups when the grid still gives every CU (256 on MI355X) two of
    // them and no segment test runs (packed rows keep the finer 128-query tiles):
    // 4096-query chunks -2 %; with one per CU (2048-query chunks) the diagonal step
    // was 5 % slower.
    const int64_t n8 = (int64_t)args.B * args.Hq * ((args.Sq + 255) / 256);
    const bool wide = args.seg == nullptr && n8 >= 2 * 256;
    FwdArgs a2 = args;
    a2.n_qtiles = (args.Sq + (wide ? 255 : 127)) / (wide ? 256 : 128);
    const unsigned n2 = (unsigned)((int64_t)args.B * args.Hq * a2.n_qtiles);
    if (args.seg != nullptr)
      hipLaunchKernelGGL((fwd_step_d128_kernel<true, 4>), dim3(n2), dim3(256), 0, stream, a2);
    else if (wide)
      hipLaunchKernelGGL((fwd_step_d128_kernel<false, 8>), dim3(n2), dim3(512), 0, stream, a2);
    else
      hipLaunchKernelGGL((fwd_step_d128_kernel<false, 4>), dim3(n2), dim3(256), 0, stream, a2);
    return check_launch("ring_attn_fwd_step");
  }
  if (args.seg != nullptr)
    hipLaunchKernelGGL((fwd_step_kernel<T, D, true>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((fwd_step_kernel<T, D, false>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream, args);
  return check_launch("ring_attn_fwd_step");
}

}  // namespace
}  // namespace ra

namespace ra {
namespace {

ra_status fwd_entry(const ra_shape* s, const void* q, const void* k, const void* v, const int32_t* seg_ids,
                    int64_t seg_len, float* o, float* lse, int merge, void* o_out, int out_kind,
                    hipStream_t hs) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.seg = seg_ids;
  a.seg_len = seg_len;
  a.o = o;
  a.lse = lse;
  a.B = s->batch;
  a.Sq = s->q_len;
  a.Sk = s->kv_len;
  a.Hq = s->heads_q;
  a.Hkv = s->heads_kv;
  a.q_offset = s->q_offset;
  a.kv_offset = s->kv_offset;
  a.causal = s->causal;
  a.scale_log2 = s->softmax_scale * kLog2e;
  a.n_qtiles = (s->q_len + kBM - 1) / kBM;
  a.merge = merge;
  a.o_out = o_out;
  a.out_kind = out_kind;
  if (s->dtype == RA_DTYPE_BF16) {
    if (s->head_dim == 128) return launch_fwd<__bf16, 128>(a, hs);
    return launch_fwd<__bf16, 64>(a, hs);
  }
  if (s->head_dim == 128) return launch_fwd<float, 128>(a, hs);
  return launch_fwd<float, 64>(a, hs);
}

}  // namespace
}  // namespace ra

extern "C" ra_status ring_attn_fwd_step(const ra_shape* s, const void* q, const void* k, const void* v,
                                        const int32_t* seg_ids, int64_t seg_len, float* o_step,
                                        float* lse_step, void* stream) {
  using namespace ra;
  ra_status st = validate_step(s, seg_ids, seg_len);
  if (st != RA_OK) return st;
  if (!q || !k || !v || !o_step || !lse_step)
    return fail(RA_ERR_INVALID_ARGUMENT, "q, k, v, o_step and lse_step must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_step) || !aligned16(lse_step))
    return fail(RA_ERR_INVALID_ARGUMENT, "q, k, v, o_step and lse_step must be 16-byte aligned");
  return fwd_entry(s, q, k, v, seg_ids, seg_len, o_step, lse_step, 0, nullptr, 0, static_cast<hipStream_t>(stream));
}

extern "C" ra_status ring_attn_fwd_step_merge(const ra_shape* s, const void* q, const void* k, const void* v,
                                              const int32_t* seg_ids, int64_t seg_len, float* o_acc,
                                              float* lse_acc, void* o_out, int32_t out_dtype, void* stream) {
  using namespace ra;
  ra_status st = validate_step(s, seg_ids, seg_len);
  if (st != RA_OK) return st;
  if (!q || !k || !v || !o_acc || !lse_acc)
    return fail(RA_ERR_INVALID_ARGUMENT, "q, k, v, o_acc and lse_acc must be non-NULL");
  if (o_out && out_dtype != RA_DTYPE_F32 && out_dtype != RA_DTYPE_BF16)
    return fail(RA_ERR_UNSUPPORTED, "out_dtype %d is not supported", out_dtype);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_acc) || !aligned16(lse_acc) ||
      (o_out && ((uintptr_t)o_out & 7u)))
    return fail(RA_ERR_INVALID_ARGUMENT, "misaligned pointer (16 bytes; o_out 8 bytes)");
  const int out_kind = o_out == nullptr ? 0 : (out_dtype == RA_DTYPE_F32 ? 1 : 2);
  return fwd_entry(s, q, k, v, seg_ids, seg_len, o_acc, lse_acc, 1, o_out, out_kind,
                   static_cast<hipStream_t>(stream));
}
