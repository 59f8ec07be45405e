// ring_attn_fwd_step for the hot shape (bf16, head_dim 128) on packed rows, wide
// grids: each wave owns 64 queries (two 32-query MFMA blocks), so every K and V
// operand it reads from LDS feeds two MFMAs -- half the LDS bytes per MFMA of a
// 32-query wave.
//   s_ij = scale * q_i . k_j over the visible keys of this chunk,
//   O_i = sum_j softmax_j(s_ij) v_j,  LSE_i = ln sum_j exp(s_ij)
// (axolotl docs "Sequence Parallelism", Implementation Details; aicassindra
// "Transformer math: SP math", context parallelism), the score matrix existing one
// 32x32 register tile at a time (archcrux, "sequence-parallel long-context
// attention OOM").
//
// A workgroup is 4 waves over the query heads of one KV head's GQA group (up to 4
// heads, the same 64 queries each; smaller groups stack query blocks instead), so
// every wave uses every K/V tile the workgroup stages.  Each wave keeps its
// queries' Q operands (64 AGPRs, B operands of the score MFMAs) and the O^T
// accumulators (128 AGPRs) in registers for the whole launch; K/V tiles of 32 keys
// come through a ring of four LDS slots filled by raw buffer loads.  Per tile and
// wave: 16 MFMAs for S^T = K Q^T and 16 for O^T += V^T P^T against 16 KiB of LDS
// operand reads.
//
// The tile loop is software-pipelined: iteration t runs
//   phase 1: S^T of tile t+1          | softmax of tile t (mask, row max, lazy
//                                     |   rescale, exp2, row sum, bf16 packing,
//                                     |   a few vector instructions per MFMA)
//   phase 2: O^T += V^T P^T of tile t | the barrier that publishes tile t+2
// then the wait states the accumulators need before anything else may read them.
// The MFMAs are inline assembly (the score MFMAs read Q from AGPRs and the P.V
// MFMAs accumulate in AGPRs, which the compiler does not allocate by itself);
// their hazards are kept by the schedule: each result is first read by vector
// instructions in a later phase, behind explicit wait states.
#include <type_traits>

#include "fwd_d128.h"

namespace ra {
namespace {

constexpr int kD = 128;
constexpr int kNW = 4;   // waves per workgroup
constexpr int kQW = 64;  // queries per wave
constexpr int kKT = 32;  // keys per staged tile

// Heads per workgroup: the largest of 4, 2, 1 that divides the GQA group.
__host__ __device__ __forceinline__ int fwd64_heads_per_wg(int group) {
  return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
}

template <bool kSeg>
__global__ __launch_bounds__(64 * kNW) void fwd64_d128_kernel(FwdArgs a) {
  // Four K and four V tile slots, each its own array (the compiler can tell the
  // slots being read from the slots still being filled).
  __shared__ __attribute__((aligned(1024))) __bf16 ks0[kKT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ks1[kKT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ks2[kKT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ks3[kKT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 vs0[kKT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 vs1[kKT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 vs2[kKT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 vs3[kKT * kD];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int group = a.Hq / a.Hkv;
  const int hpw = fwd64_heads_per_wg(group);  // heads per workgroup
  const int qpw = kNW / hpw;                  // 64-query blocks per workgroup
  const int n_hset = group / hpw;
  int rem = logical;
  const int qt_rev = rem % a.n_qtiles;
  rem /= a.n_qtiles;
  const int hset = rem % n_hset;
  rem /= n_hset;
  const int g = rem % a.Hkv;
  const int b = rem / a.Hkv;
  const int qt = a.n_qtiles - 1 - qt_rev;  // latest (heaviest causal) query tiles first
  const int hq = g * group + hset * hpw + wave % hpw;
  const int q_wg = qt * kQW * qpw;           // the workgroup's first query
  const int qw = q_wg + kQW * (wave / hpw);  // the wave's first query
  const int q_wg_last = min(q_wg + kQW * qpw, a.Sq) - 1;

  const int64_t q_rs = (int64_t)a.Hq * kD;
  const int kv_rb = a.Hkv * kD * 2;  // bytes between consecutive keys
  const char* kbase = static_cast<const char*>(a.k) + ((int64_t)b * a.Sk * a.Hkv + g) * (kD * 2);
  const char* vbase = static_cast<const char*>(a.v) + ((int64_t)b * a.Sk * a.Hkv + g) * (kD * 2);

  // Key tiles of the workgroup: every key some of its queries may see.
  int n_keys = a.Sk;
  if (a.causal) {
    const int64_t last_visible = a.q_offset + q_wg_last - a.kv_offset;
    n_keys = (int)max<int64_t>(0, min<int64_t>((int64_t)a.Sk, last_visible + 1));
  }
  int kt_begin = 0, kt_end = (n_keys + kKT - 1) / kKT;
  const int32_t* seg_row = nullptr;
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    const int lo = seg_row[a.q_offset + q_wg], hi = seg_row[a.q_offset + q_wg_last];
    int sb, se;
    seg_tile_range(seg_row + a.kv_offset, a.Sk, kKT, 0, kt_end, lo, hi, sb, se);
    kt_begin = sb;
    kt_end = max(sb, se);
  }
  const int n_t = kt_end - kt_begin;
  // A step without a live tile: merged into the running result it changes nothing
  // (the workgroup is done unless the merged output is also converted); alone it is
  // O = 0, LSE = -inf.  Either way no Q is loaded and no tile is visited.
  if (n_t <= 0) {
    if (a.merge && a.out_kind == 0) return;
    const f32x16 zero[4] = {};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qi = qw + 32 * qb + col;
      if (qi < a.Sq) fwd_epilogue<4>(a, zero, 0.0f, -INFINITY, b, hq, qi, half);
    }
    return;
  }

  // Per lane and query block qb: the query q = qw + 32 qb + col, its Q row (B
  // operands; lane = query column, k-slots = d), and the chunk keys it sees,
  // [vlo, vhi] shifted by the lane's half (causal rule, chunk end, segment span);
  // a query past the shard sees nothing.
  bf16x8 qf[2][8];
  int vlo[2], vhi[2];
  SegSpans wsp{};  // the segments of the wave's first and last query
  if constexpr (kSeg)
    wsp = seg_spans_wave(seg_row, a.seg_len, a.q_offset + min(qw, a.Sq - 1), a.q_offset + min(qw + kQW, a.Sq) - 1);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + 32 * qb + col;
    const bool qv = qi < a.Sq;
    const __bf16* qp = static_cast<const __bf16*>(a.q) + ((int64_t)b * a.Sq + (qv ? qi : 0)) * q_rs +
                       (int64_t)hq * kD + 8 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[qb][s] = qv ? load_bf16x8(qp + 16 * s) : bf16x8{};
    const int64_t qg = a.q_offset + qi;
    int64_t lo = 0, hi = a.Sk - 1;  // chunk key indices
    if (a.causal) hi = min<int64_t>(hi, qg - a.kv_offset);
    if constexpr (kSeg) {
      if (qv) {
        int64_t s_lo, s_hi;
        seg_span_lane(seg_row, a.seg_len, wsp, seg_row[qg], s_lo, s_hi);
        lo = max<int64_t>(lo, s_lo - a.kv_offset);
        hi = min<int64_t>(hi, s_hi - 1 - a.kv_offset);
      }
    }
    auto clamp30 = [](int64_t x) { return (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, x)); };
    vlo[qb] = clamp30(lo - 16 * half);
    vhi[qb] = qv ? clamp30(hi - 16 * half) : -(1 << 30);
  }
  // Pin Q to AGPRs (its only uses are the inline-asm score MFMAs).
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" : "+a"(qf[qb][s]));

  // Tiles that may hold an invisible element for some lane of the wave run the
  // masked body: [m_first, kt_end) (the causal diagonal, the chunk's ragged end,
  // for packed rows the end of the wave's sample) and, for packed rows, the tiles
  // before the first one inside the wave's sample, [kt_begin, kt_begin + n_pre).
  // Every tile does if the wave's queries run past the shard or, packed, span two
  // samples.
  int m_first = kt_begin, n_pre = 0;
  bool one_row_range = qw + kQW <= a.Sq;
  int64_t full_lo = 0, full_hi = a.Sk;  // chunk keys that every query of the wave may share a sample with
  if constexpr (kSeg) {
    one_row_range = one_row_range && wsp.s0 == wsp.s1;
    full_lo = wsp.lo0 - a.kv_offset;
    full_hi = wsp.hi0 - a.kv_offset;
  }
  if (one_row_range) {
    int64_t first_hidden = min<int64_t>(a.Sk, full_hi);  // first chunk key some query may not see
    if (a.causal) first_hidden = min<int64_t>(first_hidden, a.q_offset + qw - a.kv_offset + 1);
    int64_t mt = max<int64_t>(0, first_hidden) / kKT;  // tile holding it
    if (a.Sk % kKT != 0) mt = min<int64_t>(mt, a.Sk / kKT);
    m_first = (int)max<int64_t>(kt_begin, min<int64_t>(kt_end, mt));
    const int64_t first_full = (max<int64_t>(0, full_lo) + kKT - 1) / kKT;  // first tile inside the sample
    n_pre = (int)max<int64_t>(0, min<int64_t>(n_t, first_full - kt_begin));
  }

  f32x16 oacc[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[qb][db] = f32x16{};
  float m_run[2] = {-INFINITY, -INFINITY};  // running max of log2-scaled scores, per row
  float l_run[2] = {0.0f, 0.0f};            // running sum of this half's keys, per row

  // Copies of tile u (32 keys) into a slot: 32 rows x 256 bytes per tensor = 8
  // blocks of 1 KiB; wave w copies blocks 2w and 2w+1 of K and of V (lane l of a
  // block writes 16 bytes at 16 l and fetches the global chunk the swizzle puts
  // there).  Per-tile descriptors end at the chunk's last key: rows past it read as
  // zeros (and are masked).
  uint32_t coff[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = (2 * wave + r) * 4 + (lane >> 4);
    coff[r] = (uint32_t)(row * kv_rb + ((lane & 15) ^ swz(row)) * 16);
  }
  auto issue = [&](int u, __bf16* kdst, __bf16* vdst) {
    const int k0 = (kt_begin + u) * kKT;
    const int bytes = (min(a.Sk - k0, kKT) - 1) * kv_rb + kD * 2;  // < 2^31: kv_rb <= 4096 * 256
    const buffer_rsrc rk = make_rsrc32(kbase + (int64_t)k0 * kv_rb, bytes);
    const buffer_rsrc rv = make_rsrc32(vbase + (int64_t)k0 * kv_rb, bytes);
    char* dk = reinterpret_cast<char*>(kdst) + 2 * wave * 1024;
    char* dv = reinterpret_cast<char*>(vdst) + 2 * wave * 1024;
#pragma unroll
    for (int r = 0; r < 2; ++r) buffer_load_lds16(rk, dk + r * 1024, coff[r]);
#pragma unroll
    for (int r = 0; r < 2; ++r) buffer_load_lds16(rv, dv + r * 1024, coff[r]);
  };
  constexpr int kCopiesPerTile = 4;

  // LDS operand offsets (ra_device.h): K rows (A of S^T = K Q^T) at rA ^ (c << 5);
  // V^T (A of O^T += V^T P^T) by transposing reads at (tB0|tB1 ^ (db << 6)) + 2048 m.
  // Recomputed next to each read from per-tile opaque copies of the bases (no
  // hoisted XOR results held in registers).
  const int rA = row_read_base(lane);
  const TrBases trb = tr_bases(lane);
  int rA_t = rA, tB0_t = trb.b0, tB1_t = trb.b1;
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  auto tr_read = [](const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
  };
  auto tr_op = [&](const char* base, int j) {  // operand j = 4m + db
    const int m = j >> 2, db = j & 3;
    const int o0 = (tB0_t ^ (db << 6)) + 2048 * m, o1 = (tB1_t ^ (db << 6)) + 2048 * m;
    const bf16x4_t x0 = tr_read(base + o0), x1 = tr_read(base + o1);
    return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  auto row_op = [&](const char* base, int c) { return load_bf16x8(base + (rA_t ^ (c << 5))); };
  auto opaque_bases = [&] {
    rA_t = rA;
    tB0_t = trb.b0;
    tB1_t = trb.b1;
    asm volatile("" : "+v"(rA_t), "+v"(tB0_t), "+v"(tB1_t));
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  // st[u & 1][qb]: tile u's S^T (register i of half h = key k0 + 16h + i), two
  // buffers since tile t's softmax reads its scores while tile t+1's are computed.
  // pf[qb][m]: P^T of tile t packed to bf16 (keys 16h + 8m + j), B of the P.V MFMAs.
  f32x16 st[2][2];
  bf16x8 pf[2][2];

  struct Ops {
    bf16x8 f[8];
  };
  auto read_op = [&](bool tr, const char* base, Ops& o, int c) { o.f[c] = tr ? tr_op(base, c) : row_op(base, c); };

  // The S^T chain of a tile (16 MFMAs, query blocks interleaved, each K operand
  // feeds both) with `work(k)` in slot k's shadow; operand c+4 is read right after
  // the last use of operand c, operands 0..3 during the previous chain.
  auto s_chain = [&](int bf, const char* base, Ops& o, auto&& work) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int c = k >> 1, qb = k & 1;
      if (c == 0)
        mfma_vab0(st[bf][qb], o.f[0], qf[qb][0]);
      else
        mfma_vab_acc(st[bf][qb], o.f[c], qf[qb][c]);
      if (qb == 1 && c + 4 < 8) read_op(false, base, o, c + 4);
      work(k);
      fence();
    }
  };
  // O^T[qb][db] += V^T[m][db] P^T[qb][m]: 16 MFMAs (m-major, qb-minor).
  auto pv_chain = [&](const char* base, Ops& o, auto&& work) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int j = k >> 1, qb = k & 1, m = j >> 2, db = j & 3;
      mfma_acc(oacc[qb][db], o.f[j], pf[qb][m]);
      if (qb == 1 && j + 4 < 8) read_op(true, base, o, j + 4);
      work(k);
      fence();
    }
  };
  // The first four operands of the next chain, one per odd slot from slot 9 on.
  auto preload = [&](int k, bool tr, const char* base, Ops& o) {
    if (k >= 9 && (k & 1)) read_op(tr, base, o, (k - 9) >> 1);
  };

  // Softmax of query block qb of tile t (scores in st[bf][qb], first chunk key k0),
  // in three parts spread over the slots of the S^T chain.
  // Part 1: element mask (masked tiles) and the row max, scaled to log2 units.
  float tmax[2], nm[2];  // the tile's row max; minus the running max (0 if -inf)
  auto sm_max = [&](auto mask_tag, int bf, int qb, int k0) {
    constexpr bool kMask = decltype(mask_tag)::value;
    f32x16& s = st[bf][qb];
    if constexpr (kMask) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool vis = (i >= vlo[qb] - k0) & (i <= vhi[qb] - k0);
        s[i] = vis ? s[i] : -__builtin_inff();
      }
    }
    auto max3 = [](float x, float y, float z) { return fmaxf(fmaxf(x, y), z); };
    const float r = fmaxf(max3(max3(s[0], s[1], s[2]), max3(s[3], s[4], s[5]), max3(s[6], s[7], s[8])),
                          max3(max3(s[9], s[10], s[11]), max3(s[12], s[13], s[14]), s[15]));
    tmax[qb] = half_max(r) * a.scale_log2;
  };
  // Part 2: lazy rescaling -- the running max only moves when a row's max grows by
  // more than kFwdSlack (log2 units), so P stays <= 2^kFwdSlack and most tiles skip
  // the rescale of O.  Both halves of a row see the same tmax and m_run.  Reads O:
  // runs at least two MFMA slots after the last P.V MFMA.
  auto sm_rescale = [&](int qb) {
    const bool grow = tmax[qb] > m_run[qb] + kFwdSlack;
    if (__ballot(grow)) {
      const float al = grow ? exp2_fast(m_run[qb] - tmax[qb]) : 1.0f;  // 0 when m_run = -inf
      if (grow) m_run[qb] = tmax[qb];
      l_run[qb] *= al;
      // The accumulators are read here and nowhere earlier (no speculative copies
      // out of AGPRs on the path that does not rescale).
      asm volatile("" : "+a"(oacc[qb][0]), "+a"(oacc[qb][1]), "+a"(oacc[qb][2]), "+a"(oacc[qb][3]));
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[qb][db] *= al;
    }
    nm[qb] = (m_run[qb] == -INFINITY) ? 0.0f : -m_run[qb];
  };
  // Part 3: P = exp2(s * scale_log2 - m) for elements e, e+1 (in place) and their
  // share of the row sum; then the packing of keys 8m .. 8m+7.  Each result passes
  // through an empty asm statement, which keeps it in its slot: sunk next to its
  // first use, the packing would land right before the P.V MFMA that reads it,
  // which the compiler does not see as an MFMA (no wait states).
  auto sm_exp2 = [&](int bf, int qb, int e) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float y = exp2_fast(__builtin_fmaf(st[bf][qb][e + u], a.scale_log2, nm[qb]));
      asm volatile("" : "+v"(y));
      st[bf][qb][e + u] = y;
    }
    l_run[qb] += st[bf][qb][e] + st[bf][qb][e + 1];
  };
  auto sm_pack = [&](int bf, int qb, int m) {
    const f32x16& x = st[bf][qb];
    const int o = 8 * m;
    pf[qb][m] = to_bf16x8(x[o], x[o + 1], x[o + 2], x[o + 3], x[o + 4], x[o + 5], x[o + 6], x[o + 7]);
    asm volatile("" : "+v"(pf[qb][m]));
  };

  // Iteration t (tile t's scores in st[pc]; tile t+1's K rows in slot kn, its first
  // four operands in okn; tile t's V in slot vc).  Phase 2's barrier, once every
  // wave has read tile t's V^T operands, publishes tile t+2 and lets the copies of
  // tile t+4 go into tile t's slot; then tile t+2's first K row operands are read
  // for the next iteration.  The phases run in full even in the last iteration,
  // where "tile t+1" is whatever an earlier tile left in its slot (in bounds, never
  // used): a value an inline-asm MFMA writes must not pass through a control-flow
  // merge, where the compiler would copy it at once, unaware of the MFMA's latency.
  auto iteration = [&](auto mask_tag, auto par_tag, int t, const __bf16* kn_, const __bf16* vc_, const __bf16* k2_,
                       __bf16* ki, __bf16* vi, Ops& okn) {
    const char* kn = reinterpret_cast<const char*>(kn_);
    const char* vc = reinterpret_cast<const char*>(vc_);
    const char* k2 = reinterpret_cast<const char*>(k2_);
    constexpr int pc = decltype(par_tag)::value, pn = pc ^ 1;  // buffers of tiles t and t+1
    const int k0 = (kt_begin + t) * kKT;                       // tile t's first key
    opaque_bases();
    fence();
    // ---- phase 1: S^T of tile t+1 | softmax of tile t; tile t's first V^T operands
    Ops ovc;
    s_chain(pn, kn, okn, [&](int k) {
      // row maxima in slots 0-1, rescales in 2-3; the 32 exponentials two or four
      // per slot (block 0 in slots 2-9, block 1 in 6-13), each group of 8 packed
      // once complete
      if (k == 0) sm_max(mask_tag, pc, 0, k0);
      if (k == 1) sm_max(mask_tag, pc, 1, k0);
      if (k == 2) sm_rescale(0);
      if (k == 3) sm_rescale(1);
      if (k >= 2 && k < 10) sm_exp2(pc, 0, 2 * (k - 2));
      if (k >= 6 && k < 14) sm_exp2(pc, 1, 2 * (k - 6));
      if (k == 5) sm_pack(pc, 0, 0);
      if (k == 9) sm_pack(pc, 0, 1);
      if (k == 9) sm_pack(pc, 1, 0);
      if (k == 13) sm_pack(pc, 1, 1);
      preload(k, true, vc, ovc);
    });
    // ---- phase 2: O^T += V^T P^T of tile t | the barrier; tile t+2's first K row
    // operands
    pv_chain(vc, ovc, [&](int k) {
      if (k == 8 && t + 2 < n_t) {
        asm volatile("" ::: "memory");
        if (t + 3 < n_t)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCopiesPerTile));  // tile t+3 may stay in flight
        else
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (t + 4 < n_t) issue(t + 4, ki, vi);
      }
      preload(k, false, k2, okn);
    });
    // Wait states behind the last P.V MFMA, before any branch: a loop exit may copy
    // the accumulators at once.
    mfma_acc_gap();
    fence();
  };

  // Prologue: copies of tiles 0..3, the barrier that publishes tiles 0 and 1, then
  // S^T of tile 0 and tile 1's first K row operands.
  Ops okn;
  if (n_t > 0) {
    issue(0, ks0, vs0);
    if (n_t > 1) issue(1, ks1, vs1);
    if (n_t > 2) issue(2, ks2, vs2);
    if (n_t > 3) issue(3, ks3, vs3);
    asm volatile("" ::: "memory");
    if (n_t > 3)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCopiesPerTile));
    else if (n_t > 2)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCopiesPerTile));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    opaque_bases();
    const char* k0c = reinterpret_cast<const char*>(ks0);
    const char* k1c = reinterpret_cast<const char*>(ks1);
    Ops o0;
#pragma unroll
    for (int c = 0; c < 4; ++c) read_op(false, k0c, o0, c);
    s_chain(0, k0c, o0, [&](int k) { preload(k, false, k1c, okn); });  // tile 1 (or a stale slot)
    mfma_read_gap();
    fence();
  }
  // Iteration t reads slots t % 4 (tile t's V) and (t+1) % 4 (tile t+1's K), and
  // fills slot t % 4 with tile t+4.  Iterations whose tile t may need the element
  // mask run the masked body; they start at a multiple of four (up to three more
  // run masked: correct, only slower) so that both loops start at slot 0.
  // Loops in whole groups of four iterations, so that each starts at slot 0: a
  // masked prefix (rounded up: more masked iterations are correct, only slower),
  // the unmasked middle, the masked rest.
  const int pre4 = min(n_t, (n_pre + 3) / 4 * 4);
  const int end_plain = max(pre4, (m_first - kt_begin) / 4 * 4);
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int t = 0;
  for (; t < pre4; t += 4) {
    const BoolTag<true> mk;
    iteration(mk, P0{}, t, ks1, vs0, ks2, ks0, vs0, okn);
    if (t + 1 < n_t) iteration(mk, P1{}, t + 1, ks2, vs1, ks3, ks1, vs1, okn);
    if (t + 2 < n_t) iteration(mk, P0{}, t + 2, ks3, vs2, ks0, ks2, vs2, okn);
    if (t + 3 < n_t) iteration(mk, P1{}, t + 3, ks0, vs3, ks1, ks3, vs3, okn);
  }
  for (; t < end_plain; t += 4) {
    const BoolTag<false> um;
    iteration(um, P0{}, t, ks1, vs0, ks2, ks0, vs0, okn);
    iteration(um, P1{}, t + 1, ks2, vs1, ks3, ks1, vs1, okn);
    iteration(um, P0{}, t + 2, ks3, vs2, ks0, ks2, vs2, okn);
    iteration(um, P1{}, t + 3, ks0, vs3, ks1, ks3, vs3, okn);
  }
  for (; t < n_t; t += 4) {
    const BoolTag<true> mk;
    iteration(mk, P0{}, t, ks1, vs0, ks2, ks0, vs0, okn);
    if (t + 1 < n_t) iteration(mk, P1{}, t + 1, ks2, vs1, ks3, ks1, vs1, okn);
    if (t + 2 < n_t) iteration(mk, P0{}, t + 2, ks3, vs2, ks0, ks2, vs2, okn);
    if (t + 3 < n_t) iteration(mk, P1{}, t + 3, ks0, vs3, ks1, ks3, vs3, okn);
  }

  // (Every iteration ends with the wait states its accumulators need.)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + 32 * qb + col;
    const float l_tot = half_sum(l_run[qb]);
    const bool live = l_tot != 0.0f;  // l_tot >= 0; NaN (from NaN inputs) stays live and propagates
    const float inv = live ? 1.0f / l_tot : 0.0f;
    if (qi < a.Sq)
      fwd_epilogue<4>(a, oacc[qb], inv, live ? (m_run[qb] + log2f(l_tot)) * kLn2 : -INFINITY, b, hq, qi, half);
  }
}

}  // namespace

int64_t fwd64_d128_workgroups(const FwdArgs& args) {
  const int group = args.Hq / args.Hkv;
  const int hpw = fwd64_heads_per_wg(group);
  const int qpw = kNW / hpw;
  return (int64_t)args.B * args.Hkv * (group / hpw) * ((args.Sq + kQW * qpw - 1) / (kQW * qpw));
}

ra_status launch_fwd64_d128(FwdArgs args, hipStream_t stream) {
  const int group = args.Hq / args.Hkv;
  const int qpw = kNW / fwd64_heads_per_wg(group);
  args.n_qtiles = (args.Sq + kQW * qpw - 1) / (kQW * qpw);
  const int64_t n_wg = fwd64_d128_workgroups(args);
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  if (args.seg)
    hipLaunchKernelGGL((fwd64_d128_kernel<true>), dim3((unsigned)n_wg), dim3(64 * kNW), 0, stream, args);
  else
    hipLaunchKernelGGL((fwd64_d128_kernel<false>), dim3((unsigned)n_wg), dim3(64 * kNW), 0, stream, args);
  return check_launch("ring_attn_fwd_step (64 queries per wave)");
}

}  // namespace ra
