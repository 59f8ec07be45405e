// dQ of one backward ring step for the hot shape (bf16, head_dim 128), wide
// variant: each wave owns 64 queries (two 32-query MFMA blocks), so every K and V
// operand it reads from LDS feeds two MFMAs.
//   dQ_i += scale * sum_j P_ij (dP_ij - delta_i) k_j,  P recomputed from the final
// log-sum-exp (archcrux, "sequence-parallel long-context attention OOM").
//
// A workgroup is 4 waves over the query heads of one KV head's GQA group (up to 4
// heads, the same 64 queries each; smaller groups stack query blocks instead), so
// all of its waves share every K/V tile.  Each wave keeps its queries' Q and dO
// operands (128 AGPRs: B operands of the score MFMAs) and dQ accumulators (128
// AGPRs) in registers for the whole launch; K/V tiles of 32 keys come through a
// ring of four LDS slots filled by raw buffer loads.  Per tile and wave: 16 MFMAs
// each for S^T = K Q^T, dP^T = V dO^T and dQ^T += K^T dS^T, against 24 KiB of LDS
// operand reads -- half the bytes per MFMA of a 32-query wave.
//
// The tile loop is software-pipelined across tiles: iteration t runs
//   phase 1: S^T of tile t+1            | dS of tile t (from P and dP - delta)
//   phase 2: dQ^T += K^T dS^T, tile t   | P of tile t+1, query block 0
//   phase 3: dP^T of tile t+1           | P of tile t+1, query block 1
// so that the vector work of each tile runs beside the matrix unit.  The MFMAs are
// inline assembly (the score MFMAs read their B operand from AGPRs, which the
// compiler does not allocate by itself); their hazards are kept by the schedule:
// each phase's results are first read by vector instructions in a later phase,
// behind explicit wait states.
#include <type_traits>

#include "bwd_d128.h"

namespace ra {
namespace {

constexpr int kD = kD128;
constexpr int kNW = 4;   // waves per workgroup
constexpr int kQW = 64;  // queries per wave
constexpr int kKT = 32;  // keys per staged tile

// Heads per workgroup: the largest of 4, 2, 1 that divides the GQA group.
__host__ __device__ __forceinline__ int dq64_heads_per_wg(int group) {
  return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
}

template <bool kSeg>
__global__ __launch_bounds__(64 * kNW) void dq64_d128_kernel(BwdArgs a) {
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
  const int hpw = dq64_heads_per_wg(group);  // heads per workgroup
  const int qpw = kNW / hpw;                 // 64-query blocks per workgroup
  const int n_hset = group / hpw;
  int rem = logical;
  const int qt_rev = rem % a.n_tiles;
  rem /= a.n_tiles;
  const int hset = rem % n_hset;
  rem /= n_hset;
  const int g = rem % a.Hkv;
  const int b = rem / a.Hkv;
  const int qt = a.n_tiles - 1 - qt_rev;  // latest (heaviest causal) query tiles first
  const int hq = g * group + hset * hpw + wave % hpw;
  const int q_wg = qt * kQW * qpw;                 // the workgroup's first query
  const int qw = q_wg + kQW * (wave / hpw);        // the wave's first query
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
  // A workgroup without a live tile adds exactly zero to every accumulator: done.
  if (n_t <= 0) return;

  // Per lane and query block qb: the query q = qw + 32 qb + col, its Q and dO rows
  // (B operands; lane = query column, k-slots = d), -LSE*log2(e), and -delta
  // broadcast over a register tuple (the start of the dP^T chain, which then yields
  // dP - delta).  Visible keys of the query: the chunk range [vlo, vhi] (causal
  // rule, chunk end, segment span); a query past the shard sees nothing.
  bf16x8 qf[2][8], dof[2][8];
  float neg_lse2[2];
  f32x16 ndl[2];
  int vlo[2], vhi[2];
  SegSpans wsp{};  // the segments of the wave's first and last query
  if constexpr (kSeg)
    wsp = seg_spans_wave(seg_row, a.seg_len, a.q_offset + min(qw, a.Sq - 1), a.q_offset + min(qw + kQW, a.Sq) - 1);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + 32 * qb + col;
    const bool qv = qi < a.Sq;
    const int64_t off = ((int64_t)b * a.Sq + (qv ? qi : 0)) * q_rs + (int64_t)hq * kD + 8 * half;
    const __bf16* qp = static_cast<const __bf16*>(a.q) + off;
    const __bf16* dp = static_cast<const __bf16*>(a.d_o) + off;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qf[qb][s] = qv ? load_bf16x8(qp + 16 * s) : bf16x8{};
      dof[qb][s] = qv ? load_bf16x8(dp + 16 * s) : bf16x8{};
    }
    const int64_t li = ((int64_t)b * a.Hq + hq) * a.Sq + (qv ? qi : 0);
    const float lse_q = qv ? a.lse[li] : -INFINITY;
    neg_lse2[qb] = lse_q == -INFINITY ? -INFINITY : -lse_q * kLog2e;
    const float dl = qv ? a.delta[li] : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ndl[qb][i] = -dl;
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
  // Pin Q and dO to AGPRs (their only uses are the inline-asm score MFMAs).
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" : "+a"(qf[qb][s]), "+a"(dof[qb][s]));

  // Tiles [m_first, kt_end) may hold an invisible element for some lane of the wave
  // (the causal diagonal, the chunk's ragged end); every tile does if the wave's
  // queries run past the shard, and for packed rows.
  int m_first = kt_begin;
  if (!kSeg && qw + kQW <= a.Sq) {
    // first key (chunk index) the wave's first query does not see: keys beyond it
    // need the element mask
    int64_t first_hidden = a.Sk;
    if (a.causal) first_hidden = min<int64_t>(first_hidden, a.q_offset + qw - a.kv_offset + 1);
    int64_t mt = max<int64_t>(0, first_hidden) / kKT;  // tile holding it
    if (a.Sk % kKT != 0) mt = min<int64_t>(mt, a.Sk / kKT);
    m_first = (int)max<int64_t>(kt_begin, min<int64_t>(kt_end, mt));
  }

  f32x16 dq[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db) dq[qb][db] = f32x16{};

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

  // LDS operand offsets (see ra_device.h): K and V rows (A of S^T = K Q^T and
  // dP^T = V dO^T) at rA ^ (c << 5); K^T (A of dQ^T += K^T dS^T) by transposing
  // reads at (tB0|tB1 ^ (db << 6)) + 2048 m.  Recomputed next to each read from
  // per-tile opaque copies of the bases (no hoisted XOR results held in registers).
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

  // Element state: st[u & 1][qb] holds tile u's S^T, then the exponent, then P
  // (register i of half h = key k0 + 16h + i) -- two buffers, since tile t's P is
  // still read while tile t+1's S^T is computed; dpt[qb] holds dP - delta, then
  // dS = P (dP - delta).
  f32x16 st[2][2], dpt[2];
  bf16x8 sf[2][2];  // dS^T packed: [qb][m], keys 16h + 8m + j

  // Stage B (exponent, and the mask in masked tiles) and stage C (exp2) of P for
  // query block qb of the tile starting at chunk key k0, element i.
  auto stage_b = [&](auto mask_tag, int bf, int qb, int i, int k0) {
    constexpr bool kMask = decltype(mask_tag)::value;
    float x = __builtin_fmaf(st[bf][qb][i], a.scale_log2, neg_lse2[qb]);
    if constexpr (kMask) {
      const bool vis = (i >= vlo[qb] - k0) & (i <= vhi[qb] - k0);
      x = vis ? x : -__builtin_inff();
    }
    asm volatile("" : "+v"(x));
    st[bf][qb][i] = x;
  };
  auto stage_c = [&](int bf, int qb, int i) {
    float y = exp2_fast(st[bf][qb][i]);
    asm volatile("" : "+v"(y));
    st[bf][qb][i] = y;
  };
  // Stage D: dS = P (dP - delta), element (qb, i); packing of keys 8m .. 8m+7.
  auto stage_d = [&](int bf, int qb, int i) {
    float y = st[bf][qb][i] * dpt[qb][i];
    asm volatile("" : "+v"(y));
    dpt[qb][i] = y;
  };
  auto pack_s = [&](int qb, int m) {
    const int o = 8 * m;
    sf[qb][m] = to_bf16x8(dpt[qb][o], dpt[qb][o + 1], dpt[qb][o + 2], dpt[qb][o + 3], dpt[qb][o + 4],
                          dpt[qb][o + 5], dpt[qb][o + 6], dpt[qb][o + 7]);
  };

  // Operand sets: the 8 K or V row operands of a tile (A of the S^T or dP^T chain),
  // or its 8 K^T operands (A of the dQ^T MFMAs).  A chain reads its operand c+4 right
  // after the last use of operand c; operands 0..3 are read during the previous
  // chain's last slots.  So every read has four MFMA pairs of cover against the LDS
  // latency.
  struct Ops {
    bf16x8 f[8];
  };
  auto read_op = [&](bool tr, const char* base, Ops& o, int c) { o.f[c] = tr ? tr_op(base, c) : row_op(base, c); };

  // The S^T and dP^T chains of a tile, 16 MFMAs each (query blocks interleaved, each
  // operand feeds both), with `work(k)` in slot k's shadow.
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
  auto dp_chain = [&](const char* base, Ops& o, auto&& work) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int c = k >> 1, qb = k & 1;
      if (c == 0)
        mfma_vab(dpt[qb], o.f[0], dof[qb][0], ndl[qb]);
      else
        mfma_vab_acc(dpt[qb], o.f[c], dof[qb][c]);
      if (qb == 1 && c + 4 < 8) read_op(false, base, o, c + 4);
      work(k);
      fence();
    }
  };
  // dQ^T[qb][db] += K^T[m][db] dS^T[qb][m]: 16 MFMAs (m-major, qb-minor).
  auto dq_chain = [&](const char* base, Ops& o, auto&& work) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int j = k >> 1, qb = k & 1, m = j >> 2, db = j & 3;
      mfma_acc(dq[qb][db], o.f[j], sf[qb][m]);
      if (qb == 1 && j + 4 < 8) read_op(true, base, o, j + 4);
      work(k);
      fence();
    }
  };
  // The first four operands of the next chain, one per odd slot from slot 9 on.
  auto preload = [&](int k, bool tr, const char* base, Ops& o) {
    if (k >= 9 && (k & 1)) read_op(tr, base, o, (k - 9) >> 1);
  };

  // Iteration t (tile t in slot kc, tile t+1 in slot kn/vn): phases 1-3 above.  The
  // K row operands of tile t+1 (okn) were read in the previous iteration; phase 1
  // reads tile t's K^T operands, phase 2 tile t+1's V row operands.  In phase 3,
  // once every wave is past phase 2 (no longer reads tile t), the barrier that
  // publishes tile t+2 lets the copies of tile t+4 go into tile t's slot, and tile
  // t+2's K row operands are read for the next iteration.  The phases run in full
  // even in the last iteration, where "tile t+1" is whatever an earlier tile left in
  // its slot (in bounds, never used): a value an inline-asm MFMA writes must not pass
  // through a control-flow merge, where the compiler would copy it at once, unaware
  // of the MFMA's write latency.
  auto iteration = [&](auto mask_tag, auto par_tag, int t, const __bf16* kc_, const __bf16* kn_, const __bf16* vn_,
                       const __bf16* k2_, __bf16* ki, __bf16* vi, Ops& okn) {
    const char* kc = reinterpret_cast<const char*>(kc_);
    const char* kn = reinterpret_cast<const char*>(kn_);
    const char* vn = reinterpret_cast<const char*>(vn_);
    const char* k2 = reinterpret_cast<const char*>(k2_);
    constexpr int pc = decltype(par_tag)::value, pn = pc ^ 1;  // buffers of tiles t and t+1
    const int k0n = (kt_begin + t + 1) * kKT;  // tile t+1's first key
    opaque_bases();
    fence();
    // ---- phase 1: S^T of tile t+1 | dS of tile t and its packing; tile t's first
    // K^T operands
    Ops otc, ovn;
    s_chain(pn, kn, okn, [&](int k) {
      // dS of tile t: 32 elements, two per slot, packed by groups of 8 keys
      const int e0 = 2 * k;
      stage_d(pc, e0 >> 4, e0 & 15);
      stage_d(pc, (e0 + 1) >> 4, (e0 + 1) & 15);
      if ((k & 3) == 3) {
        const int grp = k >> 2;  // elements 8 grp .. 8 grp + 7 = (qb, m) = (grp / 2, grp % 2)
        pack_s(grp >> 1, grp & 1);
      }
      preload(k, true, kc, otc);
    });
    // ---- phase 2: dQ of tile t | P of tile t+1, query block 0; tile t+1's first V
    // row operands
    mfma_read_gap();
    fence();
    dq_chain(kc, otc, [&](int k) {
      stage_b(mask_tag, pn, 0, k, k0n);
      if (k >= 1) stage_c(pn, 0, k - 1);
      preload(k, false, vn, ovn);
    });
    // ---- phase 3: dP^T of tile t+1 | P of tile t+1, query block 1 (the last
    // element of block 0 first); the barrier, then tile t+2's first K row operands
    dp_chain(vn, ovn, [&](int k) {
      if (k == 0) stage_c(pn, 0, 15);
      stage_b(mask_tag, pn, 1, k, k0n);
      if (k >= 1) stage_c(pn, 1, k - 1);
      if (k == 4 && t + 2 < n_t) {
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
      if (k == 15) stage_c(pn, 1, 15);
    });
    // Wait states behind the last dP^T MFMA before any branch: past a loop exit its
    // registers are free, and an instruction that reused one could be overwritten by
    // the MFMA's late write.
    mfma_read_gap();
    fence();
  };

  // Prologue: copies of tiles 0..3, the barrier that publishes tiles 0 and 1, then
  // S^T, P and dP^T of tile 0 (no overlap) and tile 1's K row operands.
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
    const char* v0c = reinterpret_cast<const char*>(vs0);
    const int k00 = kt_begin * kKT;
    Ops o0, o1;
#pragma unroll
    for (int c = 0; c < 4; ++c) read_op(false, k0c, o0, c);
    s_chain(0, k0c, o0, [&](int k) { preload(k, false, v0c, o1); });
    dp_chain(v0c, o1, [](int) {});
    mfma_read_gap();
    fence();
    const bool masked0 = kt_begin >= m_first;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (masked0)
          stage_b(BoolTag<true>{}, 0, qb, i, k00);
        else
          stage_b(BoolTag<false>{}, 0, qb, i, k00);
        stage_c(0, qb, i);
      }
#pragma unroll
    for (int c = 0; c < 4; ++c) read_op(false, reinterpret_cast<const char*>(ks1), okn, c);  // tile 1 (or a stale slot)
  }
  // Iteration t reads slots t % 4 (tile t) and (t+1) % 4, and fills slot t % 4 with
  // tile t+4.  Iterations whose tile t+1 may need the element mask run the masked
  // body; they start at a multiple of four (up to three more run masked: correct,
  // only slower) so that both loops start at slot 0.
  const int first_m_it = max(0, m_first - kt_begin - 1);
  const int n_plain = min(n_t, first_m_it / 4 * 4);
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int t = 0;
  for (; t < n_plain; t += 4) {
    const BoolTag<false> um;
    iteration(um, P0{}, t, ks0, ks1, vs1, ks2, ks0, vs0, okn);
    iteration(um, P1{}, t + 1, ks1, ks2, vs2, ks3, ks1, vs1, okn);
    iteration(um, P0{}, t + 2, ks2, ks3, vs3, ks0, ks2, vs2, okn);
    iteration(um, P1{}, t + 3, ks3, ks0, vs0, ks1, ks3, vs3, okn);
  }
  for (; t < n_t; t += 4) {
    const BoolTag<true> mk;
    iteration(mk, P0{}, t, ks0, ks1, vs1, ks2, ks0, vs0, okn);
    if (t + 1 < n_t) iteration(mk, P1{}, t + 1, ks1, ks2, vs2, ks3, ks1, vs1, okn);
    if (t + 2 < n_t) iteration(mk, P0{}, t + 2, ks2, ks3, vs3, ks0, ks2, vs2, okn);
    if (t + 3 < n_t) iteration(mk, P1{}, t + 3, ks3, ks0, vs0, ks1, ks3, vs3, okn);
  }

  // The accumulators were last written by inline-asm MFMAs: wait out their latency.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(dq[0][0]), "+a"(dq[0][1]), "+a"(dq[0][2]), "+a"(dq[0][3]), "+a"(dq[1][0]), "+a"(dq[1][1]),
                 "+a"(dq[1][2]), "+a"(dq[1][3]));
  // lane = query, register 4 r4 + j of half h = d column 32 db + 8 r4 + 4 h + j.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + 32 * qb + col;
    if (qi < a.Sq) {
      float* row = a.dq + ((int64_t)b * a.Sq + qi) * q_rs + (int64_t)hq * kD;
      f32x4 cur[4][4];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) cur[db][r4] = *reinterpret_cast<const f32x4*>(row + 32 * db + 8 * r4 + 4 * half);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 v = cur[db][r4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] += a.scale * dq[qb][db][4 * r4 + j];
          *reinterpret_cast<f32x4*>(row + 32 * db + 8 * r4 + 4 * half) = v;
        }
    }
  }
}

}  // namespace

int64_t dq64_d128_workgroups(const BwdArgs& args) {
  const int group = args.Hq / args.Hkv;
  const int hpw = dq64_heads_per_wg(group);
  const int qpw = kNW / hpw;
  return (int64_t)args.B * args.Hkv * (group / hpw) * ((args.Sq + kQW * qpw - 1) / (kQW * qpw));
}

ra_status launch_dq64_d128(BwdArgs args, hipStream_t stream) {
  const int group = args.Hq / args.Hkv;
  const int qpw = kNW / dq64_heads_per_wg(group);
  args.n_tiles = (args.Sq + kQW * qpw - 1) / (kQW * qpw);
  const int64_t n_wg = dq64_d128_workgroups(args);
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  if (args.seg)
    hipLaunchKernelGGL((dq64_d128_kernel<true>), dim3((unsigned)n_wg), dim3(64 * kNW), 0, stream, args);
  else
    hipLaunchKernelGGL((dq64_d128_kernel<false>), dim3((unsigned)n_wg), dim3(64 * kNW), 0, stream, args);
  return check_launch("ring_attn_bwd_step (dQ, 64 queries per wave)");
}

}  // namespace ra
