// dK, dV of one backward ring step for the hot shape (bf16, head_dim 128), wide
// variant: each wave owns 64 keys (two 32-key MFMA blocks), so every Q and dO
// operand it reads from LDS feeds two MFMAs.
//   dV_j += sum_i P_ij dO_i,  dK_j += scale * sum_i P_ij (dP_ij - delta_i) q_i,
// summed over the query heads of the KV head's GQA group, P recomputed from the
// final log-sum-exp (archcrux, "sequence-parallel long-context attention OOM").
//
// A workgroup is 4 waves x 64 keys of one KV head.  Each wave keeps its keys' K and
// V operands (128 VGPRs) and dK/dV accumulators (256 AGPRs) in registers for the
// whole launch and walks the 32-query tiles of every query head of the group; Q,
// dO and the tile's LSE/delta/segment rows come through a ring of three LDS slots
// filled by raw buffer loads two steps ahead.  Per tile and wave: 32 score MFMAs (S
// and dP of both key blocks) and 32 gradient MFMAs, against 32 KiB of LDS operand
// reads -- half the bytes per MFMA of a 32-key wave.
#include "bwd_d128.h"

namespace ra {
namespace {

constexpr int kD = kD128;
constexpr int kNW = 4;          // waves per workgroup
constexpr int kKW = 64;         // keys per wave
constexpr int kKG = kNW * kKW;  // keys per workgroup
constexpr int kQT = 32;         // queries per staged tile

template <bool kSeg>
__global__ __launch_bounds__(64 * kNW) void dkdv64_d128_kernel(BwdArgs a) {
  // Four tile slots per tensor, each its own array so that the compiler can tell
  // the slot being read from the slots still being filled.
  __shared__ __attribute__((aligned(1024))) __bf16 qs0[kQT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 qs1[kQT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 qs2[kQT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 qs3[kQT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ds0[kQT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ds1[kQT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ds2[kQT * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ds3[kQT * kD];
  // Per slot, four 64-float rows written by one 4-byte-per-lane copy each: -LSE
  // (wave 0), delta (wave 1), and landing zones (waves 2 and 3 copy the LSE row
  // again, so that every wave issues the same number of copies per tile).  Entries 0..31 are the
  // tile's queries; lanes 32..63 of each copy read past its range and write zeros.
  __shared__ __attribute__((aligned(1024))) float xs0[4 * 64];
  __shared__ __attribute__((aligned(1024))) float xs1[4 * 64];
  __shared__ __attribute__((aligned(1024))) float xs2[4 * 64];
  __shared__ __attribute__((aligned(1024))) float xs3[4 * 64];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int kt = logical % a.n_tiles;
  const int g = (logical / a.n_tiles) % a.Hkv;
  const int b = logical / a.n_tiles / a.Hkv;
  const int group = a.Hq / a.Hkv;

  const int k0 = kt * kKG;
  const int k_last = min(k0 + kKG, a.Sk) - 1;
  const int kw = k0 + kKW * wave;  // the wave's first key; its blocks are kw and kw + 32

  const int64_t q_rs = (int64_t)a.Hq * kD, kv_rs = (int64_t)a.Hkv * kD;
  const int q_rb = a.Hq * kD * 2;  // bytes between consecutive query rows

  // K and V of the lane's key in each block as B operands of S = Q K^T and
  // dP = dO V^T.  V is negated (sign bits flipped, exact): the dP chain starts from
  // delta and yields delta - dP, so dS comes out negated with no subtraction per
  // element (undone in the final dK store).
  bf16x8 kf[2][8], vf[2][8];
  bool k_valid[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kj = kw + 32 * kb + col;
    k_valid[kb] = kj < a.Sk;
    const int64_t off = ((int64_t)b * a.Sk + (k_valid[kb] ? kj : 0)) * kv_rs + (int64_t)g * kD + 8 * half;
    const __bf16* kp = static_cast<const __bf16*>(a.k) + off;
    const __bf16* vp = static_cast<const __bf16*>(a.v) + off;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[kb][s] = k_valid[kb] ? load_bf16x8(kp + 16 * s) : bf16x8{};
      vf[kb][s] = k_valid[kb] ? neg_bf16x8(load_bf16x8(vp + 16 * s)) : bf16x8{};
    }
  }

  const int n_qt = (a.Sq + kQT - 1) / kQT;
  int qt_begin = 0, qt_end = n_qt;
  if (a.causal) {
    const int64_t first_q = a.kv_offset + k0 - a.q_offset;
    qt_begin = (int)min<int64_t>((int64_t)n_qt, max<int64_t>(0, first_q) / kQT);
  }
  const int32_t* seg_row = nullptr;
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    const int lo = seg_row[a.kv_offset + k0], hi = seg_row[a.kv_offset + k_last];
    int sb, se;
    seg_tile_range(seg_row + a.q_offset, a.Sq, kQT, qt_begin, qt_end, lo, hi, sb, se);
    qt_begin = sb;
    qt_end = max(sb, se);
  }
  const int n_q = qt_end - qt_begin;
  const int n_iter = n_q * group;

  // Tile order: first the tiles in which some element of some wave may be
  // invisible (they run the masked body), then the rest (the unmasked body).  Per
  // query head the masked tiles are a prefix [qt_begin, qt_begin + n_pre) (the
  // causal diagonal: tiles whose first query precedes the workgroup's last key)
  // and, when the shard ends inside a tile, the last tile.  A workgroup with keys
  // past the chunk end, and every packed-row workgroup, runs all its tiles masked.
  int n_pre = n_q, n_tail = 0;
  if (!kSeg && k0 + kKG <= a.Sk) {
    int64_t diag_end = qt_begin;  // first tile whose first query follows the workgroup's last key
    if (a.causal) {
      const int64_t last_rel = a.kv_offset + k0 + kKG - 1 - a.q_offset;  // last key, in query coordinates
      diag_end = last_rel < 0 ? 0 : last_rel / kQT + 1;
    }
    n_pre = (int)min<int64_t>(n_q, max<int64_t>(0, diag_end - qt_begin));
    n_tail = (a.Sq % kQT != 0 && qt_end - 1 >= qt_begin + n_pre) ? 1 : 0;
  }
  const int n_m = n_pre + n_tail;    // masked tiles per query head
  const int n_u = n_q - n_m;         // unmasked tiles per query head
  const int n_masked = n_m * group;  // sequence positions [0, n_masked) are masked
  struct TileWalk {
    int h, r;
    bool masked;
  };
  auto walk_tile = [&](const TileWalk& w, int& hq, int& qt) {
    hq = g * group + w.h;
    qt = w.masked ? (w.r < n_pre ? qt_begin + w.r : qt_end - 1) : qt_begin + n_pre + w.r;
  };
  auto walk_next = [&](TileWalk& w) {
    if (++w.r == (w.masked ? n_m : n_u)) {
      w.r = 0;
      if (++w.h == group) {
        w.h = 0;
        w.masked = false;
      }
    }
  };
  TileWalk issue_walk{0, 0, n_m > 0}, compute_walk{0, 0, n_m > 0};

  // Visibility of query q0 + 16*half + i to the lane's key of block kb:
  // lo - q0 <= i < hi - q0.  The range is the causal rule, the end of the query
  // shard and, for packed rows, the token span of the key's segment (segment ids
  // are nondecreasing, so the queries of one segment are contiguous).  32-bit:
  // offsets clamped to +-2^30, q0 <= 2^30.  A key past the chunk end sees nothing.
  int vis_lo[2], vis_hi[2];
  SegSpans wsp{};  // the segments of the wave's first and last key
  if constexpr (kSeg)
    wsp = seg_spans_wave(seg_row, a.seg_len, a.kv_offset + min(kw, a.Sk - 1), a.kv_offset + min(kw + 64, a.Sk) - 1);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int64_t kgl = a.kv_offset + kw + 32 * kb + col;
    int64_t lo = INT64_MIN / 2, hi = a.q_offset + a.Sq;  // global query indices
    if (a.causal) lo = kgl;
    if constexpr (kSeg) {
      if (k_valid[kb]) {
        int64_t s_lo, s_hi;
        seg_span_lane(seg_row, a.seg_len, wsp, seg_row[kgl], s_lo, s_hi);
        lo = max(lo, s_lo);
        hi = min(hi, s_hi);
      }
    }
    auto clamp30 = [](int64_t x) { return (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, x)); };
    vis_lo[kb] = clamp30(lo - a.q_offset - 16 * half);
    vis_hi[kb] = k_valid[kb] ? clamp30(hi - a.q_offset - 16 * half) : -(1 << 30);
  }

  f32x16 dk[2][4], dv[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      dk[kb][db] = f32x16{};
      dv[kb][db] = f32x16{};
    }

  const char* qg_base = static_cast<const char*>(a.q) + (int64_t)b * a.Sq * q_rs * 2;
  const char* dg_base = static_cast<const char*>(a.d_o) + (int64_t)b * a.Sq * q_rs * 2;

  // Copies of tile t (query head, 32 queries) global -> LDS slot: 32 rows x 256
  // bytes per tensor = 8 blocks of 1 KiB; wave w copies blocks 2w and 2w+1 of Q
  // and of dO (lane l of a block writes 16 bytes at 16*l, so it fetches the global
  // chunk the swizzle puts there), plus one 4-byte-per-lane copy of the LSE (waves
  // 0, 2, 3) or delta (wave 1) row.  Per-tile
  // descriptors end at the shard's last query: rows past it read as zeros.
  uint32_t coff[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = (2 * wave + r) * 4 + (lane >> 4);
    coff[r] = (uint32_t)(row * q_rb + ((lane & 15) ^ swz(row)) * 16);
  }
  auto issue = [&](__bf16* qs, __bf16* ds, float* xs) {
    int hq, qt;
    walk_tile(issue_walk, hq, qt);
    walk_next(issue_walk);
    const int q0 = qt * kQT;
    const int rows = min(a.Sq - q0, kQT);  // >= 1
    const int64_t hoff = (int64_t)q0 * q_rb + (int64_t)hq * (kD * 2);
    const int bytes = (rows - 1) * q_rb + kD * 2;  // < 2^31: q_rb <= 4096 * 256
    const buffer_rsrc rq = make_rsrc32(qg_base + hoff, bytes);
    const buffer_rsrc rd = make_rsrc32(dg_base + hoff, bytes);
    char* dq_ = reinterpret_cast<char*>(qs) + 2 * wave * 1024;
    char* dd_ = reinterpret_cast<char*>(ds) + 2 * wave * 1024;
    // The per-query row first: wave 0 rescales its LSE row one tile ahead and waits
    // for this copy alone.  Waves 2 and 3 copy the LSE row into their landing zones.
    const int64_t li = ((int64_t)b * a.Hq + hq) * a.Sq + q0;
    const void* src = a.lse + li;
    if (wave == 1) src = a.delta + li;
    buffer_load_lds4(make_rsrc32(src, rows * 4), xs + wave * 64, (uint32_t)lane * 4);
#pragma unroll
    for (int r = 0; r < 2; ++r) buffer_load_lds16(rq, dq_ + r * 1024, coff[r]);
#pragma unroll
    for (int r = 0; r < 2; ++r) buffer_load_lds16(rd, dd_ + r * 1024, coff[r]);
  };
  constexpr int kCopiesPerTile = 5;

  // LDS operand offsets (see ra_device.h): Q and dO rows (A of S = Q K^T and
  // dP = dO V^T) at rA ^ (c << 5); dO^T and Q^T (B of dV += P^T dO, dK += dS^T Q) by
  // transposing reads of rows 16*half + 8m + k (+4) at (tB0|tB1 ^ (db << 6)) + 2048m.
  const int rA = row_read_base(lane);
  const TrBases trb = tr_bases(lane);
  const int tB0 = trb.b0, tB1 = trb.b1;
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  auto tr_read = [](const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
  };
  // The swizzled offsets are recomputed next to each read (one XOR, in a slot with
  // spare vector issue) from per-tile copies of the three bases: kept as 16 loop
  // invariants they would cost 16 registers at the kernel's register peak.
  int rA_t = rA, tB0_t = tB0, tB1_t = tB1;
  auto tr_op = [&](const char* base, int j) {  // operand j = 4m + db
    const int m = j >> 2, db = j & 3;
    const int o0 = (tB0_t ^ (db << 6)) + 2048 * m, o1 = (tB1_t ^ (db << 6)) + 2048 * m;
    const bf16x4_t x0 = tr_read(base + o0), x1 = tr_read(base + o1);
    return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  auto row_op = [&](const char* base, int c) { return load_bf16x8(base + (rA_t ^ (c << 5))); };
  auto read16 = [&](const float* row) {  // entries 16*half .. +15 of a 64-float row
    f32x16 v;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = row[16 * half + i];
    return v;
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  // The LSE row of a tile enters the S chains as their starting accumulator,
  // -LSE/scale: the chain then yields S - LSE/scale and the exponent of P in base 2
  // is one multiplication by scale*log2(e).  Wave 0, which copied the row, rescales
  // it in place one tile ahead: it waits for its copy of tile t+1's row during tile
  // t (the row precedes the 4 row-block copies of that tile and the 5 of tile t+2)
  // and writes it back before the barrier that publishes tile t+1.
  const float neg_inv_scale = -1.0f / a.scale;

  // One 32-query tile against the wave's two 32-key blocks (lane = key, register
  // i of half h = query q0 + 16h + i), as four phases of 16 MFMA slots pinned with
  // scheduling fences so that the vector work runs beside the matrix unit:
  //   S:  S_kb = Q K_kb^T - LSE/scale  (each Q operand feeds both blocks)  | reads
  //   dP: delta - dP_kb = delta + dO (-V_kb)^T                            | P = exp2(.)
  //   dV: dV_kb += P_kb^T dO                                              | -dS = P (delta - dP)
  //   dK: dK_kb += (-dS_kb)^T Q                                           | next tile's barrier
  // Operands are read two MFMA pairs ahead.  The masked body (kMask) sets the
  // exponent of every invisible element to -inf, so P and dS are exactly 0 there.
  // In the dK phase, once the tile's last transposed Q operands are in flight, the
  // wave waits for its copies of tile t+1, joins the barrier that publishes them,
  // issues the copies of tile t+3 (into the slot tile t-1 used: four slots), and
  // reads tile t+1's first operands (fq0, fq1, lsv), which the next tile starts
  // from.
  auto tile = [&](auto mask_tag, int it, const __bf16* qt_, const __bf16* dt_, const float* xs, const __bf16* qn_,
                  float* xn, __bf16* qi, __bf16* di, float* xi, bf16x8& fq0, bf16x8& fq1, f32x16& lsv) {
    constexpr bool kMask = decltype(mask_tag)::value;
    int hq_unused, qt_cur;
    walk_tile(compute_walk, hq_unused, qt_cur);
    walk_next(compute_walk);
    const int q0 = qt_cur * kQT;
    const char* qc = reinterpret_cast<const char*>(qt_);
    const char* dc = reinterpret_cast<const char*>(dt_);
    const bool has_next = it + 1 < n_iter;
    const bool resc = wave == 0 && has_next;
    float lraw = 0.0f;
    rA_t = rA;
    tB0_t = tB0;
    tB1_t = tB1;
    asm volatile("" : "+v"(rA_t), "+v"(tB0_t), "+v"(tB1_t));  // opaque per tile: no hoisted XORs

    // ---- S phase
    f32x16 s[2], dlv;
    bf16x8 fa = fq0, fb = fq1, fd0, fd1;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int c = k >> 1, kb = k & 1;
      s[kb] = mfma_bf16(fa, kf[kb][c], c == 0 ? lsv : s[kb]);
      if (kb == 1) {
        fa = fb;
        if (c + 2 < 8) fb = row_op(qc, c + 2);
      }
      if (k == 2) dlv = read16(xs + 64);
      if (k == 4 && resc) {
        if (it + 2 < n_iter)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
        else
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
        lraw = xn[lane];
      }
      if (k == 12) fd0 = row_op(dc, 0);
      if (k == 14) fd1 = row_op(dc, 1);
      fence();
    }

    // ---- dP phase; P of element e = 16 kb + i, in place of S: exponent (stage B)
    // in slot e/2, exp2 (stage C) one slot later, packed to bf16 by groups of 8.
    f32x16 dp[2];
    bf16x8 pf[2][2], da, dbn;
    auto stage_b = [&](int e) {
      const int kb = e >> 4, i = e & 15;
      float x = s[kb][i] * a.scale_log2;
      if constexpr (kMask) {
        const bool vis = (i >= vis_lo[kb] - q0) & (i < vis_hi[kb] - q0);
        x = vis ? x : -__builtin_inff();
      }
      asm volatile("" : "+v"(x));
      s[kb][i] = x;
    };
    auto stage_c = [&](int e) {
      const int kb = e >> 4, i = e & 15;
      float y = exp2_fast(s[kb][i]);
      asm volatile("" : "+v"(y));
      s[kb][i] = y;
    };
    auto pack_p = [&](int grp) {  // elements 8 grp .. +7 = (kb, m) = (grp / 2, grp % 2)
      const int kb = grp >> 1, m = grp & 1, o = 8 * m;
      pf[kb][m] = to_bf16x8(s[kb][o], s[kb][o + 1], s[kb][o + 2], s[kb][o + 3], s[kb][o + 4], s[kb][o + 5],
                            s[kb][o + 6], s[kb][o + 7]);
    };
    {
      bf16x8 ga = fd0, gb = fd1;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int c = k >> 1, kb = k & 1;
        dp[kb] = mfma_bf16(ga, vf[kb][c], c == 0 ? dlv : dp[kb]);
        if (kb == 1) {
          ga = gb;
          if (c + 2 < 8) gb = row_op(dc, c + 2);
        }
        stage_b(2 * k);
        stage_b(2 * k + 1);
        if (k >= 1) {
          stage_c(2 * k - 2);
          stage_c(2 * k - 1);
        }
        if (k >= 5 && (k - 5) % 4 == 0) pack_p((k - 5) / 4);  // groups 0..2 at slots 5, 9, 13
        if (k == 12) da = tr_op(dc, 0);
        if (k == 14) dbn = tr_op(dc, 1);
        fence();
      }
    }

    // ---- dV phase; -dS of element (kb, i), in place of delta - dP, from the packed
    // P (the values the dV MFMAs use), two per slot in the order (kb0, m0),
    // (kb1, m0), (kb0, m1), (kb1, m1), packed by groups of 8.
    bf16x8 sf[2][2], qa, qb;
    auto stage_d = [&](int e) {
      const int grp = e >> 3, kb = grp & 1, m = grp >> 1, jj = e & 7, i = 8 * m + jj;
      const uint32_t w = __builtin_bit_cast(u32x4, pf[kb][m])[jj >> 1];
      const float p = u32_as_f32((jj & 1) ? (w & 0xffff0000u) : (w << 16));
      float y = p * dp[kb][i];
      asm volatile("" : "+v"(y));
      dp[kb][i] = y;
    };
    auto pack_s = [&](int grp) {
      const int kb = grp & 1, m = grp >> 1, o = 8 * m;
      sf[kb][m] = to_bf16x8(dp[kb][o], dp[kb][o + 1], dp[kb][o + 2], dp[kb][o + 3], dp[kb][o + 4],
                            dp[kb][o + 5], dp[kb][o + 6], dp[kb][o + 7]);
    };
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int j = k >> 1, kb = k & 1, m = j >> 2, db = j & 3;
      if (k == 0) {
        stage_c(30);
        stage_c(31);
      }
      if (k == 1) pack_p(3);
      mfma_acc(dv[kb][db], pf[kb][m], da);
      if (kb == 1) {
        da = dbn;
        if (j + 2 < 8) dbn = tr_op(dc, j + 2);
      }
      if (k >= 2) {  // pf[1][1] is packed in slot 1
        stage_d(2 * k - 4);
        stage_d(2 * k - 3);
      }
      if (k >= 6 && (k - 6) % 4 == 0) pack_s((k - 6) / 4);  // groups 0..2 at slots 6, 10, 14
      if (k == 8 && resc) {
        asm volatile("" : "+v"(lraw));  // keeps the multiplication (and the read) here
        xn[lane] = lraw * neg_inv_scale;
      }
      if (k == 12) qa = tr_op(qc, 0);
      if (k == 14) qb = tr_op(qc, 1);
      fence();
    }

    // ---- dK phase (the last four -dS elements and their packing in its first slots;
    // sf[*][1] is first used in slot 8)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int j = k >> 1, kb = k & 1, m = j >> 2, db = j & 3;
      if (k < 2) {
        stage_d(28 + 2 * k);
        stage_d(29 + 2 * k);
      }
      if (k == 2) pack_s(3);
      mfma_acc(dk[kb][db], sf[kb][m], qa);
      if (kb == 1) {
        qa = qb;
        if (j + 2 < 8) qb = tr_op(qc, j + 2);
      }
      if (k == 12 && has_next) {
        // Tile t+1: its copies (issued two tiles ago) must have landed; tile t+2's
        // may stay in flight.  The barrier publishes every wave's copies and wave 0's
        // rescaled LSE row, and tells that every wave has finished tile t-1.
        asm volatile("" ::: "memory");
        if (it + 2 < n_iter)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCopiesPerTile));
        else
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (it + 3 < n_iter) issue(qi, di, xi);
        const char* qn = reinterpret_cast<const char*>(qn_);
        lsv = read16(xn);
        fq0 = row_op(qn, 0);
        fq1 = row_op(qn, 1);
      }
      fence();
    }
    // Wait states behind the last accumulating MFMA before any branch: on the
    // loop's exit path the compiler may copy the accumulators at once.
    mfma_acc_gap();
    fence();
  };

  // Prologue: copies of tiles 0 and 1, wave 0 rescales tile 0's LSE row, the barrier
  // that publishes tile 0, copies of tile 2, and tile 0's first operands.
  bf16x8 fq0{}, fq1{};
  f32x16 lsv{};
  if (n_iter > 0) {
    issue(qs0, ds0, xs0);
    if (n_iter > 1) issue(qs1, ds1, xs1);
    if (n_iter > 1)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCopiesPerTile));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if (wave == 0) xs0[lane] = xs0[lane] * neg_inv_scale;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));  // the rescaled row is in LDS
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (n_iter > 2) issue(qs2, ds2, xs2);
    lsv = read16(xs0);
    fq0 = row_op(reinterpret_cast<const char*>(qs0), 0);
    fq1 = row_op(reinterpret_cast<const char*>(qs0), 1);
  }
  // Tile t uses slot t % 4 and issues tile t+3 into slot (t+3) % 4.  Masked tiles
  // first, in whole groups of four (a group that reaches into the unmasked tiles
  // runs masked: correct, only slower), so that both loops start at slot 0.
  const int n_masked4 = min(n_iter, (n_masked + 3) / 4 * 4);
  int it = 0;
  for (; it < n_masked4; it += 4) {
    const BoolTag<true> mk;
    tile(mk, it, qs0, ds0, xs0, qs1, xs1, qs3, ds3, xs3, fq0, fq1, lsv);
    if (it + 1 < n_iter) tile(mk, it + 1, qs1, ds1, xs1, qs2, xs2, qs0, ds0, xs0, fq0, fq1, lsv);
    if (it + 2 < n_iter) tile(mk, it + 2, qs2, ds2, xs2, qs3, xs3, qs1, ds1, xs1, fq0, fq1, lsv);
    if (it + 3 < n_iter) tile(mk, it + 3, qs3, ds3, xs3, qs0, xs0, qs2, ds2, xs2, fq0, fq1, lsv);
  }
  for (; it < n_iter; it += 4) {
    const BoolTag<false> um;
    tile(um, it, qs0, ds0, xs0, qs1, xs1, qs3, ds3, xs3, fq0, fq1, lsv);
    if (it + 1 < n_iter) tile(um, it + 1, qs1, ds1, xs1, qs2, xs2, qs0, ds0, xs0, fq0, fq1, lsv);
    if (it + 2 < n_iter) tile(um, it + 2, qs2, ds2, xs2, qs3, xs3, qs1, ds1, xs1, fq0, fq1, lsv);
    if (it + 3 < n_iter) tile(um, it + 3, qs3, ds3, xs3, qs0, xs0, qs2, ds2, xs2, fq0, fq1, lsv);
  }

  // A workgroup without a live tile adds exactly zero to every accumulator: done.
  // (Tested here rather than before the loop: an early exit there costs the loop
  // registers.)
  if (n_iter <= 0) return;
  // The accumulators were last written by inline-asm MFMAs, which the compiler's
  // hazard tracking does not see: wait out the MFMA write latency before they are read.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(dk[0][0]), "+a"(dk[0][1]), "+a"(dk[0][2]), "+a"(dk[0][3]), "+a"(dv[0][0]), "+a"(dv[0][1]),
                 "+a"(dv[0][2]), "+a"(dv[0][3]));
  asm volatile("" : "+a"(dk[1][0]), "+a"(dk[1][1]), "+a"(dk[1][2]), "+a"(dk[1][3]), "+a"(dv[1][0]), "+a"(dv[1][1]),
               "+a"(dv[1][2]), "+a"(dv[1][3]));
  // lane = d column, register i of half h = key kw + 32kb + mfma32_row(i, h).  The
  // read-modify-write of dK and dV goes in groups of 16 keys x 2 tensors so that the
  // loads of a group are in flight together (the two pointers do not alias).
  float* __restrict__ dkp = a.dk;
  float* __restrict__ dvp = a.dv;
  const float ks = -a.scale;  // dk holds -sum dS^T q (the dP chain runs on negated V)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kbase = kw + 32 * kb;
    const int64_t base = ((int64_t)b * a.Sk + kbase) * kv_rs + (int64_t)g * kD + col;
    const bool full = kbase + 32 <= a.Sk;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      float ok[16], ov[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = mfma32_row(i, half);
        const int64_t off = base + (int64_t)r * kv_rs + 32 * db;
        if (full || kbase + r < a.Sk) {
          ok[i] = dkp[off];
          ov[i] = dvp[off];
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = mfma32_row(i, half);
        const int64_t off = base + (int64_t)r * kv_rs + 32 * db;
        if (full || kbase + r < a.Sk) {
          dkp[off] = ok[i] + ks * dk[kb][db][i];
          dvp[off] = ov[i] + dv[kb][db][i];
        }
      }
    }
  }
}

}  // namespace

int64_t dkdv64_d128_workgroups(const BwdArgs& args) {
  return (int64_t)args.B * args.Hkv * ((args.Sk + kKG - 1) / kKG);
}

ra_status launch_dkdv64_d128(BwdArgs args, hipStream_t stream) {
  args.n_tiles = (args.Sk + kKG - 1) / kKG;
  const int64_t n_wg = dkdv64_d128_workgroups(args);
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  if (args.seg)
    hipLaunchKernelGGL((dkdv64_d128_kernel<true>), dim3((unsigned)n_wg), dim3(64 * kNW), 0, stream, args);
  else
    hipLaunchKernelGGL((dkdv64_d128_kernel<false>), dim3((unsigned)n_wg), dim3(64 * kNW), 0, stream, args);
  return check_launch("ring_attn_bwd_step (dK/dV, 64 keys per wave)");
}

}  // namespace ra
