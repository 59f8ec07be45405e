// dK, dV of one backward ring step for the hot shape (bf16, head_dim 128):
//   dV_j += sum_i P_ij dO_i,  dK_j += scale * sum_i P_ij (dP_ij - delta_i) q_i,
// summed over the query heads of the KV head's GQA group, P recomputed from the
// final log-sum-exp (archcrux, "sequence-parallel long-context attention OOM").
// Each wave keeps 32 keys' K and V operands and dK/dV accumulators in registers
// and walks the 64-query tiles of every query head of the group.  Q and dO tiles
// are copied global -> LDS (swizzled, row-major; raw buffer loads, no staging
// registers) two steps ahead into a ring of three slots; their transposes are
// read with transposing LDS reads.  The tile body is a hand-placed MFMA / vector
// ALU pipeline (see compute below).
#include <algorithm>

#include "bwd_d128.h"


namespace ra {
namespace {

constexpr int kD = kD128;
constexpr int kMinSplitTiles = 8;  // fewest tile positions per workgroup of a split key block

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
  __shared__ int last_flag;  // split key blocks: this workgroup completes the block

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  // Workgroup -> (b, kv head, key block, split); the splits of a key block are
  // consecutive, so they run on one XCD.
  const int split = logical % a.n_split;
  const int kblk = logical / a.n_split;  // key block, linear over (b, kv head, key tile)
  const int kt = kblk % a.n_tiles;
  const int g = (kblk / a.n_tiles) % a.Hkv;
  const int b = kblk / a.n_tiles / a.Hkv;
  const int group = a.Hq / a.Hkv;

  const int k0 = kt * 32 * NW;
  const int k_last = min(k0 + 32 * NW, a.Sk) - 1;
  const int kw = k0 + 32 * wave;
  const int kj = kw + col;
  const bool k_valid = kj < a.Sk;
  const int64_t kgl = a.kv_offset + kj;

  const int64_t q_rs = (int64_t)a.Hq * kD, kv_rs = (int64_t)a.Hkv * kD;
  const int q_rb = a.Hq * kD * 2;  // bytes between consecutive query rows

  // K and V of this lane's key as B operands of S = Q K^T and dP = dO V^T.  V is
  // negated (sign bits flipped, exact): the dP chain starts from delta and yields
  // delta - dP, so dS comes out negated with no subtraction per element (undone
  // in the final dK store).
  bf16x8 kf[8], vf[8];
  {
    const int64_t off = ((int64_t)b * a.Sk + (k_valid ? kj : 0)) * kv_rs + (int64_t)g * kD + 8 * half;
    const __bf16* kp = static_cast<const __bf16*>(a.k) + off;
    const __bf16* vp = static_cast<const __bf16*>(a.v) + off;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[s] = k_valid ? load_bf16x8(kp + 16 * s) : bf16x8{};
      vf[s] = k_valid ? neg_bf16x8(load_bf16x8(vp + 16 * s)) : bf16x8{};
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
  // Packed rows: when every key of the workgroup is in one segment, the query tiles
  // that lie entirely inside that segment, [full_lo, full_hi), need no segment test.
  bool one_seg = !kSeg;
  int64_t full_lo = 0, full_hi = n_qt;
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    seg_k = k_valid ? seg_row[kgl] : INT32_MIN;
    const int lo = seg_row[a.kv_offset + k0], hi = seg_row[a.kv_offset + k_last];
    if (lo == hi) {
      const SegSpans w = seg_spans_wave(seg_row, a.seg_len, a.kv_offset + k0, a.kv_offset + k0);
      const int64_t sp_lo = w.lo0, sp_hi = w.hi0;  // the segment's token span in the row
      full_lo = max<int64_t>(0, sp_lo - a.q_offset + QT - 1) / QT;
      full_hi = min<int64_t>(n_qt, max<int64_t>(0, sp_hi - a.q_offset) / QT);
      one_seg = true;
    }
    int sb, se;
    seg_tile_range(seg_row + a.q_offset, a.Sq, QT, qt_begin, qt_end, lo, hi, sb, se);
    qt_begin = sb;
    qt_end = max(sb, se);
  }
  const int n_q = qt_end - qt_begin;
  const int n_iter = n_q * group;
  // A workgroup without a live tile adds exactly zero to every accumulator: done.
  if (n_iter <= 0) return;
  // Split of the key block's n_iter tile positions (walk order below) over n_sp
  // workgroups, at least kMinSplitTiles positions each; workgroups past n_sp have
  // nothing to do.  This workgroup takes positions [p_begin, p_begin + len).
  const int n_sp = max(1, min(a.n_split, n_iter / kMinSplitTiles));
  if (split >= n_sp) return;
  const int p_begin = (int)((int64_t)n_iter * split / n_sp);
  const int len = (int)((int64_t)n_iter * (split + 1) / n_sp) - p_begin;

  // Tile order: first the tiles in which some element of some wave of the
  // workgroup may be invisible (they run the masked body), then the rest (the
  // unmasked body, no selects).  Per query head the masked tiles are a prefix
  // [qt_begin, qt_begin + n_pre) (the causal diagonal: tiles whose first query
  // precedes the workgroup's last key; for packed rows also the tiles before the
  // first one inside the keys' segment) and one last tile when the shard ends inside
  // it (or, packed, when it reaches past the segment's end).  A workgroup with keys
  // past the chunk end, or with keys of two segments, runs all its tiles masked.
  int n_pre = n_q, n_tail = 0;
  if (one_seg && k0 + 32 * NW <= a.Sk) {
    int64_t diag_end = qt_begin;  // first tile whose first query follows the workgroup's last key
    if (a.causal) {
      const int64_t last_rel = a.kv_offset + k0 + 32 * NW - 1 - a.q_offset;  // last key, in query coordinates
      diag_end = last_rel < 0 ? 0 : last_rel / QT + 1;
    }
    if constexpr (kSeg) diag_end = max<int64_t>(diag_end, full_lo);
    n_pre = (int)min<int64_t>(n_q, max<int64_t>(0, diag_end - qt_begin));
    bool tail = a.Sq % QT != 0;
    if constexpr (kSeg) tail |= qt_end > full_hi;
    n_tail = (tail && qt_end - 1 >= qt_begin + n_pre) ? 1 : 0;
  }
  const int n_m = n_pre + n_tail;     // masked tiles per query head
  const int n_u = n_q - n_m;          // unmasked tiles per query head
  const int n_masked = n_m * group;   // sequence positions [0, n_masked) are masked
  // Walk over that order.  The copies and the tile bodies each visit the tiles in
  // order, so each keeps a walker (query head within the group, position within
  // the head's run of masked or unmasked tiles) instead of dividing per tile.
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
  auto walk_at = [&](int pos) {  // the walker at position pos of the order
    if (pos < n_masked) return TileWalk{pos / n_m, pos % n_m, true};
    const int u = pos - n_masked;
    return TileWalk{u / n_u, u % n_u, false};
  };
  TileWalk issue_walk = walk_at(p_begin), compute_walk = walk_at(p_begin);

  // Visibility of query q0 + 16*half + i to this lane's key: lo - q0 <= i < hi - q0
  // (causal rule and the end of the query shard; 32-bit: offsets clamped to +-2^30,
  // q0 <= 2^30).  A key past the chunk end sees nothing.
  int vis_lo = -(1 << 30), vis_hi = a.Sq - 16 * half;
  if (a.causal) vis_lo = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, kgl - a.q_offset - 16 * half));
  if (!k_valid) vis_hi = -(1 << 30);

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const char* qg_base = static_cast<const char*>(a.q) + (int64_t)b * a.Sq * q_rs * 2;
  const char* dg_base = static_cast<const char*>(a.d_o) + (int64_t)b * a.Sq * q_rs * 2;

  // Copies of tile t (query head, 64 queries) global -> LDS slot, no staging
  // registers: 64 rows x 256 bytes per tensor = 16 blocks of 1 KiB, four per wave
  // (lane l of a block writes 16 bytes at 16*l, so it fetches the global chunk the
  // swizzle puts there), plus one 4-byte-per-lane copy of lse (wave 0), delta
  // (wave 1), segment ids (wave 2) or a dummy (wave 3).  Raw buffer loads with
  // per-tile descriptors ending at the shard's last query: rows past it read as
  // zeros (and are masked).
  uint32_t coff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = (4 * wave + r) * 4 + (lane >> 4);
    coff[r] = (uint32_t)(row * q_rb + ((lane & 15) ^ swz(row)) * 16);
  }
  // A tile's copies are planned once (walk step, addresses, ranges) and issued in
  // two parts: the per-query row right after the barrier that frees its slot, the
  // eight 1 KiB row blocks one per MFMA pair in the first phase of the step, instead
  // of nine back to back.  A plan past the last tile has empty ranges: its loads
  // read nothing and write zeros into the free slot.
  struct CopyPlan {
    const char* q;
    const char* d;
    const char* x;
    int bytes, xbytes;
  };
  auto plan_copy = [&](bool valid) {
    int hq, qt;
    walk_tile(issue_walk, hq, qt);
    walk_next(issue_walk);
    CopyPlan p{qg_base, dg_base, reinterpret_cast<const char*>(a.lse), 0, 0};
    if (valid) {
      const int q0 = qt * QT;
      const int rows = min(a.Sq - q0, QT);  // >= 1; the descriptors end at the tile's last valid row
      const int64_t hoff = (int64_t)q0 * q_rb + (int64_t)hq * (kD * 2);
      // The per-query row: LSE (wave 0), delta (wave 1), segment ids (wave 2), or
      // the LSE again as a dummy (wave 3).
      const int64_t li = ((int64_t)b * a.Hq + hq) * a.Sq + q0;
      const void* src = a.lse + li;
      if (wave == 1) src = a.delta + li;
      if constexpr (kSeg) {
        if (wave == 2) src = seg_row + a.q_offset + q0;
      }
      p.q = qg_base + hoff;
      p.d = dg_base + hoff;
      p.x = static_cast<const char*>(src);
      p.bytes = (rows - 1) * q_rb + kD * 2;  // < 2^31: q_rb <= 4096 * 256
      p.xbytes = rows * 4;
    }
    return p;
  };
  // The per-query row first: wave 0 rescales its LSE row one step later and waits
  // for this copy alone.
  auto issue_row = [&](const CopyPlan& p, float* xs) {
    buffer_load_lds4(make_rsrc32(p.x, p.xbytes), xs + wave * QT, (uint32_t)lane * 4);
  };
  // Row block r of the tile: Q blocks 4w .. 4w+3 (r = 0..3), dO blocks (r = 4..7).
  auto issue_block = [&](const CopyPlan& p, int r, __bf16* qs, __bf16* ds) {
    char* dst = reinterpret_cast<char*>(r < 4 ? qs : ds) + (4 * wave + (r & 3)) * 1024;
    buffer_load_lds16(make_rsrc32(r < 4 ? p.q : p.d, p.bytes), dst, coff[r & 3]);
  };
  auto issue = [&](const CopyPlan& p, __bf16* qs, __bf16* ds, float* xs) {
    issue_row(p, xs);
#pragma unroll
    for (int r = 0; r < 8; ++r) issue_block(p, r, qs, ds);
  };
  CopyPlan pend{};  // the tile whose row blocks the step's first phase issues
  __bf16* pend_q = nullptr;
  __bf16* pend_d = nullptr;
  constexpr int kCopiesPerTile = 9;
  static_assert(kCopiesPerTile == 2 * (QT / 4 / 4) + 1, "copy count per wave and tile");

  // The LSE row of a tile is used as -LSE * log2(e) (the exponent of P in base 2).
  // Wave 0, which copied it, rescales it in place one step before the tile is
  // used: it reads the row at the start of step t (after waiting for its copy of
  // tile t+1's row, which precedes that tile's 8 row-block copies and tile t+2's
  // row, if any) and writes it back after step t's arithmetic; the barrier of step
  // t+1 publishes it.  Saves 32 multiplications per lane and tile in the other waves.
  auto rescale_wait = [&](bool next2) {
    if (next2)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
  };

  // LDS operand offsets.  Q and dO rows (A of S = Q K^T, dP = dO V^T): row
  // 32*qb + key_of_row(col), 16-byte chunk 2c+half, i.e. 8192*qb + (rA ^ (c << 5)).
  // dO^T and Q^T (B of dV += P^T dO, dK += dS^T Q) by transposing reads of rows
  // 32*qb + 16*half + 8m + k (+4): per-lane bases B0 (rows +k) and B1 (rows +4+k);
  // column block db selects bits 6-7 by XOR, m and qb add 2048 and 8192 bytes.
  const int rA = row_read_base(lane);
  const TrBases trb = tr_bases(lane);
  const int tB0 = trb.b0, tB1 = trb.b1;
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  auto tr_read = [](const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
  };

  // One 64-query tile = two 32-query blocks against the wave's 32 keys.  Per block:
  // score MFMAs (S = Q K^T, dP = dO V^T; lane = key, register i of half h = query
  // q0 + 16h + i), per element P = exp(S - LSE) and dS = P (dP - delta) on the
  // vector ALU, then gradient MFMAs (dV += P^T dO, dK += dS^T Q).  With one wave per
  // SIMD the vector ALU only runs beside the matrix unit if the instruction stream
  // interleaves them and the vector instructions between two MFMAs do not depend on
  // one another, so the tile is one straight-line body of 64 MFMA slots pinned with
  // scheduling fences, and each element passes through three stages in three
  // consecutive slots (B: the exponent S*scale*log2(e) - LSE*log2(e) and, in the
  // masked body, the mask; C: exp2; D: -dS = P * (delta - dP)):
  //   P1: block 0 scores                  | block 1 operand reads
  //   P2: block 1 scores                  | block 0 elements, dO^T/Q^T reads
  //   P3: block 0 gradients               | block 1 elements (and block 0's last 2)
  //   P4: block 1 gradients               | block 1's last 2 elements
  // The score MFMAs write vector registers (read by the stages directly); the
  // gradient MFMAs accumulate dK and dV in AGPRs through inline asm (mfma_acc), since
  // the compiler gives all MFMAs of a function one register form.  A slot then holds
  // at most six independent vector instructions besides its MFMA.
  // The masked body (kMask) sets the exponent of every invisible element to -inf, so
  // P and dS are exactly 0 there: the causal rule, the ends of the query shard and
  // of the chunk and, for packed rows, the segment test.  P uses the final LSE as
  // is: a query whose LSE is -inf sees no key at all, so it only occurs in masked
  // tiles, where its elements are invisible.
  auto compute = [&](auto mask_tag, int it, const __bf16* qt_, const __bf16* dt_, const float* xs) {
    constexpr bool kMask = decltype(mask_tag)::value;
    int hq_unused, qt_cur;
    walk_tile(compute_walk, hq_unused, qt_cur);
    walk_next(compute_walk);
    const int qtile0 = qt_cur * QT;
    const char* qc = reinterpret_cast<const char*>(qt_);
    const char* dc = reinterpret_cast<const char*>(dt_);
    f32x16 s[2], dp[2];                   // S and delta - dP of the two blocks (vector registers)
    bf16x8 fq[2][8], fd[2][8];            // A operands of the score MFMAs
    bf16x8 dot[2][2][4], qtf[2][2][4];    // [qb][m][db]: dO^T and Q^T operands
    bf16x8 pf[2][2], sf[2][2];            // [qb][m]: packed P and -dS, elements 8m..8m+7
    float lq[2][16];                      // -LSE*log2(e) of the block's queries
    f32x16 dlv[2];                        // delta of the block's queries: the dP chain's start
    int sgq[2][16];                       // segment ids of the block's queries (packed rows)
    float ea[2][16];                      // element pipeline register (exponent)
    float pe[2][16], de[2][16];           // P and -dS
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    auto read_op = [&](int qb, int c) {
      fq[qb][c] = load_bf16x8(qc + 8192 * qb + (rA ^ (c << 5)));
      fd[qb][c] = load_bf16x8(dc + 8192 * qb + (rA ^ (c << 5)));
    };
    auto read_delta = [&](int qb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dlv[qb][i] = xs[QT + 32 * qb + 16 * half + i];
    };
    auto read_rows = [&](int qb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        lq[qb][i] = xs[32 * qb + 16 * half + i];
        if constexpr (kMask && kSeg) sgq[qb][i] = __builtin_bit_cast(int, xs[2 * QT + 32 * qb + 16 * half + i]);
      }
    };
    auto read_tr = [&](int qb, int m, int db) {
      const int o = (tB0 ^ (db << 6)) + 2048 * m + 8192 * qb;
      const int o1 = (tB1 ^ (db << 6)) + 2048 * m + 8192 * qb;
      const bf16x4_t d0 = tr_read(dc + o), d1 = tr_read(dc + o1);
      const bf16x4_t q0v = tr_read(qc + o), q1v = tr_read(qc + o1);
      dot[qb][m][db] = bf16x8{d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
      qtf[qb][m][db] = bf16x8{q0v[0], q0v[1], q0v[2], q0v[3], q1v[0], q1v[1], q1v[2], q1v[3]};
    };
    // Element stages; the empty statements keep each stage's result in its slot.
    auto stage_b = [&](int qb, int i) {
      float x = __builtin_fmaf(s[qb][i], a.scale_log2, lq[qb][i]);
      if constexpr (kMask) {
        const int q0 = qtile0 + 32 * qb;
        bool vis = (i >= vis_lo - q0) & (i < vis_hi - q0);
        if constexpr (kSeg) vis &= sgq[qb][i] == seg_k;
        x = vis ? x : -__builtin_inff();
      }
      asm volatile("" : "+v"(x));
      ea[qb][i] = x;
    };
    auto stage_c = [&](int qb, int i) {
      float x = exp2_fast(ea[qb][i]);
      asm volatile("" : "+v"(x));
      pe[qb][i] = x;
    };
    auto stage_d = [&](int qb, int i) {
      float y = pe[qb][i] * dp[qb][i];
      asm volatile("" : "+v"(y));
      de[qb][i] = y;
    };
    // The stages of block qb that fall in its k-th element slot (k = 0 .. 17).
    auto elements = [&](int qb, int k) {
      if (k >= 2 && k < 18) stage_d(qb, k - 2);
      if (k >= 1 && k < 17) stage_c(qb, k - 1);
      if (k < 16) stage_b(qb, k);
    };
    // bf16 packing of elements 8m + 2j, 8m + 2j + 1 (j = 0 .. 3) of P and -dS.
    auto pack = [&](int qb, int m, int j) {
      const f32x2 p2 = {pe[qb][8 * m + 2 * j], pe[qb][8 * m + 2 * j + 1]};
      const f32x2 d2 = {de[qb][8 * m + 2 * j], de[qb][8 * m + 2 * j + 1]};
      const bf16x2 pb = __builtin_convertvector(p2, bf16x2);
      const bf16x2 db2 = __builtin_convertvector(d2, bf16x2);
      pf[qb][m][2 * j] = pb[0];
      pf[qb][m][2 * j + 1] = pb[1];
      sf[qb][m][2 * j] = db2[0];
      sf[qb][m][2 * j + 1] = db2[1];
    };

    // P1: block 0 scores; block 1 operand reads in their shadow.
    read_delta(0);
#pragma unroll
    for (int c = 0; c < 8; ++c) read_op(0, c);
    fence();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s[0] = mfma_bf16(fq[0][c], kf[c], c == 0 ? f32x16{} : s[0]);
      fq[1][c] = load_bf16x8(qc + 8192 + (rA ^ (c << 5)));
      if (c == 2) read_rows(0);
      if (c == 5) read_delta(1);
      issue_block(pend, c, pend_q, pend_d);  // tile it+2 (empty ranges past the last tile)
      fence();
      dp[0] = mfma_bf16(fd[0][c], vf[c], c == 0 ? dlv[0] : dp[0]);
      fd[1][c] = load_bf16x8(dc + 8192 + (rA ^ (c << 5)));
      fence();
    }
    read_rows(1);
    fence();
    // P2: block 1 scores; block 0 elements (stages up to slot 15), its m = 0
    // transposed operands, and the packing of its elements 0..7.
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int c = k / 2;
      if (k % 2 == 0)
        s[1] = mfma_bf16(fq[1][c], kf[c], c == 0 ? f32x16{} : s[1]);
      else
        dp[1] = mfma_bf16(fd[1][c], vf[c], c == 0 ? dlv[1] : dp[1]);
      elements(0, k);
      if (k < 4) read_tr(0, 0, k);
      if (k >= 10 && k < 14) pack(0, 0, k - 10);
      fence();
    }
    // P3: block 0 gradients (slot 2(4m + db): dV, slot +1: dK); block 0's last
    // stages, block 1 elements, the packing of block 0's elements 8..15 and of block
    // 1's elements 0..7; the remaining transposed operands of block 0 (m = 1) and
    // block 1's m = 0.
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int m = k / 8, db = (k / 2) % 4;
      if (k % 2 == 0)
        mfma_acc(dv[db], pf[0][m], dot[0][m][db]);
      else
        mfma_acc(dk[db], sf[0][m], qtf[0][m][db]);
      if (k < 2) elements(0, 16 + k);
      elements(1, k);
      if (k >= 2 && k < 6) pack(0, 1, k - 2);
      if (k >= 10 && k < 14) pack(1, 0, k - 10);
      if (k < 8 && k % 2 == 0) read_tr(0, 1, db);
      if (k >= 8 && k % 2 == 1) read_tr(1, 0, db);
      fence();
    }
    // P4: block 1 gradients; block 1's last stages, the packing of its elements
    // 8..15 and its m = 1 transposed operands.
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int m = k / 8, db = (k / 2) % 4;
      if (k % 2 == 0)
        mfma_acc(dv[db], pf[1][m], dot[1][m][db]);
      else
        mfma_acc(dk[db], sf[1][m], qtf[1][m][db]);
      if (k < 2) elements(1, 16 + k);
      if (k >= 2 && k < 6) pack(1, 1, k - 2);
      if (k < 8 && k % 2 == 0) read_tr(1, 1, db);
      fence();
    }
    // Wait states behind the last accumulating MFMA before any branch: on the
    // loop's exit path the compiler may copy the accumulators at once.
    mfma_acc_gap();
    fence();
  };

  // One step: wait for tile `it` (copies issued two steps ago), publish it to the
  // workgroup, start copying tile it+2 into the slot tile it-1 used, compute.
  // The barrier is a bare s_barrier: a workgroup fence would also wait for the
  // copies still in flight.  The empty asm statements keep the compiler from
  // moving LDS accesses across it; the copies of this wave are waited for
  // explicitly (vmcnt counts them in issue order).
  auto step = [&](auto mask_tag, int it, const __bf16* qc, const __bf16* dc, const float* xc, float* x1,
                  __bf16* qn, __bf16* dn, float* xn) {
    asm volatile("" ::: "memory");
    if (it + 1 < len)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCopiesPerTile));  // tile it+1 may stay in flight
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    pend = plan_copy(it + 2 < len);
    pend_q = qn;
    pend_d = dn;
    if (it + 2 < len) issue_row(pend, xn);
    const bool resc = wave == 0 && it + 1 < len;
    float lraw = 0.0f;
    if (resc) {
      rescale_wait(it + 2 < len);
      lraw = x1[lane];
    }
    compute(mask_tag, it, qc, dc, xc);
    if (resc) {
      asm volatile("" : "+v"(lraw));  // keeps the multiplication (and the wait for the read) here
      x1[lane] = lraw * -kLog2e;
    }
  };

  // Steps it = 0 .. len-1 visit positions p_begin + it.
  issue(plan_copy(true), qs0, ds0, xs0);
  if (len > 1) issue(plan_copy(true), qs1, ds1, xs1);
  if (wave == 0) {
    rescale_wait(len > 1);
    xs0[lane] = xs0[lane] * -kLog2e;
  }
  // Masked tiles first, in whole groups of three (a group that reaches into the
  // unmasked tiles runs masked: correct, only slower), so that both loops start at
  // slot 0 of the ring.
  const int n_masked_here = max(0, min(len, n_masked - p_begin));
  const int n_masked3 = min(len, (n_masked_here + 2) / 3 * 3);
  int it = 0;
  for (; it < n_masked3; it += 3) {
    step(BoolTag<true>{}, it, qs0, ds0, xs0, xs1, qs2, ds2, xs2);
    if (it + 1 < len) step(BoolTag<true>{}, it + 1, qs1, ds1, xs1, xs2, qs0, ds0, xs0);
    if (it + 2 < len) step(BoolTag<true>{}, it + 2, qs2, ds2, xs2, xs0, qs1, ds1, xs1);
  }
  for (; it < len; it += 3) {
    step(BoolTag<false>{}, it, qs0, ds0, xs0, xs1, qs2, ds2, xs2);
    if (it + 1 < len) step(BoolTag<false>{}, it + 1, qs1, ds1, xs1, xs2, qs0, ds0, xs0);
    if (it + 2 < len) step(BoolTag<false>{}, it + 2, qs2, ds2, xs2, xs0, qs1, ds1, xs1);
  }

  // The accumulators were last written by inline-asm MFMAs, which the compiler's
  // hazard tracking does not see: wait out the MFMA write latency before they are read.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(dk[0]), "+a"(dk[1]), "+a"(dk[2]), "+a"(dk[3]), "+a"(dv[0]), "+a"(dv[1]), "+a"(dv[2]),
                 "+a"(dv[3]));
  // lane = d column, register i of half h = key kw + mfma32_row(i, h).  The
  // read-modify-write of dK and dV goes in groups of 16 keys x 2 tensors so that the
  // loads of a group are in flight together (the two pointers do not alias).
  float* __restrict__ dkp = a.dk;
  float* __restrict__ dvp = a.dv;
  const float ks = -a.scale;  // dk holds -sum dS^T q (the dP chain runs on negated V)
  const int64_t base = ((int64_t)b * a.Sk + kw) * kv_rs + (int64_t)g * kD + col;
  const bool full = kw + 32 <= a.Sk;
  if (n_sp > 1) {
    // Partial sums of a split key block: each workgroup stores its accumulators,
    // then counts itself in; the one that arrives last reads all n_sp partials back
    // and adds them up in split order (the result does not depend on arrival order)
    // before the read-modify-write of dK and dV.  The partials are written through
    // to, and read from, the memory side of the per-XCD L2 caches (the sc1 cache
    // policy of agent-scope coherence), which needs no cache-wide fence; every store
    // of this wave has completed (vmcnt 0) before the workgroup barrier and the
    // count.  Layout per workgroup: [tensor][wave][db][lane][16 registers].
    constexpr int kSc1 = 16;  // cache policy bits: sc1
    const buffer_rsrc pr = make_rsrc32(reinterpret_cast<char*>(a.part) + (int64_t)kblk * a.n_split * kDkdvPartPerWg,
                                       a.n_split * (int)kDkdvPartPerWg);
    auto poff = [&](int sp, int tensor, int db, int j4) {
      return (int)(((((sp * 2 + tensor) * NW + wave) * 4 + db) * 64 + lane) * 64 + 16 * j4);
    };
    auto put = [&](const f32x16& x, int tensor, int db) {
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4 v = {x[4 * j4], x[4 * j4 + 1], x[4 * j4 + 2], x[4 * j4 + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), pr, poff(split, tensor, db, j4), 0,
                                               kSc1);
      }
    };
    auto add_from = [&](f32x16& x, int sp, int tensor, int db, bool first) {
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, poff(sp, tensor, db, j4), 0, kSc1));
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * j4 + e] = first ? v[e] : x[4 * j4 + e] + v[e];
      }
    };
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      put(dk[db], 0, db);
      put(dv[db], 1, db);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (tid == 0)
      last_flag = __hip_atomic_fetch_add(a.count + kblk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_sp - 1;
    __syncthreads();
    if (!last_flag) return;
    for (int sp = 0; sp < n_sp; ++sp)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        add_from(dk[db], sp, 0, db, sp == 0);
        add_from(dv[db], sp, 1, db, sp == 0);
      }
  }
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    float ok[16], ov[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = mfma32_row(i, half);
      const int64_t off = base + (int64_t)r * kv_rs + 32 * db;
      if (full || kw + r < a.Sk) {
        ok[i] = dkp[off];
        ov[i] = dvp[off];
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = mfma32_row(i, half);
      const int64_t off = base + (int64_t)r * kv_rs + 32 * db;
      if (full || kw + r < a.Sk) {
        dkp[off] = ok[i] + ks * dk[db][i];
        dvp[off] = ov[i] + dv[db][i];
      }
    }
  }
}

}  // namespace

// Workgroups per key block.  Key blocks that see very different numbers of query
// tiles -- the causal diagonal chunk, packed rows -- leave most CUs idle behind
// their longest block; two workgroups per block halve that block's run.  Uniform
// chunks keep one: their dQ kernel already runs beside them on the other CUs.
int dkdv_d128_split(const BwdArgs& args) {
  constexpr int NW = 4;
  const int64_t n_blk = (int64_t)args.B * args.Hkv * ((args.Sk + 32 * NW - 1) / (32 * NW));
  if (n_blk > kDkdvCounters) return 1;
  const bool diagonal =
      args.causal && args.kv_offset + args.Sk > args.q_offset && args.kv_offset < args.q_offset + args.Sq;
  int s = (args.seg != nullptr || diagonal) ? 2 : 1;
  while (s > 1 && (size_t)(s * n_blk) * kDkdvPartPerWg > kDkdvPartBytes) --s;
  return s;
}

namespace {
__global__ void zero_counts_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
}  // namespace

ra_status launch_dkdv_d128(BwdArgs args, hipStream_t stream, void* scratch) {
  constexpr int NW = 4;  // waves (x 32 keys) per workgroup
  args.n_tiles = (args.Sk + 32 * NW - 1) / (32 * NW);
  args.n_split = dkdv_d128_split(args);
  const int64_t n_blk = (int64_t)args.B * args.Hkv * args.n_tiles;
  const int64_t n_wg = n_blk * args.n_split;
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  args.count = nullptr;
  args.part = nullptr;
  if (args.n_split > 1) {
    if (!scratch) return fail(RA_ERR_INVALID_ARGUMENT, "ring_attn_bwd_step: split dK/dV needs scratch");
    // The split is sized to the scratch (dkdv_d128_split), so this holds; checked
    // because the allocation-free entry point's scratch cannot grow.
    if (n_blk > kDkdvCounters || (size_t)n_wg * kDkdvPartPerWg > kDkdvPartBytes)
      return fail(RA_ERR_INVALID_ARGUMENT,
                  "ring_attn_bwd_step: %lld key blocks x %d splits exceed the dK/dV scratch (%zu bytes)",
                  (long long)n_blk, args.n_split, kDkdvScratchBytes);
    args.count = static_cast<int*>(scratch);
    args.part = reinterpret_cast<float*>(static_cast<char*>(scratch) + kDkdvCountBytes);
    // The arrival counters start at zero (a fill kernel: no memset node in a graph).
    hipLaunchKernelGGL(zero_counts_kernel, dim3((unsigned)((n_blk + 255) / 256)), dim3(256), 0, stream, args.count,
                       (int)n_blk);
    const ra_status st = check_launch("ring_attn_bwd_step (dK/dV counters)");
    if (st != RA_OK) return st;
  }
  if (args.seg)
    hipLaunchKernelGGL((dkdv_d128_kernel<true, NW>), dim3((unsigned)n_wg), dim3(64 * NW), 0, stream, args);
  else
    hipLaunchKernelGGL((dkdv_d128_kernel<false, NW>), dim3((unsigned)n_wg), dim3(64 * NW), 0, stream, args);
  return check_launch("ring_attn_bwd_step (dK/dV)");
}

}  // namespace ra
