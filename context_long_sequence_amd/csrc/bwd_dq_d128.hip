// dQ of one backward ring step for the hot shape (bf16, head_dim 128):
//   dQ_i += scale * sum_j P_ij (dP_ij - delta_i) k_j,  P recomputed from the final
// log-sum-exp (archcrux, "sequence-parallel long-context attention OOM").
// 4 waves x 32 queries of one query head walk the key tiles of the chunk; K and
// V tiles are copied global -> LDS (swizzled, row-major; raw buffer loads, no
// staging registers) two steps ahead into a ring of three slots, and the K^T
// operands of dQ^T += K^T dS^T come from transposing reads of the same K tile.
#include "bwd_d128.h"

#include <mutex>

namespace ra {
namespace {

constexpr int kD = kD128;
constexpr int kTile = kD128Tile;

// ------------------------------------------------------------------------------------
// dQ: 4 waves x 32 queries of one query head; walks the key tiles of the chunk.
// ------------------------------------------------------------------------------------
constexpr int kDqWaves = 4;  // waves (x 32 queries) per workgroup
static_assert(kDqWaves == 4 || kDqWaves == 8, "a 32-row tile is 8 blocks of 1 KiB, split evenly over the waves");
constexpr int kDqBlocks = 8 / kDqWaves;  // 1 KiB blocks of a tile copied by each wave
constexpr int kDqThreads = 64 * kDqWaves;

template <bool kSeg>
__global__ __launch_bounds__(kDqThreads) void dq_d128_kernel(BwdArgs a) {
  // Three K and three V tile slots, each its own array (see the copy loop below).
  __shared__ __attribute__((aligned(1024))) __bf16 ks0[kTile * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ks1[kTile * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 ks2[kTile * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 vs0[kTile * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 vs1[kTile * kD];
  __shared__ __attribute__((aligned(1024))) __bf16 vs2[kTile * kD];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
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

  const int64_t q_rs = (int64_t)a.Hq * kD;
  const int kv_rb = a.Hkv * kD * 2;  // bytes between consecutive keys
  const char* kbase = static_cast<const char*>(a.k) + ((int64_t)b * a.Sk * a.Hkv + g) * (kD * 2);
  const char* vbase = static_cast<const char*>(a.v) + ((int64_t)b * a.Sk * a.Hkv + g) * (kD * 2);

  int n_keys = a.Sk;
  if (a.causal) {
    const int64_t last_visible = a.q_offset + q_last - a.kv_offset;
    n_keys = (int)max<int64_t>(0, min<int64_t>((int64_t)a.Sk, last_visible + 1));
  }
  int kt_begin = 0, kt_end = (n_keys + kTile - 1) / kTile;
  int seg_q = 0;
  int seg_w_lo = 0, seg_w_hi = 0;  // segment ids of the wave's first and last query
  const int32_t* seg_row = nullptr;
  if constexpr (kSeg) {
    seg_row = a.seg + (int64_t)b * a.seg_len;
    const int lo = seg_row[a.q_offset + q0], hi = seg_row[a.q_offset + q_last];
    seg_q = q_valid ? seg_row[a.q_offset + qi] : lo;
    seg_w_lo = seg_row[a.q_offset + min(qw, a.Sq - 1)];
    seg_w_hi = seg_row[a.q_offset + min(qw + 32, a.Sq) - 1];
    int sb, se;
    seg_tile_range(seg_row + a.kv_offset, a.Sk, kTile, 0, kt_end, lo, hi, sb, se);
    kt_begin = sb;
    kt_end = max(sb, se);
  }
  // A workgroup without a live tile adds exactly zero to every accumulator: done.
  if (kt_begin >= kt_end) return;

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
  // The dP^T chain starts from -delta (every register of the lane holds its query's
  // -delta), so it yields dP - delta with no subtraction per element.
  f32x16 neg_dl16;
#pragma unroll
  for (int i = 0; i < 16; ++i) neg_dl16[i] = -dl;

  // Visibility of key k0 + 16*half + i: i <= lim_base - k0 (causal rule, clamped to
  // +-2^30 so that 32-bit arithmetic is exact; rows past Sq see nothing) and
  // i <= Sk - 1 - k0 - 16*half (chunk end).
  int lim_base = 1 << 30;
  if (!q_valid)
    lim_base = -(1 << 30);
  else if (a.causal)
    lim_base = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, qg - a.kv_offset - 16 * half));

  // The last chunk key the wave's first query sees (same clamp): tiles past it
  // need the element mask.
  const int wave_last_visible =
      (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, a.q_offset + qw - a.kv_offset));

  f32x16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dq[db] = f32x16{};

  // Copies: 32 rows x 256 bytes per tile and tensor = 8 blocks of 1 KiB, 8 / waves per
  // wave; lane l of a block writes 16 bytes at 16*l, so it fetches the global chunk
  // that the swizzle puts there.  Raw buffer loads with a per-tile descriptor whose
  // range ends at the chunk's last key: rows past it read as zeros (and are masked).
  uint32_t coff[kDqBlocks];
#pragma unroll
  for (int r = 0; r < kDqBlocks; ++r) {
    const int row = (kDqBlocks * wave + r) * 4 + (lane >> 4);
    coff[r] = (uint32_t)(row * kv_rb + ((lane & 15) ^ swz(row)) * 16);
  }
  auto issue = [&](int t, __bf16* kdst, __bf16* vdst) {
    const int k0 = t * kTile;
    // Through the tile's last valid key row; < 2^31 since kv_rb <= 4096 * 256.
    const int bytes = (min(a.Sk - k0, kTile) - 1) * kv_rb + kD * 2;
    const buffer_rsrc rk = make_rsrc32(kbase + (int64_t)k0 * kv_rb, bytes);
    const buffer_rsrc rv = make_rsrc32(vbase + (int64_t)k0 * kv_rb, bytes);
    char* dk = reinterpret_cast<char*>(kdst) + kDqBlocks * wave * 1024;
    char* dv = reinterpret_cast<char*>(vdst) + kDqBlocks * wave * 1024;
#pragma unroll
    for (int r = 0; r < kDqBlocks; ++r) buffer_load_lds16(rk, dk + r * 1024, coff[r]);
#pragma unroll
    for (int r = 0; r < kDqBlocks; ++r) buffer_load_lds16(rv, dv + r * 1024, coff[r]);
  };
  constexpr int kCopiesPerTile = 2 * kDqBlocks;  // per wave: K and V

  // LDS operand offsets.  K and V rows (A of S^T = K Q^T, dP^T = V dO^T): row
  // key_of_row(col), 16-byte chunk 2s+half, i.e. kA ^ (s << 5).  K^T (A of
  // dQ^T += K^T dS^T) by transposing reads of rows 16*half + 8m + k (+4): per-lane
  // bases B0 (rows +k) and B1 (rows +4+k); column block db selects bits 6-7 by XOR,
  // m adds 2048 bytes.
  const int kA = row_read_base(lane);
  const TrBases trb = tr_bases(lane);
  const int tB0 = trb.b0, tB1 = trb.b1;
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  auto tr_read = [](const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p));
  };

  auto compute = [&](int t, const __bf16* kt_, const __bf16* vt_) {
      const int k0 = t * kTile;
      bool partial = (k0 + kTile > a.Sk) || (qw + 32 > a.Sq);  // wave-uniform
      if (a.causal) partial |= (k0 + kTile - 1 > wave_last_visible);
      if constexpr (kSeg) {
        // Segment ids are nondecreasing: only blocks that straddle a segment
        // boundary need the per-element segment test.
        const int sk_lo = seg_row[a.kv_offset + k0];
        const int sk_hi = seg_row[a.kv_offset + min(k0 + kTile, a.Sk) - 1];
        partial |= !(sk_lo == sk_hi && sk_lo == seg_w_lo && seg_w_lo == seg_w_hi);
      }
      const char* kb = reinterpret_cast<const char*>(kt_);
      const char* vb = reinterpret_cast<const char*>(vt_);

      // S^T = K Q^T and dP^T = V dO^T; register i of half h = key k0 + 16h + i.
      f32x16 st = f32x16{}, dpt = neg_dl16;
      {
        bf16x8 fk[8], fv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) fk[s] = load_bf16x8(kb + (kA ^ (s << 5)));
#pragma unroll
        for (int s = 0; s < 8; ++s) fv[s] = load_bf16x8(vb + (kA ^ (s << 5)));
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          st = mfma_bf16(fk[s], qf[s], st);
          dpt = mfma_bf16(fv[s], dof[s], dpt);
        }
      }
      float p[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = exp2_fast(__builtin_fmaf(st[i], a.scale_log2, neg_lse2));
      if (partial) {  // one wave-uniform branch around the element mask
        const int lim = min(lim_base - k0, a.Sk - 1 - k0 - 16 * half);
        if constexpr (kSeg) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            // Wave-uniform addresses (scalar loads), clamped into the chunk.
            const int s_lo = seg_row[a.kv_offset + min(k0 + i, a.Sk - 1)];
            const int s_hi = seg_row[a.kv_offset + min(k0 + 16 + i, a.Sk - 1)];
            const bool vis = (i <= lim) & ((half ? s_hi : s_lo) == seg_q);
            p[i] = vis ? p[i] : 0.0f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) p[i] = (i <= lim) ? p[i] : 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = p[i] * dpt[i];
      // dQ^T += K^T dS^T: K^T rows (keys 16h + 8m + j) by transposing reads of the K tile.
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 sf = to_bf16x8(ds[8 * m], ds[8 * m + 1], ds[8 * m + 2], ds[8 * m + 3], ds[8 * m + 4],
                                    ds[8 * m + 5], ds[8 * m + 6], ds[8 * m + 7]);
        bf16x8 kt[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x4_t x0 = tr_read(kb + (tB0 ^ (db << 6)) + 2048 * m);
          const bf16x4_t x1 = tr_read(kb + (tB1 ^ (db << 6)) + 2048 * m);
          kt[db] = bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) dq[db] = mfma_bf16(kt[db], sf, dq[db]);
      }
  };

  // One step: wait for tile t (copies issued two steps ago), publish it, start
  // copying tile t+2 into the slot of tile t-1, compute.  Bare s_barrier (a
  // workgroup fence would also drain the copies in flight); the empty asm
  // statements keep the compiler from moving LDS accesses across it.
  auto step = [&](int t, const __bf16* kc, const __bf16* vc, __bf16* kn, __bf16* vn) {
    if (t + 1 < kt_end)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kCopiesPerTile));  // tile t+1 may stay in flight
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + 2 < kt_end) issue(t + 2, kn, vn);
    compute(t, kc, vc);
  };

  if (kt_begin < kt_end) {
    issue(kt_begin, ks0, vs0);
    if (kt_begin + 1 < kt_end) issue(kt_begin + 1, ks1, vs1);
    for (int t = kt_begin; t < kt_end; t += 3) {
      step(t, ks0, vs0, ks2, vs2);
      if (t + 1 < kt_end) step(t + 1, ks1, vs1, ks0, vs0);
      if (t + 2 < kt_end) step(t + 2, ks2, vs2, ks1, vs1);
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

}  // namespace

ra_status launch_dq_d128(BwdArgs args, hipStream_t stream) {
  args.n_tiles = (args.Sq + 32 * kDqWaves - 1) / (32 * kDqWaves);
  const int64_t n_wg = (int64_t)args.B * args.Hq * args.n_tiles;
  if (n_wg > INT32_MAX) return fail(RA_ERR_INVALID_ARGUMENT, "too many workgroups");
  if (args.seg)
    hipLaunchKernelGGL((dq_d128_kernel<true>), dim3((unsigned)n_wg), dim3(kDqThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((dq_d128_kernel<false>), dim3((unsigned)n_wg), dim3(kDqThreads), 0, stream, args);
  return check_launch("ring_attn_bwd_step (dQ)");
}

// One side stream per device (default priority, non-blocking) with a fork and a
// join event.  The dQ kernel of a step runs there while the dK/dV kernel of the
// same step runs on the caller's stream: the two read the same inputs and write
// disjoint outputs, and when one of them leaves CUs idle (a small grid, the
// uneven causal diagonal) the other fills them.  dK/dV, the longer of the two, is
// queued first so that its workgroups are placed first.  The caller's stream
// waits on the join, so the step is complete in that stream's order like a single
// launch.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
std::mutex g_side_mutex;

ra_status side_stream_locked(SideStream*& out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(RA_ERR_HIP, "ring_attn_bwd_step: no current device");
  SideStream& ss = g_side[dev];
  if (!ss.stream) {
    if (hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
      return fail(RA_ERR_HIP, "ring_attn_bwd_step: side stream creation failed");
  }
  out = &ss;
  return RA_OK;
}

bool bwd_d128_needs_scratch(const BwdArgs& args) {
  return dkdv64_d128_workgroups(args) < 256 && dkdv_d128_split(args) > 1;
}

ra_status launch_bwd_d128(BwdArgs args, hipStream_t stream, void* scratch, bool side) {
  // dK/dV: 64 keys per wave (half the LDS operand bytes per MFMA) when that grid
  // still gives each of the 256 CUs a workgroup; 32 keys per wave on small chunks,
  // with the query tiles of a key block split over two workgroups where the blocks'
  // work is uneven.  dQ: 64 queries per wave on the same condition.
  auto dkdv = [&](hipStream_t s) {
    return dkdv64_d128_workgroups(args) >= 256 ? launch_dkdv64_d128(args, s) : launch_dkdv_d128(args, s, scratch);
  };
  auto dq = [&](hipStream_t s) {
    return dq64_d128_workgroups(args) >= 256 ? launch_dq64_d128(args, s) : launch_dq_d128(args, s);
  };
  if (!side) {
    const ra_status st = dkdv(stream);
    return st != RA_OK ? st : dq(stream);
  }
  std::lock_guard<std::mutex> lock(g_side_mutex);
  SideStream* ss = nullptr;
  ra_status st = side_stream_locked(ss);
  if (st != RA_OK) return st;
  if (hipEventRecord(ss->fork, stream) != hipSuccess || hipStreamWaitEvent(ss->stream, ss->fork, 0) != hipSuccess)
    return fail(RA_ERR_HIP, "ring_attn_bwd_step: fork to the side stream failed");
  st = dkdv(stream);
  if (st != RA_OK) return st;
  st = dq(ss->stream);
  if (st != RA_OK) return st;
  if (hipEventRecord(ss->join, ss->stream) != hipSuccess || hipStreamWaitEvent(stream, ss->join, 0) != hipSuccess)
    return fail(RA_ERR_HIP, "ring_attn_bwd_step: join from the side stream failed");
  return RA_OK;
}

}  // namespace ra
