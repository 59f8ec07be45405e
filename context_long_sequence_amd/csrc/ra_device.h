// Device-side helpers shared by the ring-attention kernels (gfx950 / CDNA4).
//
// MFMA conventions used throughout (64-lane wavefront, lane l, half h = l / 32):
//  * v_mfma_f32_32x32x16_bf16 D = A*B + C with A 32x16, B 16x32, D 32x32.
//    A: lane l holds row (l % 32), k-slots 8h .. 8h+7 (8 bf16).
//    B: lane l holds column (l % 32), k-slots 8h .. 8h+7.
//    D: lane l holds column (l % 32), rows 8*(i/4) + 4h + (i%4) for i = 0..15.
//  * v_mfma_f32_32x32x2_f32: the same with one k-slot (h) per lane.
// The contraction index can be permuted freely as long as A and B agree; the
// kernels use that to keep operands in the registers where they are produced.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Row layout helper for 32x32 MFMA outputs: row index of accumulator register i
// in a lane of half h.
__device__ __forceinline__ int mfma32_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// acc += A*B with the accumulator in AGPRs (v_mfma_f32_32x32x16_bf16 in inline asm),
// for kernels whose other MFMAs write vector registers (the compiler picks one
// register form for all MFMAs of a function).  The compiler does not see this as
// an MFMA, so the caller keeps its hazards in order: A and B written by vector ALU
// instructions at least two instructions earlier, the accumulator touched only by
// these MFMAs, and no read of it by other instructions within 20 wait states of
// the last write.
__device__ __forceinline__ void mfma_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// D = A*B + C with B in AGPRs, C and D in VGPRs (D early-clobber: it must not share
// registers with A, B or C).
__device__ __forceinline__ void mfma_vab(f32x16& d, bf16x8 a, bf16x8 b, const f32x16& c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
}
__device__ __forceinline__ void mfma_vab0(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_vab_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// Wait states between an MFMA that wrote a VGPR and the first vector instruction
// that reads it (more than the 8-pass MFMA's requirement).
__device__ __forceinline__ void mfma_read_gap() { asm volatile("s_nop 7\n\ts_nop 7"); }
// Wait states between the last of a run of MFMAs that accumulate in AGPRs and any
// other instruction that reads those AGPRs (the 16-pass requirement, with margin).
__device__ __forceinline__ void mfma_acc_gap() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"); }

// Negation of 8 bf16 values (sign bits flipped: exact).
__device__ __forceinline__ bf16x8 neg_bf16x8(bf16x8 v) {
  const u32x4 m = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  return __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, v) ^ m);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even conversion of 8 floats to bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7) {
  f32x2 p0 = {a0, a1}, p1 = {a2, a3}, p2 = {a4, a5}, p3 = {a6, a7};
  bf16x2 r0 = __builtin_convertvector(p0, bf16x2);
  bf16x2 r1 = __builtin_convertvector(p1, bf16x2);
  bf16x2 r2 = __builtin_convertvector(p2, bf16x2);
  bf16x2 r3 = __builtin_convertvector(p3, bf16x2);
  bf16x8 out = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  return out;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const void* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void store_bf16x8(void* p, bf16x8 v) {
  *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}

// Reinterprets 32 bits as a float.  Takes the value (not a vector-element lvalue):
// bit-casting an ext_vector element in place reads the wrong element with this
// compiler, so callers always go through this by-value helper.
__device__ __forceinline__ float u32_as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(x) << 16);
}

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  static constexpr int KPL = 8;  // contraction values per lane per instruction
  using frag = bf16x8;
  static __device__ __forceinline__ frag load(const __bf16* p) { return load_bf16x8(p); }
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) { return mfma_bf16(a, b, c); }
  static __device__ __forceinline__ frag pack(const float* p) {
    return to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
  }
};

template <>
struct Mfma<float> {
  static constexpr int KPL = 1;
  using frag = float;
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) { return mfma_f32(a, b, c); }
  static __device__ __forceinline__ frag pack(const float* p) { return p[0]; }
};

// Row of the K tile that feeds accumulator row r of a 32-key block, chosen so
// that accumulator register i of half-wave h holds key 16h + i.
__host__ __device__ __forceinline__ int key_of_row(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// ---- LDS tiles of 128-element bf16 rows (256 B per row, no padding) ------------------
// The 16 chunks of 16 bytes of row r are stored XOR-swizzled at chunk position
// c ^ swz(r), swz(r) = 4*(r & 3) + 2*((r >> 2) & 1) + ((r >> 4) & 1).  Both operand
// read patterns of the kernels are then conflict-free: 16 lanes reading one logical
// chunk of rows {0-3, 16-19, 4-7, 20-23} (or the +8 set) with 16-byte reads, and 32
// lanes of transposing 8-byte reads covering 4 consecutive rows x 64 bytes (the
// (r & 3) << 2 term spreads those 4 rows over all 64 banks).  Rows are filled by
// direct global->LDS loads (lane l of a wave writes bytes [16l, 16l+16) of a 1 KiB
// block = 4 rows), so the swizzle is applied on the global side by choosing which
// chunk each lane fetches.
typedef __attribute__((address_space(3))) void* lds_void_ptr;

__host__ __device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | (((row >> 2) & 1) << 1) | ((row >> 4) & 1); }

__host__ __device__ __forceinline__ int tile_off(int row, int chunk) { return row * 256 + ((chunk ^ swz(row)) << 4); }

// Byte offsets of the two MFMA operand reads of such tiles.
//
// Row reads (16 bytes): lane l reads chunk 2s + l/32 of row key_of_row(l % 32) (plus
// a multiple of 32 rows); its offset is row_read_base(l) ^ (s << 5).
__host__ __device__ __forceinline__ int row_read_base(int lane) {
  const int r = key_of_row(lane & 31), h = lane >> 5;
  return r * 256 + 32 * (2 * (r & 3) + ((r >> 2) & 1)) + 16 * (h ^ ((r >> 4) & 1));
}
// Transposing reads (ds_read_b64_tr_b16): within a group of 16 lanes, lane j
// receives element j % 4 of the 8-byte words addressed by lanes j/4 + 4k (k = 0..3).
// Addressing row r0 + k at columns c0 + 4m .. +3 from lane m + 4k therefore hands
// lane j rows r0 .. r0+3 of column c0 + j.  Two reads (rows +0..3, +4..7) give lane l
// the 8 bf16 of one MFMA operand: column 32*db + l % 32 of rows 16*(l/32) + 8m ..
// +7 (plus a multiple of 32 rows).  With the swizzle above their offsets are
// (b0 ^ (db << 6)) + 2048*m and (b1 ^ (db << 6)) + 2048*m.
struct TrBases {
  int b0, b1;
};
__host__ __device__ __forceinline__ TrBases tr_bases(int lane) {
  const int s16 = lane & 15, mm = s16 & 3, kk = s16 >> 2, h = lane >> 5;
  const int x = 2 * ((lane >> 4) & 1) + (mm >> 1);
  const int sub8 = 8 * (mm & 1);
  return TrBases{(16 * h + kk) * 256 + 64 * kk + 16 * (x ^ h) + sub8,
                 (16 * h + 4 + kk) * 256 + 64 * kk + 16 * (x ^ (2 + h)) + sub8};
}

// Combines the two half-waves: lane l and lane l^32 both get op(x[l mod 32],
// x[32 + l mod 32]) (v_permlane32_swap: one VALU op, no LDS round trip).
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource (gfx9 layout: stride 0, range checked per byte offset).
// Loads whose 16 bytes end past `bytes` return zeros instead of touching memory.
typedef __amdgpu_buffer_rsrc_t buffer_rsrc;
__device__ __forceinline__ buffer_rsrc make_rsrc(const void* base, int64_t bytes) {
  const int n = (int)(bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
// The same for a range known to lie in [0, 2^31).
__device__ __forceinline__ buffer_rsrc make_rsrc32(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 4 bytes per lane from base + voffset into LDS at dst + 4*lane (dst wave-uniform).
__device__ __forceinline__ void buffer_load_lds4(buffer_rsrc rs, void* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)dst, 4, voffset, 0, 0, 0);
}
// 16 bytes per lane from base + voffset into LDS at dst + 16*lane (dst wave-uniform).
__device__ __forceinline__ void buffer_load_lds16(buffer_rsrc rs, void* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)dst, 16, voffset, 0, 0, 0);
}

// Merge of two partial results of the same query row over disjoint key sets: the
// running (L, O) and a step's (Ls, Os), log-sum-exps in natural log.  With
// M = max(L, Ls): L' = M + ln(e^(L-M) + e^(Ls-M)), O' = e^(L-L') O + e^(Ls-L') Os.
// Both -inf (no key seen yet): `live` is false and the pair stays as it is.  The
// merge kernel and the forward step's fused epilogue share these two functions, so
// both give the same bits.
struct MergeWeights {
  float w, ws, inv, lse;
  bool live;
};
__device__ __forceinline__ MergeWeights merge_weights(float L, float Ls) {
  MergeWeights r;
  // fmaxf drops a NaN operand; a NaN log-sum-exp (NaN inputs) must reach the result
  // instead of being taken for the identity when the other side is -inf.
  const bool nan_in = __builtin_isnan(L) || __builtin_isnan(Ls);
  const float m = nan_in ? __builtin_nanf("") : fmaxf(L, Ls);
  r.live = m != -INFINITY;
  if (!r.live) {
    r.w = r.ws = r.inv = 0.0f;
    r.lse = -INFINITY;
    return r;
  }
  r.w = __expf(L - m);    // 0 when L = -inf
  r.ws = __expf(Ls - m);  // 0 when Ls = -inf
  const float tot = r.w + r.ws;
  r.inv = 1.0f / tot;
  r.lse = m + __logf(tot);
  return r;
}
__device__ __forceinline__ f32x4 merge_o(f32x4 o, f32x4 os, const MergeWeights& mw) {
  const f32x4 term_s = os * (mw.ws * mw.inv);
  return (mw.w == 0.0f) ? term_s : (mw.ws == 0.0f ? o : o * (mw.w * mw.inv) + term_s);
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 o) {
  const f32x2 p0 = {o[0], o[1]}, p1 = {o[2], o[3]};
  const bf16x2 r0 = __builtin_convertvector(p0, bf16x2);
  const bf16x2 r1 = __builtin_convertvector(p1, bf16x2);
  return bf16x4{r0[0], r0[1], r1[0], r1[1]};
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).  waitcnt_vm(n): at most n vector-memory operations outstanding;
// waitcnt_vm_lgkm0(n): the same and no LDS operation outstanding.
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int waitcnt_vm_lgkm0(int n) { return 0x0070 | (n & 15) | ((n >> 4) << 14); }

// Workgroup -> XCD remap.  Consecutive workgroup ids are dispatched round-robin
// over the 8 XCDs of an MI355X; this returns a logical id such that each XCD
// receives one contiguous range of logical ids (so workgroups that share K/V
// tiles share that XCD's L2).  A bijection on [0, n).
__device__ __forceinline__ int xcd_logical_id(int w, int n) {
  constexpr int kXcd = 8;
  const int xcd = w % kXcd;
  const int local = w / kXcd;
  const int base = n / kXcd, rem = n % kXcd;
  // XCD x owns base + (x < rem) ids; its range starts at x*base + min(x, rem).
  return xcd * base + min(xcd, rem) + local;
}

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

// Token spans of the segments of a wave's tokens [t_first, t_last] of a row of `n`
// nondecreasing segment ids: the segments s0 of t_first and s1 of t_last, and their
// spans [lo0, hi0), [lo1, hi1).  Wave-collective (call with every lane active and
// wave-uniform arguments): the four bounds are found by 64-way searches run side by
// side, in which each lane tests one point of the remaining range per round -- a few
// dependent rounds of loads instead of a binary search's one load per halving.
struct SegSpans {
  int s0, s1;
  int64_t lo0, hi0, lo1, hi1;
};
__device__ __forceinline__ SegSpans seg_spans_wave(const int32_t* row, int64_t n, int64_t t_first, int64_t t_last) {
  const int lane = threadIdx.x & 63;
  SegSpans r;
  r.s0 = row[t_first];
  r.s1 = row[t_last];
  // bound k is the first index whose id is >= s (k even) or > s (k odd), s = s0 for
  // k < 2, s1 otherwise; it lies in [L[k], H[k]], narrowed by the tokens themselves.
  int64_t L[4] = {0, t_first + 1, 0, t_last + 1};
  int64_t H[4] = {t_first, n, t_last, n};
  for (int round = 0; round < 12; ++round) {
    bool active = false;
    int64_t step[4], p[4];
    int v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      active |= L[k] < H[k];
      step[k] = (H[k] - L[k] + 63) / 64;
      p[k] = L[k] + (int64_t)lane * step[k];
    }
    if (!active) break;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = (L[k] < H[k] && p[k] < H[k]) ? row[p[k]] : 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (L[k] >= H[k]) continue;
      const int sk = k < 2 ? r.s0 : r.s1;
      const bool t = p[k] >= H[k] || ((k & 1) ? v[k] > sk : v[k] >= sk);
      const uint64_t m = __ballot(t);
      if (m == 0) {
        L[k] = L[k] + 63 * step[k] + 1;  // past the last point tested
      } else {
        const int j = (int)__builtin_ctzll(m);
        const int64_t hj = L[k] + (int64_t)j * step[k];
        if (j == 0) {
          H[k] = L[k];
        } else {
          const int64_t l_new = L[k] + (int64_t)(j - 1) * step[k] + 1;
          H[k] = hj < H[k] ? hj : H[k];
          L[k] = l_new;
        }
      }
    }
  }
  r.lo0 = L[0];
  r.hi0 = L[1];
  r.lo1 = L[2];
  r.hi1 = L[3];
  return r;
}

// Token span [lo, hi) of segment `s` in a row of `n` nondecreasing segment ids:
// lo = first index with id >= s, hi = first index with id > s (binary searches).
// With ids that decrease somewhere the span is some range inside [0, n] (never an
// access outside the row).
__device__ __forceinline__ void seg_span(const int32_t* row, int64_t n, int s, int64_t& lo, int64_t& hi) {
  int64_t a = 0, b = n;
  while (a < b) {
    const int64_t m = (a + b) >> 1;
    if (row[m] < s)
      a = m + 1;
    else
      b = m;
  }
  lo = a;
  b = n;
  while (a < b) {
    const int64_t m = (a + b) >> 1;
    if (row[m] <= s)
      a = m + 1;
    else
      b = m;
  }
  hi = a;
}

// The span [lo, hi) of segment `s` of one of the wave's tokens, from the wave's
// spans when s is the segment of its first or last token, else by seg_span (a block
// of three or more samples).
__device__ __forceinline__ void seg_span_lane(const int32_t* row, int64_t n, const SegSpans& w, int s, int64_t& lo,
                                              int64_t& hi) {
  if (s == w.s0) {
    lo = w.lo0;
    hi = w.hi0;
  } else if (s == w.s1) {
    lo = w.lo1;
    hi = w.hi1;
  } else {
    seg_span(row, n, s, lo, hi);
  }
}

}  // namespace ra
