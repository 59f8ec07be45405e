// ring_attn_bwd_preprocess: delta_i = dO_i . O_i per (b, h, i), the row term of
// the softmax gradient dS = P o (dP - delta) used by every backward ring step.
// The backward recomputes the probabilities rather than storing them (archcrux,
// "sequence-parallel long-context attention OOM"), so only this [B, Hq, Sq]
// vector is kept beside the forward's O and LSE.
// HBM-bound: each (b, i, h) row of d values is read by a group of lanes with
// 16-byte loads and reduced with cross-lane shuffles.
#include "ra_device.h"
#include "ra_host.h"

namespace ra {
namespace {

constexpr int kThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void delta_kernel(int64_t n_rows, int Sq, int Hq, const T* __restrict__ o,
                                                         const T* __restrict__ d_o, float* __restrict__ delta) {
  constexpr int E = 16 / sizeof(T);   // elements per 16-byte load
  constexpr int L = D / E;            // lanes per row (8, 16 or 32)
  constexpr int R = kThreads / L;     // rows per workgroup pass
  const int sub = threadIdx.x % L;
  for (int64_t row = (int64_t)blockIdx.x * R + threadIdx.x / L; row < n_rows; row += (int64_t)gridDim.x * R) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + sub * E);
    const u32x4 c = *reinterpret_cast<const u32x4*>(d_o + row * D + sub * E);
    float acc = 0.0f;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc += bf16_to_f32(a[j] & 0xFFFFu) * bf16_to_f32(c[j] & 0xFFFFu);
        acc += bf16_to_f32(a[j] >> 16) * bf16_to_f32(c[j] >> 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += u32_as_f32(a[j]) * u32_as_f32(c[j]);
    }
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (sub == 0) {
      const int h = (int)(row % Hq);
      const int64_t bi = row / Hq;
      const int i = (int)(bi % Sq);
      const int64_t b = bi / Sq;
      delta[(b * Hq + h) * Sq + i] = acc;
    }
  }
}

template <typename T, int D>
void launch(int64_t n_rows, int Sq, int Hq, const void* o, const void* d_o, float* delta, hipStream_t s) {
  constexpr int R = kThreads / (D / (16 / sizeof(T)));
  const int64_t blocks = std::min<int64_t>((n_rows + R - 1) / R, 1 << 20);
  hipLaunchKernelGGL((delta_kernel<T, D>), dim3((unsigned)blocks), dim3(kThreads), 0, s, n_rows, Sq, Hq,
                     static_cast<const T*>(o), static_cast<const T*>(d_o), delta);
}

}  // namespace
}  // namespace ra

extern "C" ra_status ring_attn_bwd_preprocess(int32_t B, int32_t Sq, int32_t Hq, int32_t d, int32_t dtype,
                                              const void* o, const void* d_o, float* delta, void* stream) {
  using namespace ra;
  if (B < 1 || Sq < 1 || Hq < 1) return fail(RA_ERR_INVALID_ARGUMENT, "batch, q_len and heads_q must be >= 1");
  if (dtype != RA_DTYPE_F32 && dtype != RA_DTYPE_BF16) return fail(RA_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (d != 64 && d != 128) return fail(RA_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", d);
  if (!o || !d_o || !delta) return fail(RA_ERR_INVALID_ARGUMENT, "o, d_o and delta must be non-NULL");
  if (!aligned16(o) || !aligned16(d_o) || !aligned16(delta))
    return fail(RA_ERR_INVALID_ARGUMENT, "o, d_o and delta must be 16-byte aligned");
  const int64_t n_rows = (int64_t)B * Sq * Hq;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dtype == RA_DTYPE_BF16) {
    if (d == 128) launch<__bf16, 128>(n_rows, Sq, Hq, o, d_o, delta, hs);
    else launch<__bf16, 64>(n_rows, Sq, Hq, o, d_o, delta, hs);
  } else {
    if (d == 128) launch<float, 128>(n_rows, Sq, Hq, o, d_o, delta, hs);
    else launch<float, 64>(n_rows, Sq, Hq, o, d_o, delta, hs);
  }
  return check_launch("ring_attn_bwd_preprocess");
}
