// gdn_kda.h -- KDA per-channel gate on gfx950.
//
// The KDA gate guide (MindSpeed-Ops issue page, "core computation logic")
// defines, per element of g [T, H, D]:
//     yg = -exp(A_log[h]) * softplus(g + dt_bias[h, d]),
//     softplus(x) = x for x > 20, else log(1 + e^x),
// evaluated in fp32 and rounded to the output dtype.
//
// softplus is gate_softplus (hardware exp2/log2 with Kahan's log1p correction).
//
// Purely elementwise and HBM-bound (2-4 bytes in and out per element, a few
// flops).  The vector kernel gives each thread 8 consecutive channels of one
// (token, head) row: one 16-byte (2-byte types) or 32-byte (fp32) load and
// store, the head's scale exp(A_log[h]) computed once for the 8, and the 8
// biases read from a 32-byte slice of dt_bias that stays in cache.  Rows are
// visited grid-stride, so any T fits one launch.  The scalar kernel covers D
// not a multiple of 8 and pointers not aligned for the vector accesses.
#pragma once
#include "gdn_common.h"

namespace gdn {

typedef _Float16 f16;

template <typename T> __device__ __forceinline__ float kda_in(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T kda_out(float x) { return (T)x; }  // RNE

template <typename T> struct Vec8;
template <> struct Vec8<float> { f32x4 a, b; };
template <> struct Vec8<bf16> { bf16x8 a; };
template <> struct Vec8<f16> { f16 a __attribute__((ext_vector_type(8))); };

template <typename T> __device__ __forceinline__ void vec8_unpack(const Vec8<T>& v, float (&x)[8]);
template <> __device__ __forceinline__ void vec8_unpack<float>(const Vec8<float>& v, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = v.a[j];
    x[4 + j] = v.b[j];
  }
}
template <> __device__ __forceinline__ void vec8_unpack<bf16>(const Vec8<bf16>& v, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)v.a[j];
}
template <> __device__ __forceinline__ void vec8_unpack<f16>(const Vec8<f16>& v, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)v.a[j];
}

template <typename T> __device__ __forceinline__ Vec8<T> vec8_pack(const float (&x)[8]);
template <> __device__ __forceinline__ Vec8<float> vec8_pack<float>(const float (&x)[8]) {
  return {f32x4{x[0], x[1], x[2], x[3]}, f32x4{x[4], x[5], x[6], x[7]}};
}
template <> __device__ __forceinline__ Vec8<bf16> vec8_pack<bf16>(const float (&x)[8]) {
  const f32x4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
  const bf16x4 a = __builtin_convertvector(lo, bf16x4), b = __builtin_convertvector(hi, bf16x4);
  return {__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7)};
}
template <> __device__ __forceinline__ Vec8<f16> vec8_pack<f16>(const float (&x)[8]) {
  Vec8<f16> v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v.a[j] = (f16)x[j];
  return v;
}

// rows = T * H rows of D channels; D % 8 == 0; g, yg aligned to sizeof(Vec8).
// Thread t of a workgroup owns vector (t % vpr) of row (t / vpr) within each
// block of rows_per_wg rows; vpr = D / 8.
// g and yg may be the same buffer (in place); they are not declared __restrict__.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void gdn_kda_gate_vec_kernel(const TI* g,
                                                               const float* __restrict__ A_log,
                                                               const float* __restrict__ dt_bias,
                                                               TO* yg, int64_t rows, int H, int D) {
  const int vpr = D >> 3;
  const int rows_per_wg = blockDim.x / vpr;
  const int tr = threadIdx.x / vpr, v = threadIdx.x - tr * vpr;
  if (tr >= rows_per_wg) return;  // threads beyond the last whole row of the block
  const int d0 = v << 3;
  const int64_t step = (int64_t)gridDim.x * rows_per_wg;
  for (int64_t r = (int64_t)blockIdx.x * rows_per_wg + tr; r < rows; r += step) {
    const int h = (int)(r % H);
    float x[8], b[8];
    vec8_unpack<TI>(*reinterpret_cast<const Vec8<TI>*>(g + r * D + d0), x);
    if (dt_bias) {
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(dt_bias + (int64_t)h * D + d0);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(dt_bias + (int64_t)h * D + d0 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j] = b0[j];
        b[4 + j] = b1[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = 0.f;
    }
    const float s = -expf(A_log[h]);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = s * gate_softplus(x[j] + b[j]);
    *reinterpret_cast<Vec8<TO>*>(yg + r * D + d0) = vec8_pack<TO>(x);
  }
}

// Any D and alignment: one element per thread per iteration.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void gdn_kda_gate_scalar_kernel(const TI* g,
                                                                  const float* __restrict__ A_log,
                                                                  const float* __restrict__ dt_bias,
                                                                  TO* yg, int64_t n, int H, int D) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += step) {
    const int64_t row = e / D;
    const int d = (int)(e - row * D);
    const int h = (int)(row % H);
    const float x = kda_in(g[e]) + (dt_bias ? dt_bias[(int64_t)h * D + d] : 0.f);
    yg[e] = kda_out<TO>(-expf(A_log[h]) * gate_softplus(x));
  }
}

}  // namespace gdn
