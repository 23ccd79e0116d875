// gdn_decode.h -- recurrent (token-by-token) GDN step on gfx950, for decoding.
//
// The Ascend GDN blog ("GDN sequence structure and Triton introduction")
// describes the state as updated once per arriving token.  Per token t of a
// sequence and value head (a = e^{g_t}, g_t the gated decay of the KDA gate
// guide's formula in its per-head form):
//     p   = H^T k_t                      (H = S^T, K x V, fp32)
//     H  <- a H + beta_t k_t (v_t - a p)^T
//     o_t = scale * H^T q_t
// The state is read from and written back to the caller's [N][HV][K][V] fp32
// tensor -- the layout gdn_fwd's initial and final states use -- and lives
// in registers across the call's T tokens.
//
// One workgroup per (sequence, value head, 64 value columns); lane j of each of
// the four waves owns column j, wave w owns rows [w K/4, (w+1) K/4).  Row
// segments of the state are 256 contiguous bytes per wave (coalesced).  The two
// contractions over K (p, o) are summed across the waves through LDS: three
// workgroup barriers per token.  HBM-bound: 2 K V x 4 bytes of state per
// (sequence, head) per call, plus the token's q, k, v, o.
#pragma once
#include "gdn_common.h"

namespace gdn {

template <typename E, int K, int V>
__global__ __launch_bounds__(256) void gdn_decode_kernel(Geo geo, const E* __restrict__ q,
                                                         const E* __restrict__ k,
                                                         const E* __restrict__ v,
                                                         const float* __restrict__ g_raw,
                                                         const float* __restrict__ beta,
                                                         const float* __restrict__ A_log,
                                                         const float* __restrict__ dt_bias,
                                                         float* __restrict__ state,
                                                         E* __restrict__ o) {
  constexpr int R = K / 4;        // rows per wave
  constexpr int NCB = V / 64;     // 64-column blocks per head
  __shared__ float sk[K], sq[K], sp[4][64], so[4][64];
  const int b = blockIdx.x;
  const int cb = b % NCB, hv = (b / NCB) % geo.HV, n = b / (NCB * geo.HV);
  const int h = hv / geo.G;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = 64 * cb + lane, row0 = wave * R;
  float* st = state + (((size_t)n * geo.HV + hv) * K + row0) * V + j;

  float Hs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) Hs[r] = st[(size_t)r * V];
  const float decay_scale = -expf(A_log[hv]);
  const float bias = dt_bias ? dt_bias[hv] : 0.f;

  for (int t = 0; t < geo.T; ++t) {
    const size_t tok = (size_t)n * geo.T + t;
    if (threadIdx.x < K) sk[threadIdx.x] = (float)k[(tok * geo.H + h) * K + threadIdx.x];
    else if (threadIdx.x < 2 * K) sq[threadIdx.x - K] = (float)q[(tok * geo.H + h) * K + threadIdx.x - K];
    const float a = expf(decay_scale * gate_softplus(g_raw[tok * geo.HV + hv] + bias));
    const float bt = beta[tok * geo.HV + hv];
    const float vj = (float)v[(tok * geo.HV + hv) * V + j];
    __syncthreads();
    float pp = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) pp += Hs[r] * sk[row0 + r];
    sp[wave][lane] = pp;
    __syncthreads();
    const float p = sp[0][lane] + sp[1][lane] + sp[2][lane] + sp[3][lane];
    const float c = bt * (vj - a * p);
    float po = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      Hs[r] = a * Hs[r] + sk[row0 + r] * c;
      po += Hs[r] * sq[row0 + r];
    }
    so[wave][lane] = po;
    __syncthreads();
    if (wave == 0)
      o[(tok * geo.HV + hv) * V + j] =
          (E)(geo.scale * (so[0][lane] + so[1][lane] + so[2][lane] + so[3][lane]));
  }
#pragma unroll
  for (int r = 0; r < R; ++r) st[(size_t)r * V] = Hs[r];
}

}  // namespace gdn
