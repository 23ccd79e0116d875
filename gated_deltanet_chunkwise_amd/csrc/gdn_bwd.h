// gdn_bwd.h -- chunkwise backward pass of the gated delta rule on gfx950.
//
// The pages name the backward kernels (a per-chunk dv, the dq/dk/dw/dg kernel,
// the dg kernel, the WY backward and the dh/du pass of the state recurrence:
// the Ascend GDN blog, "Ascend-affine tiling", and the G_T_CONTIG page, "fix")
// without writing their formulas.  They follow from differentiating the
// chunk form of the forward pass (per chunk, G the chunk-local cumulative
// gate, natural log, e^{dG}_{ij} = e^{G_i - G_j}, M the causal mask j <= i):
//     A = strictly_lower(beta_i e^{dG} K K^T),  T = (I + A)^{-1}
//     w = T diag(beta e^G) K,   u = T diag(beta) V
//     v_new = u - w H_c,        H_{c+1} = e^{G_last} H_c + kd^T v_new
//     o = scale [(e^G * Q) H_c + P v_new],  P = (Q K^T) * M * e^{dG}
// with kd = diag(e^{G_last - G}) K.  For L = sum <do, o> + <dht, H_final>:
//   * dv_local = scale P^T do (prep kernel);
//   * backwards over chunks, from dH = dht (state kernel):
//       dv_new = dv_local + kd dH_{c+1},
//       dH_c   = e^{G_last} dH_{c+1} + scale (e^G * Q)^T do - w^T dv_new;
//   * per chunk (dq/dk kernel), with dPm = scale (do v_new^T) * M * e^{dG}:
//       dq = scale e^G * (do H_c^T) + dPm K,
//       dk = dPm^T Q + e^{G_last - G} * (v_new dH_{c+1}^T),   dw = -dv_new H_c^T,
//       dG_i += sum_j R_ij - sum_j R_ji (R = dPm * Q K^T) + q_i . dq_inter_i
//               - x_i,  x_i = k_i . dk_kd_i,
//       dG_last += sum_i x_i + e^{G_last} <dH_{c+1}, H_c>;
//   * WY backward (wy kernel), with dT = dw (diag(beta e^G) K)^T + dv_new (diag(beta) V)^T:
//       X_w = T^T dw, X_u = T^T dv_new,  dk += beta e^G X_w,  dv = beta X_u,
//       dbeta = e^G k . X_w + v . X_u + sum_j dA_ij e^{dG} (K K^T)_ij,
//       dA = -strictly_lower(T^T dT T^T),  dS = dA * beta_i e^{dG},
//       dk += (dS + dS^T) K,  dG_i += sum_j Z_ij - sum_j Z_ji (Z = dA * A)
//              + beta_i e^{G_i} k_i . X_w_i;
//   * dg_t = sum_{i >= t in the chunk} dG_i (the chunk-local cumsum reversed),
//     then through the gate g = -exp(A_log) softplus(x), x = g_raw + dt_bias:
//       dg_raw = dg (-exp(A_log)) softplus'(x),  dA_log = sum dg g,
//       ddt_bias = sum dg_raw;
//   * dq, dk of a key head sum its value heads (a key-head sum kernel; with one
//     value head per key head the dq/dk and WY kernels write them directly).
// The forward intermediates are recomputed first by the forward kernels: WY
// (also storing T) and the state pass in its CHAIN_PLAIN mode (H_c and v_new
// row-major, in the call's dtype like T).
//
// Arithmetic.  fp32 calls run every product on the fp32 MFMA
// (v_mfma_f32_16x16x4f32, operands staged as fp32 in LDS).  bf16 calls run
// every product on the bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32
// accumulation: the forward recompute (WY, state pass), the prep kernel
// (gdn_bwd_prep_bf16_kernel: q, k, do exact, P and scale e^G do rounded to
// bf16 once), the backward state pass (operands in the call's dtype, the state
// gradient accumulating in fp32), dq/dk (gdn_bwd_dqk_bf16_kernel) and the WY
// backward (gdn_bwd_wy_bf16_kernel: k, v exact; dw, dv_new, T, dT, Y and dS
// rounded to bf16 once each).  The gate backward, the chunk-local reductions
// and the sums are fp32 VALU work.  q, k, v, do are read, and dq, dk, dv
// written, in the call's dtype.  Workspace intermediates: T, H_c, v_new, dH,
// dv_new and dw are row-major in the call's dtype (rounded once when stored;
// the bf16 MFMAs take them as stored, the dot of H_c with dH widens them to
// fp32); dq, dk partials and the per-chunk sums are fp32 row-major; the state
// pass's operands (wtf, kdf)
// and the dO term bq are fragments in the call's dtype (bq is rounded to it
// once per chunk, before the state pass adds it to the fp32 dH):
//   hcp, dhn [hv][slot][V][K]          H_c^T, (dL/dH_{c+1})^T
//   vnp, dvn [hv][slot][V][64]         v_new^T, (dL/dv_new)^T
//   tmat     [hv][slot][64][64]        T
//   dqp, dkp, dwp [hv][slot][64][K]    per value head dq (several value heads
//                                      per key head only), dk; dw
//   dgp      [hv][slot][64]            dG from the dq/dk kernel
//   dAp, dbp [hv][slot]                per-chunk sums for dA_log, ddt_bias
// and fragment-major operands of the backward state pass (k32 fragments in
// the call's dtype as in the forward state pass, lane l = row l%16, k-slot
// group l/16; D tiles fp32):
//   wtf      [hv][slot][K/16][2][lane]  A operand (rows k, k over the chunk): w^T
//   kdf      [hv][slot][4][K/32][lane]  A operand (rows c, k over K): kd
//   bq       [hv][slot][V/16][K/16][lane] D tiles (rows k, column v) in the
//                                       call's dtype: scale (e^G * Q)^T do
//   dvl      [hv][slot][V/16][4][lane]  D tiles (rows c, column v): dv_local
#pragma once
#include "gdn_kernels.h"

namespace gdn {

// fp32 LDS row stride for n columns: n + 4, so the 16 rows x 4 columns (or
// 4 rows x 16 columns) that one MFMA operand read touches fall in distinct banks.
template <int N> struct Pad { static constexpr int v = N + 4; };
constexpr int kCP = kChunk + 4;  // stride of 64-column fp32 tiles

// The per-chunk backward kernels (prep, dq/dk, WY backward) map block ids to
// (value head, chunk slot) as WY does (xcd_slot_block): a key head's value
// heads on one XCD, slot-major there, so the q / k rows they share come
// through one L2 at about the same time.
// The per-chunk backward kernels run eight waves per workgroup (two per SIMD,
// so one wave's LDS waits overlap the other's MFMAs).  A 64 x N result (N = K
// or V) is split in row halves x column quarters: wave w owns row tiles
// 2 (w/4), 2 (w/4) + 1 and columns [(w%4) N/4, (w%4+1) N/4).  A 64 x 64 result:
// wave w owns row tile w/2 and column tiles 2 (w%2), 2 (w%2) + 1.
constexpr int kBwdThreads = 512;

// acc (one 16x16 fp32 D tile) += sum_{kk < KD} A(m, kk) B(kk, n), where
// A(m, kk) = a[m * sam + kk * sak] and B(kk, n) = b[kk * sbk + n * sbn], with
// a and b at the tile's origin (m, n in 0..15).  MFMA j of each 16-wide step
// takes kk = s + 4 (lane / 16) + j in both operands.  D tile lane l holds rows
// 4 (l / 16) + r, column l % 16.
template <int KD, int MR, int NR>
__device__ __forceinline__ void mm_block(f32x4 (&acc)[MR][NR], const float* a, int sam, int sak,
                                         const float* b, int sbk, int sbn);
template <int KD>
__device__ __forceinline__ void mm16(f32x4& acc, const float* a, int sam, int sak, const float* b,
                                     int sbk, int sbn) {
  f32x4 t[1][1] = {{acc}};
  mm_block<KD, 1, 1>(t, a, sam, sak, b, sbk, sbn);
  acc = t[0][0];
}

// acc[r][c] (MR x NR D tiles) += sum_{kk < KD} A_r(m, kk) B_c(kk, n), with A_r
// the row tile r of A (origin a + 16 r sam) and B_c the column tile c of B
// (origin b + 16 c sbn); each kk's operands are loaded once for all MR x NR
// products, which also gives MR x NR independent accumulation chains.
// The operands of a 16-wide k step are loaded one step ahead (two register
// buffers), so each LDS wait covers a whole step's reads while the previous
// step's MFMAs run.
template <int KD, int MR, int NR>
__device__ __forceinline__ void mm_block(f32x4 (&acc)[MR][NR], const float* a, int sam, int sak,
                                         const float* b, int sbk, int sbn) {
  const int lane = lane_id(), l16 = lane & 15, kq = lane >> 4;
  const float* ap = a + l16 * sam + 4 * kq * sak;
  const float* bp = b + l16 * sbn + 4 * kq * sbk;
  constexpr int NS = KD / 16;
  float av[2][4][MR], bv[2][4][NR];
  auto load = [&](int buf, int s) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r = 0; r < MR; ++r) av[buf][j][r] = ap[16 * r * sam + (16 * s + j) * sak];
#pragma unroll
      for (int c = 0; c < NR; ++c) bv[buf][j][c] = bp[16 * c * sbn + (16 * s + j) * sbk];
    }
  };
  load(0, 0);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s + 1 < NS) load((s + 1) & 1, s + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int c = 0; c < NR; ++c)
          acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s & 1][j][r], bv[s & 1][j][c],
                                                           acc[r][c], 0, 0, 0);
  }
}

// The first `ncols` (0, 1 or 2; uniform per wave) of two column tiles of one
// row tile: acc[c] += A B_c.
template <int KD>
__device__ __forceinline__ void mm_pair(f32x4 (&acc)[2], int ncols, const float* a, int sam,
                                        int sak, const float* b, int sbk, int sbn) {
  if (ncols >= 2) {
    f32x4 t[1][2] = {{acc[0], acc[1]}};
    mm_block<KD, 1, 2>(t, a, sam, sak, b, sbk, sbn);
    acc[0] = t[0][0];
    acc[1] = t[0][1];
  } else if (ncols == 1) {
    mm16<KD>(acc[0], a, sam, sak, b, sbk, sbn);
  }
}

// x from another lane of the same 16-lane row, by a DPP control (a VALU
// operand modifier: no LDS round trip, unlike a shuffle).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of each lane group (the columns of a D tile row), in
// every lane of the group: quad_perm [1,0,3,2] and [2,3,0,1] sum each quad,
// row_half_mirror adds the other quad of the half row, row_mirror the other
// half row.
__device__ __forceinline__ float sum16(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}
// Sum over the 4 lane groups (the rows 4g + r of a D tile column, per r).
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}
__device__ __forceinline__ float sum64(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}
// The wave's sum, uniform: DPP row sums, then the four rows' sums read from
// lanes 0, 16, 32, 48 (no LDS permutes, no per-lane address registers).
__device__ __forceinline__ float wave_sum(float x) {
  x = sum16(x);
  const int b = __float_as_int(x);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// Rows [0, ROWS) into an fp32 LDS tile (stride ld): row r reads
// src + (t0 + r) * row_stride, rows >= len are zero.  N columns, THREADS threads.
template <int N, typename E, int ROWS = kChunk, int THREADS = 256>
__device__ __forceinline__ void stage_rows(float* dst, int ld, const E* src, int64_t t0,
                                           int64_t row_stride, int len) {
  constexpr int PER = ROWS * N / 8 / THREADS;  // 8-element pieces per thread
  static_assert(PER * 8 * THREADS == ROWS * N, "whole pieces per thread");
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int m = tid + THREADS * it, row = m / (N / 8), c0 = 8 * (m % (N / 8));
    float e[8];
    if (row < len) {
      ld8(src + (t0 + row) * row_stride + c0, e);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = 0.f;
    }
    *reinterpret_cast<f32x4*>(dst + row * ld + c0) = f32x4{e[0], e[1], e[2], e[3]};
    *reinterpret_cast<f32x4*>(dst + row * ld + c0 + 4) = f32x4{e[4], e[5], e[6], e[7]};
  }
}

// The 8 elements of a k32 fragment in k-slot order (kslot(g, i), i = 0..7).
__device__ __forceinline__ void frag_elems(const Frag<bf16>& f, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)f.x[i];
}
__device__ __forceinline__ void frag_elems(const Frag<float>& f, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = f.lo[i];
    x[4 + i] = f.hi[i];
  }
}

// ---------------------------------------------------------------------------
// Prep, one workgroup per (chunk slot, value head): dv_local, the state pass's
// dH term bq = scale (e^G * Q)^T do, and its kd and w^T operand fragments
// (dtype E, as the forward state pass's operands).
template <typename E, int K, int V, bool VARLEN>
__global__ __launch_bounds__(kBwdThreads) void gdn_bwd_prep_kernel(
    Geo geo, const E* __restrict__ qg, const E* __restrict__ kg, const E* __restrict__ dog,
    const int4* __restrict__ cmap, const float* __restrict__ gam, const Frag<E>* __restrict__ wf,
    Frag<E>* __restrict__ wtf, Frag<E>* __restrict__ kdf, Quad<E>* __restrict__ bq,
    f32x4* __restrict__ dvl) {
  constexpr int KP = Pad<K>::v, VP = Pad<V>::v, KT = K / 16, KB = K / 32, NV = V / 16;
  constexpr int TH = kBwdThreads, NW = TH / 64;
  __shared__ __align__(16) float Qs[kChunk * KP];  // q, later w
  __shared__ __align__(16) float Ks[kChunk * KP];
  __shared__ __align__(16) float Ds[kChunk * VP];  // do, later scale e^G do
  __shared__ __align__(16) float Ps[kChunk * kCP];
  __shared__ float sg[kChunk];

  int hv, slot;
  xcd_slot_block(blockIdx.x, geo.H, geo.G, geo.slots, hv, slot);
  int n, len;
  int64_t t0;
  if (!chunk_of_slot<VARLEN>(geo, cmap, slot, n, t0, len)) return;
  const int h = hv / geo.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, lc = lane & 15;
  const size_t hs = (size_t)hv * geo.slots + slot;
  const int pit = wave >> 1, pj0 = 2 * (wave & 1);

  stage_rows<K, E, kChunk, TH>(Qs, KP, qg + (size_t)h * K, t0, (int64_t)geo.H * K, len);
  stage_rows<K, E, kChunk, TH>(Ks, KP, kg + (size_t)h * K, t0, (int64_t)geo.H * K, len);
  stage_rows<V, E, kChunk, TH>(Ds, VP, dog + (size_t)hv * V, t0, (int64_t)geo.HV * V, len);
  if (tid < kChunk) sg[tid] = gam[hs * kChunk + tid];
  __syncthreads();

  // P = (Q K^T) * M * e^{dG}
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int jt = pj0 + b;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (jt <= pit) mm16<K>(acc, Qs + 16 * pit * KP, KP, 1, Ks + 16 * jt * KP, 1, KP);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * pit + 4 * g + r, j = 16 * jt + lc;
      Ps[i * kCP + j] = j <= i ? acc[r] * fast_exp2(sg[i] - sg[j]) : 0.f;
    }
  }
  __syncthreads();

  // dv_local = scale P^T do: D tiles (rows c = 16 ct + .., column v).
  for (int f = wave; f < 4 * NV; f += NW) {
    const int ct = f / NV, vt = f - ct * NV;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    mm16<kChunk>(acc, Ps + 16 * ct, 1, kCP, Ds + 16 * vt, VP, 1);
    dvl[((hs * NV + vt) * 4 + ct) * 64 + lane] = acc * geo.scale;
  }
  // kd fragments (rows c, k over K).
  {
    const float gl = sg[kChunk - 1];
    for (int f = wave; f < 4 * KB; f += NW) {
      const int ct = f / KB, kb = f - ct * KB, c = 16 * ct + lc;
      const float e = fast_exp2(gl - sg[c]);
      const f32x4 lo = *reinterpret_cast<const f32x4*>(Ks + c * KP + 32 * kb + 4 * g);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(Ks + c * KP + 32 * kb + 16 + 4 * g);
      kdf[((hs * 4 + ct) * KB + kb) * 64 + lane] = frag_from_tiles<E>(lo * e, hi * e);
    }
  }
  __syncthreads();
  // do rows times scale e^{G_c}, then bq = Q^T (scale e^G do): D tiles
  // (rows k, column v).
  for (int e = tid; e < kChunk * (V / 4); e += TH) {
    const int c = e / (V / 4), v4 = 4 * (e - c * (V / 4));
    *reinterpret_cast<f32x4*>(Ds + c * VP + v4) *= geo.scale * fast_exp2(sg[c]);
  }
  __syncthreads();
  for (int f = wave; f < KT * NV; f += NW) {
    const int mt = f / NV, vt = f - mt * NV;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    mm16<kChunk>(acc, Qs + 16 * mt, 1, KP, Ds + 16 * vt, VP, 1);
    bq[((hs * NV + vt) * KT + mt) * 64 + lane] = make_quad<E>(acc);
  }
  __syncthreads();
  // w from its forward fragments (rows c = 16 ct + lane%16, k = 32 kb + kslot)
  // into Qs, then w^T fragments (rows k, k over the chunk).
  for (int f = wave; f < 4 * KB; f += NW) {
    const int ct = f / KB, kb = f - ct * KB, c = 16 * ct + lc;
    float x[8];
    frag_elems(wf[((hs * 4 + ct) * KB + kb) * 64 + lane], x);
    *reinterpret_cast<f32x4*>(Qs + c * KP + 32 * kb + 4 * g) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(Qs + c * KP + 32 * kb + 16 + 4 * g) = f32x4{x[4], x[5], x[6], x[7]};
  }
  __syncthreads();
  for (int f = wave; f < KT * 2; f += NW) {
    const int mt = f >> 1, cb = f & 1, kk = 16 * mt + lc;
    f32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = Qs[(32 * cb + 4 * g + i) * KP + kk];
      hi[i] = Qs[(32 * cb + 16 + 4 * g + i) * KP + kk];
    }
    wtf[(hs * KT * 2 + f) * 64 + lane] = frag_from_tiles<E>(lo, hi);
  }
}

// ---------------------------------------------------------------------------
// Backward state pass: one wave per (sequence, value head, 16 value columns),
// chunks in reverse order; dL/dH (K x 16, fp32) lives in registers as K/16 D
// tiles (rows k, column v).  Per chunk: store dH (= dL/dH_{c+1}), then
//   dv_new = dv_local + kd dH,   dH <- e^{G_last} dH + bq - w^T dv_new,
// with kd, w^T and dH, dv_new as MFMA operands in the dtype E (as in the
// forward state pass).  After the first chunk dH is dL/dh0.  The operands are
// loaded in two halves, each right after its previous use, so that a half's
// loads overlap the other half's products: (kd, dv_local) for v_new's product,
// (w^T, bq, e^{G_last}) for the update.
template <typename E, int K, int V, bool VARLEN>
__global__ __launch_bounds__(64) void gdn_bwd_chain_kernel(
    Geo geo, const Frag<E>* __restrict__ kdf, const f32x4* __restrict__ dvl,
    const Frag<E>* __restrict__ wtf, const Quad<E>* __restrict__ bq, const float* __restrict__ gam,
    const int* __restrict__ seq_slot, const float* __restrict__ dht, float* __restrict__ dh0,
    E* __restrict__ dhn, E* __restrict__ dvn) {
  constexpr int NV = V / 16, KT = K / 16, KB = K / 32;
  int hv, rest;
  head_major_block(blockIdx.x, geo.HV, geo.N * NV, hv, rest);
  const int n = rest / NV, vt = rest - n * NV;
  int s0, s1;
  if constexpr (VARLEN) {
    s0 = seq_slot[n];
    s1 = seq_slot[n + 1];
  } else {
    s0 = n * geo.NT;
    s1 = s0 + geo.NT;
  }
  const int lane = lane_id(), g = lane >> 4, lc = lane & 15, v = 16 * vt + lc;
  const size_t sbase = ((size_t)n * geo.HV + hv) * K * V;
  const size_t hbase = (size_t)hv * geo.slots;

  f32x4 dH[KT];
  load_state<K, V>(dH, dht, sbase, v, g);
  Frag<E> kd[4][KB], wt[KT][2];
  f32x4 dl[4], b[KT];
  float gl = 0.f;
  auto load_a = [&](size_t hs) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      dl[ct] = dvl[((hs * NV + vt) * 4 + ct) * 64 + lane];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kd[ct][kb] = kdf[((hs * 4 + ct) * KB + kb) * 64 + lane];
    }
  };
  auto load_b = [&](size_t hs) {
    gl = gam[hs * kChunk + lane];  // lane 63 holds the chunk's last cumulative gate
#pragma unroll
    for (int mt = 0; mt < KT; ++mt) {
      b[mt] = quad_f32(bq[((hs * NV + vt) * KT + mt) * 64 + lane]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) wt[mt][cb] = wtf[((hs * KT + mt) * 2 + cb) * 64 + lane];
    }
  };
  if (s1 > s0) {
    load_a(hbase + s1 - 1);
    load_b(hbase + s1 - 1);
  }
  for (int s = s1 - 1; s >= s0; --s) {
    const size_t hs = hbase + s, nxt = hbase + (s > s0 ? s - 1 : s0);  // in bounds
    // transposed: lane (v, g) holds rows 4g..4g+3 of each tile, contiguous in dH^T
    Quad<E>* hp = reinterpret_cast<Quad<E>*>(dhn + hs * K * V + (size_t)v * K + 4 * g);
#pragma unroll
    for (int mt = 0; mt < KT; ++mt) hp[4 * mt] = make_quad<E>(dH[mt]);
    Frag<E> hb[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) hb[kb] = frag_from_tiles<E>(dH[2 * kb], dH[2 * kb + 1]);
    f32x4 dv[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      dv[ct] = dl[ct];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) mma_k32(dv[ct], kd[ct][kb], hb[kb]);
    }
    asm volatile("" ::: "memory");
    load_a(nxt);
    asm volatile("" ::: "memory");
    Quad<E>* vp = reinterpret_cast<Quad<E>*>(dvn + hs * kChunk * V + (size_t)v * kChunk + 4 * g);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) vp[4 * ct] = make_quad<E>(dv[ct]);
    const Frag<E> nb[2] = {frag_from_tiles<E>(-dv[0], -dv[1]), frag_from_tiles<E>(-dv[2], -dv[3])};
    const float dec = fast_exp2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), kChunk - 1)));
#pragma unroll
    for (int mt = 0; mt < KT; ++mt) {
      dH[mt] = dH[mt] * dec + b[mt];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) mma_k32(dH[mt], wt[mt][cb], nb[cb]);
    }
    asm volatile("" ::: "memory");
    load_b(nxt);
    asm volatile("" ::: "memory");
  }
  if (dh0) {
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dh0[sbase + (size_t)(16 * mt + 4 * g + r) * V + v] = dH[mt][r];
  }
}

// ---------------------------------------------------------------------------
// Backward state pass with the K rows split over K/32 waves: one workgroup per
// (sequence, value head, 16 value columns); wave q holds rows 32q..32q+31 of
// dL/dH and reads only those rows' kd and w^T fragments and bq tiles (a
// quarter of the one-wave variant's operand stream at K = 128).  Per chunk,
// in reverse order:
//   store the wave's rows of dH;
//   partial products kd[:, rows of q] dH[rows of q], four 16-row tiles;
//   reduce-scatter through LDS: the owner of chunk-row tile ct (ct mod KB = q)
//   forms dv_new tile ct = dv_local + (P_0 + P_1 + ...), summed in wave order,
//   stores it and exchanges -dv_new rounded to the dtype;
//   dH[rows of q] <- e^{G_last} dH[rows of q] + bq[rows of q] - w^T[rows of q] dv_new.
// Two workgroup barriers per chunk; operands loaded two chunks ahead.
template <typename E, int K, int V>
struct BwdKsStep {
  static constexpr int KB = K / 32, KT = K / 16, NV = V / 16, OWN = 4 / KB;
  Frag<E> kd[4];      // kd, chunk-row tile ct, k block q
  Frag<E> wt[2][2];   // w^T, row tile 2q + j, chunk block cb
  f32x4 dl[OWN];      // dv_local, chunk-row tiles q + KB j
  Quad<E> b[2];       // bq, row tiles 2q + j
  float gl;           // lane l: entry l of the chunk's gate row

  template <int Q>
  __device__ __forceinline__ void load(const Frag<E>* __restrict__ kdf, const f32x4* __restrict__ dvl,
                                       const Frag<E>* __restrict__ wtf, const Quad<E>* __restrict__ bq,
                                       const float* __restrict__ gam, size_t hs, int vt, int lane) {
    gl = gam[hs * kChunk + lane];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) kd[ct] = kdf[((hs * 4 + ct) * KB + Q) * 64 + lane];
#pragma unroll
    for (int j = 0; j < OWN; ++j) dl[j] = dvl[((hs * NV + vt) * 4 + Q + KB * j) * 64 + lane];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      b[j] = bq[((hs * NV + vt) * KT + 2 * Q + j) * 64 + lane];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) wt[j][cb] = wtf[((hs * KT + 2 * Q + j) * 2 + cb) * 64 + lane];
    }
  }
};

template <typename E, int K, int V, int D, int Q>
__device__ __forceinline__ void bwd_chain_ks_wave(ChainKsLds<E, K, V>& sh, const Frag<E>* __restrict__ kdf,
                                                  const f32x4* __restrict__ dvl,
                                                  const Frag<E>* __restrict__ wtf,
                                                  const Quad<E>* __restrict__ bq, const float* __restrict__ gam,
                                                  const float* __restrict__ dht, float* __restrict__ dh0,
                                                  E* __restrict__ dhn, E* __restrict__ dvn, int s0,
                                                  int s1, size_t hbase, size_t sbase, int vt) {
  using Step = BwdKsStep<E, K, V>;
  constexpr int KB = Step::KB, OWN = Step::OWN;
  const int lane = lane_id(), g = lane >> 4, v = 16 * vt + (lane & 15);
  f32x4 dH[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dH[j][r] = dht ? dht[sbase + (size_t)(32 * Q + 16 * j + 4 * g + r) * V + v] : 0.f;

  auto chunk = [&](const Step& S, size_t hs) {
    // transposed: lane (v, g) holds rows 4g..4g+3 of each tile, contiguous in dH^T
    Quad<E>* hp = reinterpret_cast<Quad<E>*>(dhn + hs * K * V + (size_t)v * K + 4 * g);
    hp[4 * (2 * Q)] = make_quad<E>(dH[0]);
    hp[4 * (2 * Q + 1)] = make_quad<E>(dH[1]);
    const Frag<E> hb = frag_from_tiles<E>(dH[0], dH[1]);
    f32x4 p[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      p[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      mma_k32(p[ct], S.kd[ct], hb);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      if (ct % KB != Q) sh.part[Q][ct][lane] = p[ct];
    wait_lgkm0();
    ring_barrier();
    Quad<E> own[OWN];
    Quad<E>* vp = reinterpret_cast<Quad<E>*>(dvn + hs * kChunk * V + (size_t)v * kChunk + 4 * g);
#pragma unroll
    for (int j = 0; j < OWN; ++j) {
      const int ct = Q + KB * j;
      f32x4 acc = Q == 0 ? p[ct] : sh.part[0][ct][lane];
#pragma unroll
      for (int w2 = 1; w2 < KB; ++w2) acc += (w2 == Q ? p[ct] : sh.part[w2][ct][lane]);
      const f32x4 dv = S.dl[j] + acc;
      vp[4 * ct] = make_quad<E>(dv);
      own[j] = make_quad<E>(-dv);
      sh.vx[ct][lane] = own[j];
    }
    wait_lgkm0();
    ring_barrier();
    Quad<E> vq[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) vq[ct] = (ct % KB == Q) ? own[ct / KB] : sh.vx[ct][lane];
    Frag<E> nb[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) nb[cb] = frag_join(vq[2 * cb], vq[2 * cb + 1]);
    const float dec = fast_exp2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(S.gl), kChunk - 1)));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dH[j] = dH[j] * dec + quad_f32(S.b[j]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) mma_k32(dH[j], S.wt[j][cb], nb[cb]);
    }
  };

  if (s0 < s1) {
    // chunks s1-1 down to s0; loads clamped to s0 (in bounds), the exit
    // jumps past the loop
    Step buf[D];
#pragma unroll
    for (int j = 0; j < D; ++j) buf[j].template load<Q>(kdf, dvl, wtf, bq, gam, hbase + max(s1 - 1 - j, s0), vt, lane);
    for (int s = s1 - 1;; s -= D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (s - j < s0) goto done;
        chunk(buf[j], hbase + s - j);
        buf[j].template load<Q>(kdf, dvl, wtf, bq, gam, hbase + max(s - j - D, s0), vt, lane);
        asm volatile("" ::: "memory");
      }
    }
  }
done:
  if (dh0) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) dh0[sbase + (size_t)(32 * Q + 16 * j + 4 * g + r) * V + v] = dH[j][r];
  }
}

template <typename E, int K, int V, bool VARLEN, int D>
__global__ __launch_bounds__(64 * (K / 32)) void gdn_bwd_chain_ks_kernel(
    Geo geo, const Frag<E>* __restrict__ kdf, const f32x4* __restrict__ dvl,
    const Frag<E>* __restrict__ wtf, const Quad<E>* __restrict__ bq, const float* __restrict__ gam,
    const int* __restrict__ seq_slot, const int* __restrict__ seq_order,
    const float* __restrict__ dht, float* __restrict__ dh0, E* __restrict__ dhn,
    E* __restrict__ dvn) {
  static_assert(K == 64 || K == 128, "two or four waves");
  constexpr int NV = V / 16;
  __shared__ ChainKsLds<E, K, V> sh;
  // packed sequences longest first (seq_order), for launches whose
  // workgroups run in several rounds
  int hv, n, vt;
  if (VARLEN && seq_order != nullptr) {
    int r;
    rank_major_block(blockIdx.x, geo.HV, NV, hv, r, vt);
    n = seq_order[r];
  } else {
    int rest;
    head_major_block(blockIdx.x, geo.HV, geo.N * NV, hv, rest);
    n = rest / NV;
    vt = rest - n * NV;
  }
  int s0, s1;
  if constexpr (VARLEN) {
    s0 = seq_slot[n];
    s1 = seq_slot[n + 1];
  } else {
    s0 = n * geo.NT;
    s1 = s0 + geo.NT;
  }
  const size_t sbase = ((size_t)n * geo.HV + hv) * K * V;
  const size_t hbase = (size_t)hv * geo.slots;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave == 0)
    bwd_chain_ks_wave<E, K, V, D, 0>(sh, kdf, dvl, wtf, bq, gam, dht, dh0, dhn, dvn, s0, s1, hbase, sbase, vt);
  else if (wave == 1)
    bwd_chain_ks_wave<E, K, V, D, 1>(sh, kdf, dvl, wtf, bq, gam, dht, dh0, dhn, dvn, s0, s1, hbase, sbase, vt);
  if constexpr (K == 128) {
    if (wave == 2)
      bwd_chain_ks_wave<E, K, V, D, 2>(sh, kdf, dvl, wtf, bq, gam, dht, dh0, dhn, dvn, s0, s1, hbase, sbase, vt);
    else if (wave == 3)
      bwd_chain_ks_wave<E, K, V, D, 3>(sh, kdf, dvl, wtf, bq, gam, dht, dh0, dhn, dvn, s0, s1, hbase, sbase, vt);
  }
}

// dq / dk / dw / dG, one workgroup per (chunk slot, value head); with one value
// head per key head dq is written final, else per value head.  The products
// over V run in two LDS stagings: (do, dv_new, H_c) for dq_inter and dw, then
// (do, v_new, dH_{c+1}) for dPm and dk_kd; the products over K and over the
// chunk then stage q and k.
template <typename E, int K, int V, bool VARLEN>
__global__ __launch_bounds__(kBwdThreads) void gdn_bwd_dqk_kernel(
    Geo geo, const E* __restrict__ qg, const E* __restrict__ kg, const E* __restrict__ dog,
    const int4* __restrict__ cmap, const float* __restrict__ gam, const float* __restrict__ vnp,
    const float* __restrict__ dvn, const float* __restrict__ hcp, const float* __restrict__ dhn,
    float* __restrict__ dqp, float* __restrict__ dkp, float* __restrict__ dwp,
    float* __restrict__ dgp, E* __restrict__ dqg) {
  constexpr int KP = Pad<K>::v, VP = Pad<V>::v, NKT = K / 64, TH = kBwdThreads;
  constexpr int PH1 = kChunk * VP + V * kCP + V * KP, PH2 = 2 * kChunk * KP + kChunk * kCP;
  __shared__ __align__(16) float lds[PH1 > PH2 ? PH1 : PH2];
  __shared__ float sg[kChunk], dG[kChunk], red[2];
  float* const Ds = lds;                                // do            [64][V]
  float* const Xs = lds + kChunk * VP;                  // dv_new^T, then v_new^T  [V][64]
  float* const Hs = lds + kChunk * VP + V * kCP;        // H_c^T, then dH_{c+1}^T  [V][K]
  float* const Qs = lds;
  float* const Ks = lds + kChunk * KP;
  float* const Pd = lds + 2 * kChunk * KP;

  int hv, slot;
  xcd_slot_block(blockIdx.x, geo.H, geo.G, geo.slots, hv, slot);
  int n, len;
  int64_t t0;
  if (!chunk_of_slot<VARLEN>(geo, cmap, slot, n, t0, len)) return;
  const int h = hv / geo.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, lc = lane & 15;
  const size_t hs = (size_t)hv * geo.slots + slot;
  const int rt0 = 2 * (wave >> 2), kc0 = (wave & 3) * (K / 4);  // 64 x K ownership
  const int pit = wave >> 1, pj0 = 2 * (wave & 1);               // 64 x 64 ownership
  const float* Hc = hcp + hs * K * V;
  const float* dHn = dhn + hs * K * V;

  stage_rows<V, E, kChunk, TH>(Ds, VP, dog + (size_t)hv * V, t0, (int64_t)geo.HV * V, len);
  stage_rows<kChunk, float, V, TH>(Xs, kCP, dvn + hs * kChunk * V, 0, kChunk, V);
  stage_rows<K, float, V, TH>(Hs, KP, Hc, 0, K, V);
  if (tid < kChunk) {
    sg[tid] = gam[hs * kChunk + tid];
    dG[tid] = 0.f;
  }
  if (tid < 2) red[tid] = 0.f;
  __syncthreads();
  const float gl = sg[kChunk - 1];

  // dq_inter = scale e^G (do H_c^T) and dw = -dv_new H_c^T (B operand: H_c^T,
  // rows v).
  // (ncols of a 64 x 64 row tile's column pair below or on the diagonal)
  const int npair = pit >= pj0 + 1 ? 2 : pit >= pj0 ? 1 : 0;
  f32x4 dq[2][NKT], dk[2][NKT];
  {
    f32x4 dw[2][NKT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) dq[a][nt] = dw[a][nt] = dk[a][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    mm_block<V, 2, NKT>(dq, Ds + 16 * rt0 * VP, VP, 1, Hs + kc0, KP, 1);
    mm_block<V, 2, NKT>(dw, Xs + 16 * rt0, 1, kCP, Hs + kc0, KP, 1);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * (rt0 + a) + 4 * g + r;
          dq[a][nt][r] *= geo.scale * fast_exp2(sg[i]);
          dwp[(hs * kChunk + i) * K + kc0 + 16 * nt + lc] = -dw[a][nt][r];
        }
  }
  __syncthreads();
  stage_rows<kChunk, float, V, TH>(Xs, kCP, vnp + hs * kChunk * V, 0, kChunk, V);
  // dH_{c+1} replaces H_c in LDS; each thread first reads the H_c values at the
  // positions it overwrites, for <dH_{c+1}, H_c>.
  {
    constexpr int PER = K * V / 8 / TH;
    float acc = 0.f;
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int m = tid + TH * it, row = m / (K / 8), c0 = 8 * (m % (K / 8));
      float e[8];
      ld8(dHn + (size_t)row * K + c0, e);
      float* dst = Hs + row * KP + c0;
      const f32x4 h0 = *reinterpret_cast<const f32x4*>(dst);
      const f32x4 h1 = *reinterpret_cast<const f32x4*>(dst + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += h0[j] * e[j] + h1[j] * e[4 + j];
      *reinterpret_cast<f32x4*>(dst) = f32x4{e[0], e[1], e[2], e[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{e[4], e[5], e[6], e[7]};
    }
    acc = sum64(acc);
    if (lane == 0) atomicAdd(&red[0], acc);
  }
  __syncthreads();
  // dPm = scale (do v_new^T) * M * e^{dG}
  f32x4 dPm[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  mm_pair<V>(dPm, npair, Ds + 16 * pit * VP, VP, 1, Xs + 16 * pj0, kCP, 1);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int jt = pj0 + b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * pit + 4 * g + r, j = 16 * jt + lc;
      dPm[b][r] = j <= i ? dPm[b][r] * geo.scale * fast_exp2(sg[i] - sg[j]) : 0.f;
    }
  }
  // dk_kd = e^{G_last - G} (v_new dH_{c+1}^T)
  mm_block<V, 2, NKT>(dk, Xs + 16 * rt0, 1, kCP, Hs + kc0, KP, 1);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dk[a][nt][r] *= fast_exp2(gl - sg[16 * (rt0 + a) + 4 * g + r]);
  __syncthreads();

  stage_rows<K, E, kChunk, TH>(Qs, KP, qg + (size_t)h * K, t0, (int64_t)geo.H * K, len);
  stage_rows<K, E, kChunk, TH>(Ks, KP, kg + (size_t)h * K, t0, (int64_t)geo.H * K, len);
  __syncthreads();
  // R = dPm * (Q K^T): dG_i += row sums, dG_j -= column sums; dPm to LDS.
  f32x4 sq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  mm_pair<K>(sq, npair, Qs + 16 * pit * KP, KP, 1, Ks + 16 * pj0 * KP, 1, KP);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int jt = pj0 + b;
    float cs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rr = dPm[b][r] * sq[b][r];
      cs += rr;
      const float rs = sum16(rr);
      if (lc == 0) atomicAdd(&dG[16 * pit + 4 * g + r], rs);
      Pd[(16 * pit + 4 * g + r) * kCP + 16 * jt + lc] = dPm[b][r];
    }
    cs = sum_groups(cs);
    if (g == 0) atomicAdd(&dG[16 * jt + lc], -cs);
  }
  // dG_i += q_i . dq_inter_i;  x_j = k_j . dk_kd_j: dG_j -= x_j, sum x -> red[1].
  {
    float xs = 0.f;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * (rt0 + a) + 4 * g + r;
        float qd = 0.f, kx = 0.f;
#pragma unroll
        for (int nt = 0; nt < NKT; ++nt) {
          const int kk = kc0 + 16 * nt + lc;
          qd += Qs[i * KP + kk] * dq[a][nt][r];
          kx += Ks[i * KP + kk] * dk[a][nt][r];
        }
        qd = sum16(qd);
        kx = sum16(kx);
        if (lc == 0) atomicAdd(&dG[i], qd - kx);
        xs += lc == 0 ? kx : 0.f;
      }
    xs = sum64(xs);
    if (lane == 0) atomicAdd(&red[1], xs);
  }
  __syncthreads();
  // dq += dPm K;  dk += dPm^T Q.
  mm_block<kChunk, 2, NKT>(dq, Pd + 16 * rt0 * kCP, kCP, 1, Ks + kc0, KP, 1);
  mm_block<kChunk, 2, NKT>(dk, Pd + 16 * rt0, 1, kCP, Qs + kc0, KP, 1);
#pragma unroll
  for (int nt = 0; nt < NKT; ++nt) {
    const int kc = kc0 + 16 * nt;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int it = rt0 + a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * g + r;
        const size_t o = (hs * kChunk + i) * K + kc + lc;
        // one value head per key head: dq is final here
        if (geo.G == 1) {
          if (i < len) dqg[((t0 + i) * geo.H + h) * K + kc + lc] = (E)dq[a][nt][r];
        } else {
          dqp[o] = dq[a][nt][r];
        }
        dkp[o] = dk[a][nt][r];
      }
    }
  }
  if (tid < kChunk) {
    float x = dG[tid];
    if (tid == kChunk - 1) x += red[1] + fast_exp2(gl) * red[0];
    dgp[hs * kChunk + tid] = x;
  }
}

// ---------------------------------------------------------------------------
// The dq / dk / dw / dG kernel for bf16 calls: the same products on the bf16
// MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation), with every operand
// staged in LDS as bf16.  q, k and do are bf16 already; H_c, dH_{c+1}, v_new,
// dv_new and dPm are rounded to bf16 once, when staged (the forward output
// kernel takes H_c and v_new the same way); <dH_{c+1}, H_c> is summed from the
// fp32 values.  A k32 operand needs its 32 reduction indices contiguous in a
// tile row, so tiles whose reduction index is a column of the stored layout
// are written transposed (4 x 4 or 4 x 8 blocks per thread, one 8-byte LDS
// store per transposed row piece, column groups swizzled by tswz) and read
// with frag_from_trow; the others are copied row by row and read with
// frag_from_row.  LDS is ~72 KB (two workgroups per CU).

// bf16 LDS row stride for N columns: N + 8 elements (a multiple of 16 bytes).
template <int N> struct PadB { static constexpr int v = N + 8; };

// Rows [0, kChunk) of a bf16 source into a bf16 LDS tile (stride ld), rows
// >= len zero; 16 bytes per thread per piece.
template <int N, int THREADS>
__device__ __forceinline__ void stage_rows_b(bf16* dst, int ld, const bf16* src, int64_t t0,
                                             int64_t row_stride, int len) {
  constexpr int PER = kChunk * N / 8 / THREADS;
  static_assert(PER * 8 * THREADS == kChunk * N, "whole pieces per thread");
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int m = tid + THREADS * it, row = m / (N / 8), c0 = 8 * (m % (N / 8));
    bf16x8 x = {};
    if (row < len) x = *reinterpret_cast<const bf16x8*>(src + (t0 + row) * row_stride + c0);
    *reinterpret_cast<bf16x8*>(dst + row * ld + c0) = x;
  }
}

// dst[c][r] = src[r][c] for r < SR, c < SC: fp32 source (row stride SC) into
// a transposed bf16 LDS tile (row stride DS, column groups swizzled by
// tswz(c)).  One 4 x 4 block per thread and step.
template <int SR, int SC, int DS, int THREADS>
__device__ __forceinline__ void stage_t(bf16* dst, const float* src) {
  constexpr int BC = SC / 4, NB = (SR / 4) * BC, PER = (NB + THREADS - 1) / THREADS;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int b = threadIdx.x + THREADS * it;
    if (NB % THREADS == 0 || b < NB) {
      const int r0 = 4 * (b / BC), c0 = 4 * (b % BC);
      f32x4 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = *reinterpret_cast<const f32x4*>(src + (size_t)(r0 + j) * SC + c0);
#pragma unroll
      for (int j = 0; j < 4; ++j) st4(dst + (c0 + j) * DS + (r0 ^ tswz(c0 + j)), x[0][j], x[1][j], x[2][j], x[3][j]);
    }
  }
}

// The same from a bf16 source.
template <int SR, int SC, int DS, int THREADS>
__device__ __forceinline__ void stage_t(bf16* dst, const bf16* src) {
  constexpr int BC = SC / 4, NB = (SR / 4) * BC, PER = (NB + THREADS - 1) / THREADS;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int b = threadIdx.x + THREADS * it;
    if (NB % THREADS == 0 || b < NB) {
      const int r0 = 4 * (b / BC), c0 = 4 * (b % BC);
      bf16x4 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = *reinterpret_cast<const bf16x4*>(src + (size_t)(r0 + j) * SC + c0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<bf16x4*>(dst + (c0 + j) * DS + (r0 ^ tswz(c0 + j))) =
            bf16x4{x[0][j], x[1][j], x[2][j], x[3][j]};
    }
  }
}

// ---------------------------------------------------------------------------
// The prep kernel for bf16 calls: the products of gdn_bwd_prep_kernel on the
// bf16 MFMA (fp32 accumulation).  q, k and do are staged exactly; P (for
// dv_local) and scale e^G do (for the dH term) are rounded to bf16 once.
// LDS (~73 KB at K = V = 128: two workgroups per CU), phase by phase:
//   A: q, k natural rows            -> P (registers), kd fragments
//   B: P^T (t-w) over k's rows; do^T and (scale e^G do)^T (t-w) -> dv_local
//   C: q^T (t-w) over P^T           -> bq = q^T (scale e^G do)
//   D: w natural over q             -> w^T fragments
template <int K, int V, bool VARLEN>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(4))) void gdn_bwd_prep_bf16_kernel(
    Geo geo, const bf16* __restrict__ qg, const bf16* __restrict__ kg, const bf16* __restrict__ dog,
    const int4* __restrict__ cmap, const float* __restrict__ gam, const Frag<bf16>* __restrict__ wf,
    Frag<bf16>* __restrict__ wtf, Frag<bf16>* __restrict__ kdf, Quad<bf16>* __restrict__ bq,
    f32x4* __restrict__ dvl) {
  constexpr int SK = PadB<K>::v, SC = PadB<kChunk>::v;
  constexpr int KT = K / 16, KB = K / 32, NV = V / 16, TH = kBwdThreads, NW = TH / 64;
  constexpr int RX = kChunk * SK;                                  // q, then w
  constexpr int RY = kChunk * SK > K * SC ? kChunk * SK : K * SC;  // k, then P^T, then q^T
  constexpr int RZ = 2 * V * SC;                                   // do^T, (s do)^T
  __shared__ __align__(16) bf16 lds[RX + RY + RZ];
  __shared__ float sg[kChunk];
  bf16* const Qn = lds;
  bf16* const Wn = lds;
  bf16* const Kn = lds + RX;
  bf16* const Pt = lds + RX;
  bf16* const Qt = lds + RX;
  bf16* const Dt = lds + RX + RY;
  bf16* const Dst = Dt + V * SC;

  int hv, slot;
  xcd_slot_block(blockIdx.x, geo.H, geo.G, geo.slots, hv, slot);
  int n, len;
  int64_t t0;
  if (!chunk_of_slot<VARLEN>(geo, cmap, slot, n, t0, len)) return;
  const int h = hv / geo.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, lc = lane & 15;
  const size_t hs = (size_t)hv * geo.slots + slot;
  const int pit = wave >> 1, pj0 = 2 * (wave & 1);

  // do rows: 4 rows x 8 columns per thread, loaded now, staged in B
  constexpr int DCB = V / 8, DNB = (kChunk / 4) * DCB, DPER = (DNB + TH - 1) / TH;
  bf16x8 dx[DPER][4];
#pragma unroll
  for (int it = 0; it < DPER; ++it) {
    const int b = tid + TH * it;
    if (DNB % TH == 0 || b < DNB) {
      const int r0 = 4 * (b / DCB), c0 = 8 * (b % DCB);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dx[it][j] = bf16x8{};
        if (r0 + j < len) dx[it][j] = *reinterpret_cast<const bf16x8*>(dog + ((t0 + r0 + j) * geo.HV + hv) * V + c0);
      }
    }
  }
  stage_rows_b<K, TH>(Qn, SK, qg + (size_t)h * K, t0, (int64_t)geo.H * K, len);
  stage_rows_b<K, TH>(Kn, SK, kg + (size_t)h * K, t0, (int64_t)geo.H * K, len);
  if (tid < kChunk) sg[tid] = gam[hs * kChunk + tid];
  __syncthreads();

  // A. P = (Q K^T) * M * e^{dG} (registers), and the kd fragments.
  f32x4 pm[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int jt = pj0 + b;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (jt <= pit) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        mma_k32(acc, frag_from_row(Qn + (16 * pit + lc) * SK + 32 * kb),
                frag_from_row(Kn + (16 * jt + lc) * SK + 32 * kb));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * pit + 4 * g + r, j = 16 * jt + lc;
      pm[b][r] = j <= i ? acc[r] * fast_exp2(sg[i] - sg[j]) : 0.f;
    }
  }
  {
    const float gl = sg[kChunk - 1];
    for (int f = wave; f < 4 * KB; f += NW) {
      const int ct = f / KB, kb = f - ct * KB, c = 16 * ct + lc;
      const float e = fast_exp2(gl - sg[c]);
      const f32x4 lo = to_f32x4(*reinterpret_cast<const bf16x4*>(Kn + c * SK + 32 * kb + 4 * g));
      const f32x4 hi = to_f32x4(*reinterpret_cast<const bf16x4*>(Kn + c * SK + 32 * kb + 16 + 4 * g));
      kdf[((hs * 4 + ct) * KB + kb) * 64 + lane] = frag_from_tiles<bf16>(lo * e, hi * e);
    }
  }
  __syncthreads();
  // B. P^T, do^T and (scale e^G do)^T; dv_local = scale P^T do.
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int j = 16 * (pj0 + b) + lc;
    *reinterpret_cast<bf16x4*>(Pt + j * SC + ((16 * pit + 4 * g) ^ tswz(j))) = to_bf16x4(pm[b]);
  }
#pragma unroll
  for (int it = 0; it < DPER; ++it) {
    const int b = tid + TH * it;
    if (DNB % TH == 0 || b < DNB) {
      const int r0 = 4 * (b / DCB), c0 = 8 * (b % DCB);
      float sc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[j] = geo.scale * fast_exp2(sg[r0 + j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = c0 + e, col = r0 ^ tswz(c0 + e);
        const bf16x4 d = {dx[it][0][e], dx[it][1][e], dx[it][2][e], dx[it][3][e]};
        *reinterpret_cast<bf16x4*>(Dt + row * SC + col) = d;
        *reinterpret_cast<bf16x4*>(Dst + row * SC + col) =
            to_bf16x4(f32x4{(float)d[0] * sc[0], (float)d[1] * sc[1], (float)d[2] * sc[2], (float)d[3] * sc[3]});
      }
    }
  }
  __syncthreads();
  for (int f = wave; f < 4 * NV; f += NW) {
    const int ct = f / NV, vt = f - ct * NV;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
      mma_k32(acc, frag_from_trow(Pt, 16 * ct + lc, SC, 32 * ib), frag_from_trow(Dt, 16 * vt + lc, SC, 32 * ib));
    dvl[((hs * NV + vt) * 4 + ct) * 64 + lane] = acc * geo.scale;
  }
  __syncthreads();
  // C. q^T from the natural rows (4 rows x 8 columns per thread); bq.
  {
    constexpr int CB = K / 8, NB = (kChunk / 4) * CB;
    for (int b = tid; b < NB; b += TH) {
      const int r0 = 4 * (b / CB), c0 = 8 * (b % CB);
      bf16x8 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = *reinterpret_cast<const bf16x8*>(Qn + (r0 + j) * SK + c0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16x4 col = {x[0][e], x[1][e], x[2][e], x[3][e]};
        *reinterpret_cast<bf16x4*>(Qt + (c0 + e) * SC + (r0 ^ tswz(c0 + e))) = col;
      }
    }
  }
  __syncthreads();
  for (int f = wave; f < KT * NV; f += NW) {
    const int mt = f / NV, vt = f - mt * NV;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      mma_k32(acc, frag_from_trow(Qt, 16 * mt + lc, SC, 32 * cb), frag_from_trow(Dst, 16 * vt + lc, SC, 32 * cb));
    bq[((hs * NV + vt) * KT + mt) * 64 + lane] = make_quad<bf16>(acc);
  }
  // D. w from its forward fragments (rows c = 16 ct + lane%16, k = 32 kb + kslot)
  // into the q rows' space (free since q^T was built), then w^T fragments.
  for (int f = wave; f < 4 * KB; f += NW) {
    const int ct = f / KB, kb = f - ct * KB, c = 16 * ct + lc;
    const Frag<bf16> x = wf[((hs * 4 + ct) * KB + kb) * 64 + lane];
    *reinterpret_cast<bf16x4*>(Wn + c * SK + 32 * kb + 4 * g) = __builtin_shufflevector(x.x, x.x, 0, 1, 2, 3);
    *reinterpret_cast<bf16x4*>(Wn + c * SK + 32 * kb + 16 + 4 * g) = __builtin_shufflevector(x.x, x.x, 4, 5, 6, 7);
  }
  __syncthreads();
  for (int f = wave; f < KT * 2; f += NW) {
    const int mt = f >> 1, cb = f & 1, kk = 16 * mt + lc;
    bf16x8 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i] = Wn[(32 * cb + 4 * g + i) * SK + kk];
      y[4 + i] = Wn[(32 * cb + 16 + 4 * g + i) * SK + kk];
    }
    wtf[(hs * KT * 2 + f) * 64 + lane] = Frag<bf16>{y};
  }
}

// (at most 128 VGPRs: two eight-wave workgroups per CU)
template <int K, int V, bool VARLEN>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(4))) void gdn_bwd_dqk_bf16_kernel(
    Geo geo, const bf16* __restrict__ qg, const bf16* __restrict__ kg,
    const bf16* __restrict__ dog, const int4* __restrict__ cmap, const float* __restrict__ gam,
    const bf16* __restrict__ vnp, const bf16* __restrict__ dvn, const bf16* __restrict__ hcp,
    const bf16* __restrict__ dhn, float* __restrict__ dqp, float* __restrict__ dkp,
    bf16* __restrict__ dwp, float* __restrict__ dgp, bf16* __restrict__ dqg) {
  constexpr int SK = PadB<K>::v, SV = PadB<V>::v, SC = PadB<kChunk>::v;
  constexpr int NKT = K / 64, TH = kBwdThreads;
  constexpr int P12 = 2 * kChunk * SV + K * SV, P3 = 2 * kChunk * SK + 2 * K * SC;
  static_assert(kChunk * SC <= kChunk * SK, "dPm tiles fit in the q / k tiles");
  __shared__ __align__(16) bf16 lds[P12 > P3 ? P12 : P3];
  __shared__ float sg[kChunk], dG[kChunk], red[2];
  bf16* const Ds = lds;                        // do [64][V]
  bf16* const Xs = lds + kChunk * SV;          // dv_new, then v_new [64][V] (transposed-written)
  bf16* const Hs = lds + 2 * kChunk * SV;      // H_c, then dH_{c+1} [K][V] (transposed-written)
  bf16* const Qs = lds;                        // q [64][K], then dPm [64][64]
  bf16* const Ks = lds + kChunk * SK;          // k [64][K], then dPm^T [64][64] (transposed-written)
  bf16* const Qt = lds + 2 * kChunk * SK;      // q^T [K][64] (transposed-written)
  bf16* const Kt = Qt + K * SC;                // k^T [K][64] (transposed-written)
  bf16* const Pd = Qs;
  bf16* const Pt = Ks;

  int hv, slot;
  xcd_slot_block(blockIdx.x, geo.H, geo.G, geo.slots, hv, slot);
  int n, len;
  int64_t t0;
  if (!chunk_of_slot<VARLEN>(geo, cmap, slot, n, t0, len)) return;
  const int h = hv / geo.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, lc = lane & 15;
  const size_t hs = (size_t)hv * geo.slots + slot;
  const int rt0 = 2 * (wave >> 2), kc0 = (wave & 3) * (K / 4);  // 64 x K ownership
  const int pit = wave >> 1, pj0 = 2 * (wave & 1);               // 64 x 64 ownership
  const bf16* Hc = hcp + hs * K * V;
  const bf16* dHn = dhn + hs * K * V;

  // H_c^T and dH_{c+1}^T ([V][K] bf16) in 4 x 4 blocks: their dot in fp32;
  // H_c goes to LDS now, dH_{c+1} stays in registers (already rounded to bf16,
  // transposed) until the second staging.
  constexpr int HBC = K / 4, HNB = (V / 4) * HBC, HPER = (HNB + TH - 1) / TH;
  bf16x4 hd[HPER][4];
  {
    float acc = 0.f;
#pragma unroll
    for (int it = 0; it < HPER; ++it) {
      const int b = tid + TH * it;
      if (HNB % TH == 0 || b < HNB) {
        const int r0 = 4 * (b / HBC), c0 = 4 * (b % HBC);
        f32x4 hc[4], dh[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hc[j] = to_f32x4(*reinterpret_cast<const bf16x4*>(Hc + (size_t)(r0 + j) * K + c0));
          dh[j] = to_f32x4(*reinterpret_cast<const bf16x4*>(dHn + (size_t)(r0 + j) * K + c0));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 p = hc[j] * dh[j];
          acc += (p[0] + p[1]) + (p[2] + p[3]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          st4(Hs + (c0 + j) * SV + (r0 ^ tswz(c0 + j)), hc[0][j], hc[1][j], hc[2][j], hc[3][j]);
          hd[it][j] = to_bf16x4(f32x4{dh[0][j], dh[1][j], dh[2][j], dh[3][j]});
        }
      }
    }
    acc = wave_sum(acc);
    if (tid < kChunk) {
      sg[tid] = gam[hs * kChunk + tid];
      dG[tid] = 0.f;
    }
    if (tid == 0) red[1] = 0.f;
    if (tid == 64) red[0] = 0.f;
    __syncthreads();
    if (lane == 0) atomicAdd(&red[0], acc);
  }
  stage_rows_b<V, TH>(Ds, SV, dog + (size_t)hv * V, t0, (int64_t)geo.HV * V, len);
  stage_t<V, kChunk, SV, TH>(Xs, dvn + hs * kChunk * V);
  __syncthreads();
  const float gl = sg[kChunk - 1];

  // dq_inter = scale e^G (do H_c^T) and dw = -dv_new H_c^T.
  const int npair = pit >= pj0 + 1 ? 2 : pit >= pj0 ? 1 : 0;
  f32x4 dq[2][NKT], dk[2][NKT];
  {
    f32x4 dw[2][NKT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) dq[a][nt] = dw[a][nt] = dk[a][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int vb = 0; vb < V / 32; ++vb) {
      Frag<bf16> da[2], xa[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        da[a] = frag_from_row(Ds + (16 * (rt0 + a) + lc) * SV + 32 * vb);
        xa[a] = frag_from_trow(Xs, 16 * (rt0 + a) + lc, SV, 32 * vb);
      }
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) {
        const Frag<bf16> hb = frag_from_trow(Hs, kc0 + 16 * nt + lc, SV, 32 * vb);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          mma_k32(dq[a][nt], da[a], hb);
          mma_k32(dw[a][nt], xa[a], hb);
        }
      }
    }
    // (lane base + constant offsets: no per-store 64-bit address arithmetic)
    bf16* const dwl = dwp + (hs * kChunk + 16 * rt0 + 4 * g) * K + kc0 + lc;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = geo.scale * fast_exp2(sg[16 * (rt0 + a) + 4 * g + r]);
#pragma unroll
        for (int nt = 0; nt < NKT; ++nt) {
          dq[a][nt][r] *= e;
          dwl[(16 * a + r) * K + 16 * nt] = (bf16)(-dw[a][nt][r]);
        }
      }
    // scaled here, not deferred to the end (which would keep the factors live)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) asm volatile("" : "+v"(dq[a][nt]));
  }
  __syncthreads();
  // v_new and dH_{c+1} replace dv_new and H_c.
  stage_t<V, kChunk, SV, TH>(Xs, vnp + hs * kChunk * V);
#pragma unroll
  for (int it = 0; it < HPER; ++it) {
    const int b = tid + TH * it;
    if (HNB % TH == 0 || b < HNB) {
      const int r0 = 4 * (b / HBC), c0 = 4 * (b % HBC);
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<bf16x4*>(Hs + (c0 + j) * SV + (r0 ^ tswz(c0 + j))) = hd[it][j];
    }
  }
  __syncthreads();
  // dPm = scale (do v_new^T) * M * e^{dG};  dk_kd = e^{G_last - G} (v_new dH_{c+1}^T)
  f32x4 dPm[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll 1
  for (int vb = 0; vb < V / 32; ++vb) {
    const Frag<bf16> da = frag_from_row(Ds + (16 * pit + lc) * SV + 32 * vb);
    if (npair >= 1) mma_k32(dPm[0], da, frag_from_trow(Xs, 16 * pj0 + lc, SV, 32 * vb));
    if (npair >= 2) mma_k32(dPm[1], da, frag_from_trow(Xs, 16 * (pj0 + 1) + lc, SV, 32 * vb));
    Frag<bf16> xa[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) xa[a] = frag_from_trow(Xs, 16 * (rt0 + a) + lc, SV, 32 * vb);
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      const Frag<bf16> hb = frag_from_trow(Hs, kc0 + 16 * nt + lc, SV, 32 * vb);
#pragma unroll
      for (int a = 0; a < 2; ++a) mma_k32(dk[a][nt], xa[a], hb);
    }
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int jt = pj0 + b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * pit + 4 * g + r, j = 16 * jt + lc;
      dPm[b][r] = j <= i ? dPm[b][r] * geo.scale * fast_exp2(sg[i] - sg[j]) : 0.f;
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = fast_exp2(gl - sg[16 * (rt0 + a) + 4 * g + r]);
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) dk[a][nt][r] *= e;
    }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) asm volatile("" : "+v"(dk[a][nt]));
  __syncthreads();

  // q and k: rows [64][K] and transposed [K][64] from one load of 4 rows x 8
  // columns per thread (q on threads 0..255, k on 256..511).
  {
    constexpr int CB = K / 8, NB = (kChunk / 4) * CB;
    static_assert(NB <= 256, "one block per thread");
    const int half = tid >> 8, t = tid & 255;
    if (t < NB) {
      const bf16* src = (half ? kg : qg) + (size_t)h * K;
      bf16* nat = half ? Ks : Qs;
      bf16* tr = half ? Kt : Qt;
      const int r0 = 4 * (t / CB), c0 = 8 * (t % CB);
      bf16x8 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = bf16x8{};
        if (r0 + j < len) x[j] = *reinterpret_cast<const bf16x8*>(src + ((t0 + r0 + j) * geo.H) * K + c0);
        *reinterpret_cast<bf16x8*>(nat + (r0 + j) * SK + c0) = x[j];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<bf16x4*>(tr + (c0 + e) * SC + (r0 ^ tswz(c0 + e))) =
            bf16x4{x[0][e], x[1][e], x[2][e], x[3][e]};
    }
  }
  __syncthreads();
  // R = dPm * (Q K^T): dG_i += row sums, dG_j -= column sums.
  f32x4 sq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int kb = 0; kb < K / 32; ++kb) {
    const Frag<bf16> qa = frag_from_row(Qs + (16 * pit + lc) * SK + 32 * kb);
    if (npair >= 1) mma_k32(sq[0], qa, frag_from_row(Ks + (16 * pj0 + lc) * SK + 32 * kb));
    if (npair >= 2) mma_k32(sq[1], qa, frag_from_row(Ks + (16 * (pj0 + 1) + lc) * SK + 32 * kb));
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int jt = pj0 + b;
    float cs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rr = dPm[b][r] * sq[b][r];
      cs += rr;
      const float rs = sum16(rr);
      if (lc == 0) atomicAdd(&dG[16 * pit + 4 * g + r], rs);
    }
    cs = sum_groups(cs);
    if (g == 0) atomicAdd(&dG[16 * jt + lc], -cs);
  }
  // dG_i += q_i . dq_inter_i;  x_j = k_j . dk_kd_j: dG_j -= x_j, sum x -> red[1].
  {
    float xs = 0.f;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * (rt0 + a) + 4 * g + r;
        float qd = 0.f, kx = 0.f;
#pragma unroll
        for (int nt = 0; nt < NKT; ++nt) {
          const int kk = kc0 + 16 * nt + lc;
          qd += (float)Qs[i * SK + kk] * dq[a][nt][r];
          kx += (float)Ks[i * SK + kk] * dk[a][nt][r];
        }
        qd = sum16(qd);
        kx = sum16(kx);
        if (lc == 0) atomicAdd(&dG[i], qd - kx);
        xs += lc == 0 ? kx : 0.f;
      }
    xs = wave_sum(xs);
    if (lane == 0) atomicAdd(&red[1], xs);
  }
  __syncthreads();
  // dPm (rows i) over q's tile, dPm^T (rows j, transposed-written) over k's.
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int j = 16 * (pj0 + b) + lc, i0 = 16 * pit + 4 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) Pd[(i0 + r) * SC + j] = (bf16)dPm[b][r];
    st4(Pt + j * SC + (i0 ^ tswz(j)), dPm[b][0], dPm[b][1], dPm[b][2], dPm[b][3]);
  }
  __syncthreads();
  // dq += dPm K;  dk += dPm^T Q.
#pragma unroll
  for (int cb = 0; cb < kChunk / 32; ++cb) {
    Frag<bf16> pa[2], pta[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      pa[a] = frag_from_row(Pd + (16 * (rt0 + a) + lc) * SC + 32 * cb);
      pta[a] = frag_from_trow(Pt, 16 * (rt0 + a) + lc, SC, 32 * cb);
    }
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      const Frag<bf16> kb = frag_from_trow(Kt, kc0 + 16 * nt + lc, SC, 32 * cb);
      const Frag<bf16> qb = frag_from_trow(Qt, kc0 + 16 * nt + lc, SC, 32 * cb);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        mma_k32(dq[a][nt], pa[a], kb);
        mma_k32(dk[a][nt], pta[a], qb);
      }
    }
  }
  {
    const size_t o = (hs * kChunk + 16 * rt0 + 4 * g) * K + kc0 + lc;
    float* const dkl = dkp + o;
    float* const dql = dqp + o;
    const int i0 = 16 * rt0 + 4 * g;
    bf16* const dqo = dqg + ((t0 + i0) * geo.H + h) * K + kc0 + lc;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int nt = 0; nt < NKT; ++nt) {
          const int off = (16 * a + r) * K + 16 * nt;
          // one value head per key head: dq is final here
          if (geo.G == 1) {
            if (i0 + 16 * a + r < len) dqo[(size_t)(16 * a + r) * geo.H * K + 16 * nt] = (bf16)dq[a][nt][r];
          } else {
            dql[off] = dq[a][nt][r];
          }
          dkl[off] = dk[a][nt][r];
        }
  }
  if (tid < kChunk) {
    float x = dG[tid];
    if (tid == kChunk - 1) x += red[1] + fast_exp2(gl) * red[0];
    dgp[hs * kChunk + tid] = x;
  }
}

// ---------------------------------------------------------------------------
// WY backward, the chunk-local dG scan and the gate backward, one workgroup
// per (chunk slot, value head).  Adds its dk terms to dkp (or, with one value
// head per key head, writes the final dk); writes dv (dtype), dbeta and dg_raw
// (fp32) for the chunk's tokens and the chunk's sums for dA_log and ddt_bias.
template <typename E, int K, int V, bool VARLEN>
__global__ __launch_bounds__(kBwdThreads) void gdn_bwd_wy_kernel(
    Geo geo, const E* __restrict__ kg, const E* __restrict__ vg, const float* __restrict__ g_raw,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    const int4* __restrict__ cmap, const float* __restrict__ gam, const float* __restrict__ bet,
    const float* __restrict__ tmat, const float* __restrict__ dwp, const float* __restrict__ dvn,
    const float* __restrict__ dgp, float* __restrict__ dkp, E* __restrict__ dvg,
    float* __restrict__ dbeta, float* __restrict__ dg_raw, float* __restrict__ dAp,
    float* __restrict__ dbp, E* __restrict__ dkg) {
  constexpr int KP = Pad<K>::v, VP = Pad<V>::v, NKT = K / 64, NVT = V / 64, TH = kBwdThreads;
  __shared__ __align__(16) float Ks[kChunk * KP];
  __shared__ __align__(16) float Vs[kChunk * VP];  // later dT, dS
  __shared__ __align__(16) float Wd[kChunk * KP];
  __shared__ __align__(16) float Dv[V * kCP];      // dv_new^T [V][64], later Y
  __shared__ __align__(16) float Tt[kChunk * kCP];
  __shared__ float sg[kChunk], sb[kChunk], dG[kChunk], dB[kChunk];
  float* const dTs = Vs;
  float* const Ys = Dv;

  int hv, slot;
  xcd_slot_block(blockIdx.x, geo.H, geo.G, geo.slots, hv, slot);
  const size_t hs = (size_t)hv * geo.slots + slot;
  int n, len;
  int64_t t0;
  if (!chunk_of_slot<VARLEN>(geo, cmap, slot, n, t0, len)) {
    if (threadIdx.x == 0) {
      dAp[hs] = 0.f;
      dbp[hs] = 0.f;
    }
    return;
  }
  const int h = hv / geo.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, lc = lane & 15;
  const int rt0 = 2 * (wave >> 2), kc0 = (wave & 3) * (K / 4), vc0 = (wave & 3) * (V / 4);
  const int pit = wave >> 1, pj0 = 2 * (wave & 1);

  stage_rows<K, E, kChunk, TH>(Ks, KP, kg + (size_t)h * K, t0, (int64_t)geo.H * K, len);
  stage_rows<V, E, kChunk, TH>(Vs, VP, vg + (size_t)hv * V, t0, (int64_t)geo.HV * V, len);
  stage_rows<K, float, kChunk, TH>(Wd, KP, dwp + hs * kChunk * K, 0, K, kChunk);
  stage_rows<kChunk, float, V, TH>(Dv, kCP, dvn + hs * kChunk * V, 0, kChunk, V);
  stage_rows<kChunk, float, kChunk, TH>(Tt, kCP, tmat + hs * kChunk * kChunk, 0, kChunk, kChunk);
  if (tid < kChunk) {
    sg[tid] = gam[hs * kChunk + tid];
    sb[tid] = bet[hs * kChunk + tid];
    dG[tid] = 0.f;
    dB[tid] = 0.f;
  }
  // the dq/dk kernel's dk terms of this wave's tiles, loaded now and used at
  // the end (their latency hides behind the whole kernel)
  float dk0[2][NKT][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dk0[a][nt][r] = dkp[(hs * kChunk + 16 * (rt0 + a) + 4 * g + r) * K + kc0 + 16 * nt + lc];
  __syncthreads();

  // dT (strictly lower part; the rest does not reach dA).
  const int npair = pit >= pj0 + 1 ? 2 : pit >= pj0 ? 1 : 0;
  f32x4 dT[2];
  {
    f32x4 x[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 y[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    mm_pair<K>(x, npair, Wd + 16 * pit * KP, KP, 1, Ks + 16 * pj0 * KP, 1, KP);
    mm_pair<V>(y, npair, Dv + 16 * pit, 1, kCP, Vs + 16 * pj0 * VP, 1, VP);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = 16 * (pj0 + b) + lc;
      const float fw = sb[j] * fast_exp2(sg[j]), fu = sb[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * pit + 4 * g + r;
        dT[b][r] = j < i ? x[b][r] * fw + y[b][r] * fu : 0.f;
      }
    }
  }
  // X_w = T^T dw: dk += beta e^G X_w and the k . X_w terms of dbeta and dG.
  f32x4 dk[2][NKT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) dk[a][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  mm_block<kChunk, 2, NKT>(dk, Tt + 16 * rt0, 1, kCP, Wd + kc0, KP, 1);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int jt = rt0 + a;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * jt + 4 * g + r;
      const float eg = fast_exp2(sg[j]);
      float kx = 0.f;
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) kx += Ks[j * KP + kc0 + 16 * nt + lc] * dk[a][nt][r];
      kx = sum16(kx);
      if (lc == 0) {
        atomicAdd(&dB[j], eg * kx);
        atomicAdd(&dG[j], sb[j] * eg * kx);
      }
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) dk[a][nt][r] *= sb[j] * eg;
    }
  }
  // X_u = T^T dv_new: dv = beta X_u, the v . X_u term of dbeta.
  f32x4 xu[2][NVT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nv = 0; nv < NVT; ++nv) xu[a][nv] = f32x4{0.f, 0.f, 0.f, 0.f};
  mm_block<kChunk, 2, NVT>(xu, Tt + 16 * rt0, 1, kCP, Dv + vc0 * kCP, 1, kCP);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int jt = rt0 + a;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * jt + 4 * g + r;
      float vx = 0.f;
#pragma unroll
      for (int nv = 0; nv < NVT; ++nv) {
        const int vv = vc0 + 16 * nv + lc;
        vx += Vs[j * VP + vv] * xu[a][nv][r];
        if (j < len) dvg[((t0 + j) * geo.HV + hv) * V + vv] = (E)(sb[j] * xu[a][nv][r]);
      }
      vx = sum16(vx);
      if (lc == 0) atomicAdd(&dB[j], vx);
    }
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) dTs[(16 * pit + 4 * g + r) * kCP + 16 * (pj0 + b) + lc] = dT[b][r];
  __syncthreads();
  // Y = T^T dT.
  {
    f32x4 y[1][2] = {{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}};
    mm_block<kChunk, 1, 2>(y, Tt + 16 * pit, 1, kCP, dTs + 16 * pj0, kCP, 1);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) Ys[(16 * pit + 4 * g + r) * kCP + 16 * (pj0 + b) + lc] = y[0][b][r];
  }
  __syncthreads();
  // dA = -strictly_lower(Y T^T); with S = K K^T and A = beta_i e^{dG} S:
  // dG += rows - columns of dA * A, dbeta += rows of dA e^{dG} S, dS = dA beta e^{dG}.
  f32x4 dS[2];
  f32x4 yy[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  f32x4 ss[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  mm_pair<kChunk>(yy, npair, Ys + 16 * pit * kCP, kCP, 1, Tt + 16 * pj0 * kCP, 1, kCP);
  mm_pair<K>(ss, npair, Ks + 16 * pit * KP, KP, 1, Ks + 16 * pj0 * KP, 1, KP);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int jt = pj0 + b;
    const f32x4 y = yy[b], sk = ss[b];
    const int c = 16 * jt + lc;
    float cs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ar = 16 * pit + 4 * g + r;
      // above the diagonal e^{G_a - G_c} can overflow: select, never multiply by 0
      const float da = c < ar ? -y[r] : 0.f;
      const float e = c < ar ? fast_exp2(sg[ar] - sg[c]) : 0.f;
      const float des = da * e * sk[r];
      const float z = des * sb[ar];
      cs += z;
      const float rz = sum16(z), rb = sum16(des);
      if (lc == 0) {
        atomicAdd(&dG[ar], rz);
        atomicAdd(&dB[ar], rb);
      }
      dS[b][r] = da * sb[ar] * e;
    }
    cs = sum_groups(cs);
    if (g == 0) atomicAdd(&dG[c], -cs);
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) dTs[(16 * pit + 4 * g + r) * kCP + 16 * (pj0 + b) + lc] = dS[b][r];
  __syncthreads();
  // dk += (dS + dS^T) K; add the dq/dk kernel's terms and store.
  mm_block<kChunk, 2, NKT>(dk, dTs + 16 * rt0 * kCP, kCP, 1, Ks + kc0, KP, 1);
  mm_block<kChunk, 2, NKT>(dk, dTs + 16 * rt0, 1, kCP, Ks + kc0, KP, 1);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int jt = rt0 + a;
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      const int kc = kc0 + 16 * nt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jt + 4 * g + r;
        const size_t o = (hs * kChunk + j) * K + kc + lc;
        // one value head per key head: dk is final here
        if (geo.G == 1) {
          if (j < len) dkg[((t0 + j) * geo.H + h) * K + kc + lc] = (E)(dk0[a][nt][r] + dk[a][nt][r]);
        } else {
          dkp[o] = dk0[a][nt][r] + dk[a][nt][r];
        }
      }
    }
  }
  __syncthreads();
  // dg = reversed chunk-local cumsum of dG; gate backward.
  if (wave == 0) {
    float x = dG[lane] + dgp[hs * kChunk + lane];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(x, off, 64);
      if (lane + off < 64) x += y;
    }
    float sa = 0.f, sbias = 0.f;
    if (lane < len) {
      const int64_t t = t0 + lane;
      const float xr = g_raw[t * geo.HV + hv] + (dt_bias ? dt_bias[hv] : 0.f);
      const float ea = expf(A_log[hv]);
      const float gt = -ea * gate_softplus(xr);
      const float slope = xr > 20.f ? 1.f : 1.f / (1.f + fast_exp2(-xr * kLog2e));
      const float dgr = x * (-ea) * slope;
      dbeta[t * geo.HV + hv] = dB[lane];
      dg_raw[t * geo.HV + hv] = dgr;
      sa = x * gt;
      sbias = dgr;
    }
    sa = sum64(sa);
    sbias = sum64(sbias);
    if (lane == 0) {
      dAp[hs] = sa;
      dbp[hs] = sbias;
    }
  }
}

// ---------------------------------------------------------------------------
// The WY backward for bf16 calls: the products of gdn_bwd_wy_kernel on the bf16
// MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation) with every operand staged
// in LDS as bf16: k and v exactly, dw, dv_new, T, dT, Y and dS rounded once
// when staged.  The masks, decays, dbeta / dG sums and the gate backward are
// the fp32 kernel's.  Operands whose reduction index is a column of the stored
// layout are written transposed (swizzled by tswz, read with frag_from_trow);
// the others as natural rows (frag_from_row).  LDS is K natural plus one pool
// reused phase by phase (~70 KB at K = V = 128: two workgroups per CU):
//   1 (dT):        dw [64][K], v [64][V], dv_new [64][V] (transposed-written)
//   2 (X_w, X_u):  dw^T [K][64] (t-w), dv_new^T [V][64], T^T [64][64] (t-w)
//   3 (Y):         dT^T (t-w), T^T; then Y natural
//   4 (dA, dS):    Y, T natural, K
//   5 (dk):        K^T (t-w), dS natural, dS^T (t-w)
// dw, dv_new and T are read from memory once, at the start, into registers (as
// bf16), and written to LDS in each layout when its phase comes.
template <int R, int C>
struct Blk4 {  // 4 x 4 blocks of an R x C matrix, one per thread and step
  static constexpr int BC = C / 4, NB = (R / 4) * BC, PER = (NB + kBwdThreads - 1) / kBwdThreads;
};

// (at most 128 VGPRs: two eight-wave workgroups per CU)
template <int K, int V, bool VARLEN>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(4))) void gdn_bwd_wy_bf16_kernel(
    Geo geo, const bf16* __restrict__ kg, const bf16* __restrict__ vg,
    const float* __restrict__ g_raw, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const int4* __restrict__ cmap,
    const float* __restrict__ gam, const float* __restrict__ bet, const bf16* __restrict__ tmat,
    const bf16* __restrict__ dwp, const bf16* __restrict__ dvn, const float* __restrict__ dgp,
    float* __restrict__ dkp, bf16* __restrict__ dvg, float* __restrict__ dbeta,
    float* __restrict__ dg_raw, float* __restrict__ dAp, float* __restrict__ dbp,
    bf16* __restrict__ dkg) {
  constexpr int SK = PadB<K>::v, SV = PadB<V>::v, SC = PadB<kChunk>::v;
  constexpr int NKT = K / 64, NVT = V / 64, TH = kBwdThreads;
  constexpr int KN = kChunk * SK;
  constexpr int P1 = kChunk * SK + 2 * kChunk * SV;
  constexpr int P2 = (K + V + kChunk) * SC;
  constexpr int P5 = (K + 2 * kChunk) * SC;
  constexpr int POOL = P1 > P2 ? (P1 > P5 ? P1 : P5) : (P2 > P5 ? P2 : P5);
  constexpr int TT = (K + V) * SC;  // T^T, phases 2-3
  static_assert(TT >= 2 * kChunk * SC, "dT^T and Y fit below T^T");
  __shared__ __align__(16) bf16 lds[KN + POOL];
  __shared__ float sg[kChunk], sb[kChunk], dG[kChunk], dB[kChunk];
  bf16* const Kn = lds;
  bf16* const pool = lds + KN;
  bf16* const Wn = pool;                    // 1: dw
  bf16* const Vn = pool + kChunk * SK;      // 1: v
  bf16* const Dn = Vn + kChunk * SV;        // 1: dv_new (t-w from [V][64])
  bf16* const Wt = pool;                    // 2: dw^T (t-w)
  bf16* const Dt = pool + K * SC;           // 2: dv_new^T rows
  bf16* const Tt = pool + TT;               // 2-3: T^T (t-w)
  bf16* const dTt = pool;                   // 3: dT^T (t-w)
  bf16* const Yn = pool + kChunk * SC;      // 3-4: Y
  bf16* const Tn = pool;                    // 4: T
  bf16* const Kt = pool;                    // 5: K^T (t-w)
  bf16* const Sn = pool + K * SC;           // 5: dS
  bf16* const St = Sn + kChunk * SC;        // 5: dS^T (t-w)

  int hv, slot;
  xcd_slot_block(blockIdx.x, geo.H, geo.G, geo.slots, hv, slot);
  const size_t hs = (size_t)hv * geo.slots + slot;
  int n, len;
  int64_t t0;
  if (!chunk_of_slot<VARLEN>(geo, cmap, slot, n, t0, len)) {
    if (threadIdx.x == 0) {
      dAp[hs] = 0.f;
      dbp[hs] = 0.f;
    }
    return;
  }
  const int h = hv / geo.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, lc = lane & 15;
  const int rt0 = 2 * (wave >> 2), kc0 = (wave & 3) * (K / 4), vc0 = (wave & 3) * (V / 4);
  // The chunk's rows as wave-uniform base pointers with 32-bit offsets (the
  // host rejects 64 H K or 64 HV V beyond int32): per-element 64-bit addresses
  // kept from here to the stores spilled to scratch memory.
  const int kstride = geo.H * K, vstride = geo.HV * V;
  const bf16* const vrow = vg + (t0 * geo.HV + hv) * V;
  bf16* const dvrow = dvg + (t0 * geo.HV + hv) * V;
  bf16* const dkrow = dkg + (t0 * geo.H + h) * K;
  float* const dkpc = dkp + hs * kChunk * K;
  const int pit = wave >> 1, pj0 = 2 * (wave & 1);

  // dw [64][K], dv_new^T [V][64] and T [64][64] (bf16) into registers,
  // 4 x 4 blocks per thread: row j of block b is w[b][j].
  using BW = Blk4<kChunk, K>;
  using BD = Blk4<V, kChunk>;
  using BT = Blk4<kChunk, kChunk>;
  bf16x4 wr[BW::PER][4], dr[BD::PER][4], tr[BT::PER][4];
  auto fetch = [&](auto B, bf16x4 (&dst)[decltype(B)::PER][4], const bf16* src, int C) {
    using Bk = decltype(B);
#pragma unroll
    for (int it = 0; it < Bk::PER; ++it) {
      const int b = tid + TH * it;
      if (Bk::NB % TH == 0 || b < Bk::NB) {
        const int r0 = 4 * (b / Bk::BC), c0 = 4 * (b % Bk::BC);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          dst[it][j] = *reinterpret_cast<const bf16x4*>(src + (size_t)(r0 + j) * C + c0);
      }
    }
  };
  fetch(BW{}, wr, dwp + hs * kChunk * K, K);
  fetch(BD{}, dr, dvn + hs * kChunk * V, kChunk);
  fetch(BT{}, tr, tmat + hs * kChunk * kChunk, kChunk);
  // natural rows of a held block matrix: dst[(r0 + j) * ld + c0 ..] = row j
  auto put_nat = [&](auto B, const bf16x4 (&src)[decltype(B)::PER][4], bf16* dst, int ld) {
    using Bk = decltype(B);
#pragma unroll
    for (int it = 0; it < Bk::PER; ++it) {
      const int b = tid + TH * it;
      if (Bk::NB % TH == 0 || b < Bk::NB) {
        const int r0 = 4 * (b / Bk::BC), c0 = 4 * (b % Bk::BC);
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<bf16x4*>(dst + (r0 + j) * ld + c0) = src[it][j];
      }
    }
  };
  // transposed, swizzled: dst[c][r] = m[r][c]
  auto put_tr = [&](auto B, const bf16x4 (&src)[decltype(B)::PER][4], bf16* dst, int ld) {
    using Bk = decltype(B);
#pragma unroll
    for (int it = 0; it < Bk::PER; ++it) {
      const int b = tid + TH * it;
      if (Bk::NB % TH == 0 || b < Bk::NB) {
        const int r0 = 4 * (b / Bk::BC), c0 = 4 * (b % Bk::BC);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 col;
#pragma unroll
          for (int i = 0; i < 4; ++i) col[i] = src[it][i][j];
          *reinterpret_cast<bf16x4*>(dst + (c0 + j) * ld + (r0 ^ tswz(c0 + j))) = col;
        }
      }
    }
  };

  stage_rows_b<K, TH>(Kn, SK, kg + (size_t)h * K, t0, (int64_t)geo.H * K, len);
  stage_rows_b<V, TH>(Vn, SV, vg + (size_t)hv * V, t0, (int64_t)geo.HV * V, len);
  put_nat(BW{}, wr, Wn, SK);
  put_tr(BD{}, dr, Dn, SV);
  if (tid < kChunk) {
    sg[tid] = gam[hs * kChunk + tid];
    sb[tid] = bet[hs * kChunk + tid];
    dG[tid] = 0.f;
    dB[tid] = 0.f;
  }
  __syncthreads();

  // 1. dT (strictly lower part): x = dw K^T, y = dv_new V^T.
  const int npair = pit >= pj0 + 1 ? 2 : pit >= pj0 ? 1 : 0;
  f32x4 dT[2];
  {
    f32x4 x[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 y[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (npair > 0) {
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) {
        const Frag<bf16> a = frag_from_row(Wn + (16 * pit + lc) * SK + 32 * kb);
        mma_k32(x[0], a, frag_from_row(Kn + (16 * pj0 + lc) * SK + 32 * kb));
        if (npair > 1) mma_k32(x[1], a, frag_from_row(Kn + (16 * (pj0 + 1) + lc) * SK + 32 * kb));
      }
#pragma unroll
      for (int vb = 0; vb < V / 32; ++vb) {
        const Frag<bf16> a = frag_from_trow(Dn, 16 * pit + lc, SV, 32 * vb);
        mma_k32(y[0], a, frag_from_row(Vn + (16 * pj0 + lc) * SV + 32 * vb));
        if (npair > 1) mma_k32(y[1], a, frag_from_row(Vn + (16 * (pj0 + 1) + lc) * SV + 32 * vb));
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = 16 * (pj0 + b) + lc;
      const float fw = sb[j] * fast_exp2(sg[j]), fu = sb[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * pit + 4 * g + r;
        dT[b][r] = j < i ? x[b][r] * fw + y[b][r] * fu : 0.f;
      }
    }
  }
  __syncthreads();
  put_tr(BW{}, wr, Wt, SC);
  put_nat(BD{}, dr, Dt, SC);
  put_tr(BT{}, tr, Tt, SC);
  __syncthreads();

  // 2. X_w = T^T dw: dk += beta e^G X_w and the k . X_w terms of dbeta, dG;
  //    X_u = T^T dv_new: dv = beta X_u and the v . X_u term of dbeta.
  f32x4 dk[2][NKT], xu[2][NVT];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) dk[a][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nv = 0; nv < NVT; ++nv) xu[a][nv] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll 1
  for (int ib = 0; ib < 2; ++ib) {
    Frag<bf16> ta[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) ta[a] = frag_from_trow(Tt, 16 * (rt0 + a) + lc, SC, 32 * ib);
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      const Frag<bf16> wb = frag_from_trow(Wt, kc0 + 16 * nt + lc, SC, 32 * ib);
#pragma unroll
      for (int a = 0; a < 2; ++a) mma_k32(dk[a][nt], ta[a], wb);
    }
#pragma unroll
    for (int nv = 0; nv < NVT; ++nv) {
      const Frag<bf16> db = frag_from_row(Dt + (vc0 + 16 * nv + lc) * SC + 32 * ib);
#pragma unroll
      for (int a = 0; a < 2; ++a) mma_k32(xu[a][nv], ta[a], db);
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int jt = rt0 + a;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * jt + 4 * g + r;
      const float eg = fast_exp2(sg[j]);
      float kx = 0.f, vx = 0.f;
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) kx += (float)Kn[j * SK + kc0 + 16 * nt + lc] * dk[a][nt][r];
#pragma unroll
      for (int nv = 0; nv < NVT; ++nv) {
        const int vv = vc0 + 16 * nv + lc;
        if (j < len) {
          vx += (float)vrow[j * vstride + vv] * xu[a][nv][r];
          dvrow[j * vstride + vv] = (bf16)(sb[j] * xu[a][nv][r]);
        }
      }
      kx = sum16(kx);
      vx = sum16(vx);
      if (lc == 0) {
        atomicAdd(&dB[j], eg * kx + vx);
        atomicAdd(&dG[j], sb[j] * eg * kx);
      }
#pragma unroll
      for (int nt = 0; nt < NKT; ++nt) dk[a][nt][r] *= sb[j] * eg;
    }
  }
  __syncthreads();
  // 3. Y = T^T dT.
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int j = 16 * (pj0 + b) + lc;
    *reinterpret_cast<bf16x4*>(dTt + j * SC + ((16 * pit + 4 * g) ^ tswz(j))) = to_bf16x4(dT[b]);
  }
  __syncthreads();
  {
    f32x4 y[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const Frag<bf16> ta = frag_from_trow(Tt, 16 * pit + lc, SC, 32 * ib);
#pragma unroll
      for (int b = 0; b < 2; ++b) mma_k32(y[b], ta, frag_from_trow(dTt, 16 * (pj0 + b) + lc, SC, 32 * ib));
    }
    // Y natural (below T^T, apart from dT^T)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) Yn[(16 * pit + 4 * g + r) * SC + 16 * (pj0 + b) + lc] = (bf16)y[b][r];
  }
  __syncthreads();
  put_nat(BT{}, tr, Tn, SC);
  __syncthreads();
  // 4. dA = -strictly_lower(Y T^T); with S = K K^T and A = beta_i e^{dG} S:
  //    dG += rows - columns of dA * A, dbeta += rows of dA e^{dG} S, dS = dA beta e^{dG}.
  f32x4 dS[2];
  {
    f32x4 yy[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 ss[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (npair > 0) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const Frag<bf16> a = frag_from_row(Yn + (16 * pit + lc) * SC + 32 * mb);
        mma_k32(yy[0], a, frag_from_row(Tn + (16 * pj0 + lc) * SC + 32 * mb));
        if (npair > 1) mma_k32(yy[1], a, frag_from_row(Tn + (16 * (pj0 + 1) + lc) * SC + 32 * mb));
      }
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) {
        const Frag<bf16> a = frag_from_row(Kn + (16 * pit + lc) * SK + 32 * kb);
        mma_k32(ss[0], a, frag_from_row(Kn + (16 * pj0 + lc) * SK + 32 * kb));
        if (npair > 1) mma_k32(ss[1], a, frag_from_row(Kn + (16 * (pj0 + 1) + lc) * SK + 32 * kb));
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int jt = pj0 + b;
      const f32x4 y = yy[b], sk = ss[b];
      const int c = 16 * jt + lc;
      float cs = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ar = 16 * pit + 4 * g + r;
        // above the diagonal e^{G_a - G_c} can overflow: select, never multiply by 0
        const float da = c < ar ? -y[r] : 0.f;
        const float e = c < ar ? fast_exp2(sg[ar] - sg[c]) : 0.f;
        const float des = da * e * sk[r];
        const float z = des * sb[ar];
        cs += z;
        const float rz = sum16(z), rb = sum16(des);
        if (lc == 0) {
          atomicAdd(&dG[ar], rz);
          atomicAdd(&dB[ar], rb);
        }
        dS[b][r] = da * sb[ar] * e;
      }
      cs = sum_groups(cs);
      if (g == 0) atomicAdd(&dG[c], -cs);
    }
  }
  __syncthreads();
  // the dq/dk kernel's dk terms of this wave's tiles (loaded here, not at the
  // start, to keep 16 registers free through the phases before)
  float dk0[2][NKT][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dk0[a][nt][r] = dkpc[(16 * (rt0 + a) + 4 * g + r) * K + kc0 + 16 * nt + lc];
  // 5. dk += (dS + dS^T) K.  K^T from the natural rows (4 rows x 8 columns per thread).
  {
    constexpr int CB = K / 8, NB = (kChunk / 4) * CB;
#pragma unroll
    for (int b = tid; b < NB; b += TH) {
      const int r0 = 4 * (b / CB), c0 = 8 * (b % CB);
      bf16x8 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = *reinterpret_cast<const bf16x8*>(Kn + (r0 + j) * SK + c0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 col = {x[0][e], x[1][e], x[2][e], x[3][e]};
        *reinterpret_cast<bf16x4*>(Kt + (c0 + e) * SC + (r0 ^ tswz(c0 + e))) = col;
      }
    }
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int j = 16 * (pj0 + b) + lc;
    *reinterpret_cast<bf16x4*>(St + j * SC + ((16 * pit + 4 * g) ^ tswz(j))) = to_bf16x4(dS[b]);
#pragma unroll
    for (int r = 0; r < 4; ++r) Sn[(16 * pit + 4 * g + r) * SC + j] = (bf16)dS[b][r];
  }
  __syncthreads();
#pragma unroll 1
  for (int ib = 0; ib < 2; ++ib) {
    Frag<bf16> sa[2], sat[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      sa[a] = frag_from_row(Sn + (16 * (rt0 + a) + lc) * SC + 32 * ib);
      sat[a] = frag_from_trow(St, 16 * (rt0 + a) + lc, SC, 32 * ib);
    }
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      const Frag<bf16> kb = frag_from_trow(Kt, kc0 + 16 * nt + lc, SC, 32 * ib);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        mma_k32(dk[a][nt], sa[a], kb);
        mma_k32(dk[a][nt], sat[a], kb);
      }
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int jt = rt0 + a;
#pragma unroll
    for (int nt = 0; nt < NKT; ++nt) {
      const int kc = kc0 + 16 * nt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jt + 4 * g + r;
        const int o = j * K + kc + lc;
        // one value head per key head: dk is final here
        if (geo.G == 1) {
          if (j < len) dkrow[j * kstride + kc + lc] = (bf16)(dk0[a][nt][r] + dk[a][nt][r]);
        } else {
          dkpc[o] = dk0[a][nt][r] + dk[a][nt][r];
        }
      }
    }
  }
  __syncthreads();
  // dg = reversed chunk-local cumsum of dG; gate backward.
  if (wave == 0) {
    float x = dG[lane] + dgp[hs * kChunk + lane];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(x, off, 64);
      if (lane + off < 64) x += y;
    }
    float sa = 0.f, sbias = 0.f;
    if (lane < len) {
      const int64_t t = t0 + lane;
      const float xr = g_raw[t * geo.HV + hv] + (dt_bias ? dt_bias[hv] : 0.f);
      const float ea = expf(A_log[hv]);
      const float gt = -ea * gate_softplus(xr);
      const float slope = xr > 20.f ? 1.f : 1.f / (1.f + fast_exp2(-xr * kLog2e));
      const float dgr = x * (-ea) * slope;
      dbeta[t * geo.HV + hv] = dB[lane];
      dg_raw[t * geo.HV + hv] = dgr;
      sa = x * gt;
      sbias = dgr;
    }
    sa = sum64(sa);
    sbias = sum64(sbias);
    if (lane == 0) {
      dAp[hs] = sa;
      dbp[hs] = sbias;
    }
  }
}

// ---------------------------------------------------------------------------
// dq, dk of key head h: the sum of its G value heads' terms, in head order,
// rounded to the dtype.  A pure stream (2 G fp32 reads, 2 dtype writes per
// element), so every thread takes one 4-element piece of one chunk's rows and
// issues all of its loads at once: workgroup (slot, h, p) covers pieces
// 256 p .. 256 p + 255 of the chunk's 64 x K elements / 4.
template <int K>
constexpr int qk_sum_parts() { return kChunk * K / 4 / 256; }

template <typename E, int K, bool VARLEN>
__global__ __launch_bounds__(256) void gdn_bwd_qk_sum_kernel(Geo geo, const int4* __restrict__ cmap,
                                                             const float* __restrict__ dqp,
                                                             const float* __restrict__ dkp,
                                                             E* __restrict__ dqg, E* __restrict__ dkg) {
  constexpr int PARTS = qk_sum_parts<K>();
  const int part = blockIdx.x % PARTS, rest = blockIdx.x / PARTS;
  const int slot = rest % geo.slots, h = rest / geo.slots;
  int n, len;
  int64_t t0;
  if (!chunk_of_slot<VARLEN>(geo, cmap, slot, n, t0, len)) return;
  const int e = 4 * (threadIdx.x + 256 * part);
  const int c = e / K, kk = e - c * K;
  if (c >= len) return;
  f32x4 sq = {0.f, 0.f, 0.f, 0.f}, sk = {0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < geo.G; ++r) {
    const size_t o = (((size_t)(h * geo.G + r) * geo.slots + slot) * kChunk + c) * K + kk;
    sq += *reinterpret_cast<const f32x4*>(dqp + o);
    sk += *reinterpret_cast<const f32x4*>(dkp + o);
  }
  const size_t d = ((t0 + c) * geo.H + h) * K + kk;
  st4(dqg + d, sq[0], sq[1], sq[2], sq[3]);
  st4(dkg + d, sk[0], sk[1], sk[2], sk[3]);
}

// dA_log[hv], ddt_bias[hv]: sums of the per-chunk terms over the slots in slot
// order (a fixed tree per thread count), one workgroup per value head.
__global__ __launch_bounds__(256) void gdn_bwd_param_kernel(Geo geo, const float* __restrict__ dAp,
                                                            const float* __restrict__ dbp,
                                                            float* __restrict__ dA_log,
                                                            float* __restrict__ ddt_bias) {
  __shared__ float sa[4], sb[4];
  const int hv = blockIdx.x, tid = threadIdx.x;
  float a = 0.f, b = 0.f;
  for (int s = tid; s < geo.slots; s += 256) {
    a += dAp[(size_t)hv * geo.slots + s];
    b += dbp[(size_t)hv * geo.slots + s];
  }
  a = sum64(a);
  b = sum64(b);
  if ((tid & 63) == 0) {
    sa[tid >> 6] = a;
    sb[tid >> 6] = b;
  }
  __syncthreads();
  if (tid == 0) {
    dA_log[hv] = (sa[0] + sa[1]) + (sa[2] + sa[3]);
    if (ddt_bias) ddt_bias[hv] = (sb[0] + sb[1]) + (sb[2] + sb[3]);
  }
}

}  // namespace gdn
