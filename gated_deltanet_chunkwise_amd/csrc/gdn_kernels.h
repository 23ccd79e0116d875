// gdn_kernels.h -- gfx950 kernels of the GDN chunkwise forward pass.
//
// Pipeline (one stream, no host sync):
//   chunk map  (packed sequences only)  cu_seqlens -> chunk slot table
//   WY         per (slot, hv), gate prologue first: g = -exp(A_log)
//              softplus(g_raw + dt_bias), chunk-local cumsum G (times log2 e),
//              stored with beta as [HV][slot][64] rows: stride 1 along T, the
//              relayout the G_T_CONTIG page does with a host transpose, here
//              fused into the kernel that first needs the gates.  Then
//              A = strictly_lower(beta_i k_i.k_j e^{G_i-G_j}),
//              T = (I+A)^-1, w = T diag(beta e^G) K, u = T diag(beta) V and
//              kd^T = (diag(e^{G_last-G}) K)^T.
//   chain      per (sequence, hv, 16 value columns): sequential over chunks,
//              state H (K x 16 fp32) in registers:
//                 v_new = u - w H;  H <- e^{G_last} H + kd^T v_new
//              stores the chunk-start state and v_new for the output stage.
//   output     per (slot, hv): o = scale [ diag(e^G) Q H_c + (Q K^T * causal *
//              e^{G_i-G_j}) v_new ]  (the chunk_fwd_o stage of the Ascend GDN
//              blog, with its inter-chunk q.S and intra-chunk masked QK^T terms).
//
// Intermediates are stored "fragment-major": every per-chunk tensor is laid
// out in the exact per-lane order in which its consumer feeds it to the MFMA
// (see gdn_common.h), so producer stores and consumer loads are single
// 8/16/32-byte accesses per lane, contiguous across the wave.
#pragma once
#include "gdn_common.h"

namespace gdn {

// ---------------------------------------------------------------------------
// Small vector helpers: 8 consecutive elements, loaded/stored as 16/32 bytes.
__device__ __forceinline__ void ld8(const bf16* p, float (&e)[8]) {
  bf16x8 t = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = (float)t[j];
}
__device__ __forceinline__ void ld8(const float* p, float (&e)[8]) {
  f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int j = 0; j < 4; ++j) { e[j] = a[j]; e[4 + j] = b[j]; }
}
__device__ __forceinline__ void st8(bf16* p, const float (&e)[8]) {
  bf16x8 t;
#pragma unroll
  for (int j = 0; j < 8; ++j) t[j] = (bf16)e[j];
  *reinterpret_cast<bf16x8*>(p) = t;
}
__device__ __forceinline__ void st8(float* p, const float (&e)[8]) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{e[0], e[1], e[2], e[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{e[4], e[5], e[6], e[7]};
}
__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4*>(p) = to_bf16x4(f32x4{a, b, c, d});
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Multiply element i of a k32 fragment by s[i] (in fp32, rounded back once).
__device__ __forceinline__ Frag<bf16> frag_scale(const Frag<bf16>& f, const float (&s)[8]) {
  f32x4 lo = to_f32x4(__builtin_shufflevector(f.x, f.x, 0, 1, 2, 3));
  f32x4 hi = to_f32x4(__builtin_shufflevector(f.x, f.x, 4, 5, 6, 7));
  lo *= f32x4{s[0], s[1], s[2], s[3]};
  hi *= f32x4{s[4], s[5], s[6], s[7]};
  return frag_from_tiles<bf16>(lo, hi);
}
__device__ __forceinline__ Frag<float> frag_scale(const Frag<float>& f, const float (&s)[8]) {
  return {f.lo * f32x4{s[0], s[1], s[2], s[3]}, f.hi * f32x4{s[4], s[5], s[6], s[7]}};
}

// fp32 k32 fragment -> operand dtype (one rounding).
template <typename E> __device__ __forceinline__ Frag<E> to_frag(const Frag<float>& f);
template <> __device__ __forceinline__ Frag<bf16> to_frag<bf16>(const Frag<float>& f) {
  return frag_from_tiles<bf16>(f.lo, f.hi);
}
template <> __device__ __forceinline__ Frag<float> to_frag<float>(const Frag<float>& f) { return f; }

// k offset (0..31) of fragment element i for lane group g.
__device__ __forceinline__ int kslot(int g, int i) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

// ---------------------------------------------------------------------------
// Chunk map for packed sequences (G_T_CONTIG page, "varlen checklist": int64
// offsets, chunk positions relative to each sequence start).  One workgroup.
// Offsets are clamped to [0, T] and made non-decreasing (running maximum), so
// the table never addresses outside the buffers even for malformed input;
// for valid input this is the identity.  Writes cmap[slot] = (seq, first
// token, length, 0) for used slots, (-1, 0, 0, 0) for the rest, and
// seq_slot[n] = first slot of sequence n, seq_slot[N] = slots used.
//
// It also writes seq_order, a permutation of the sequences by decreasing chunk
// count: a counting sort over min(count, kOrderBuckets - 1), so sequences of
// that many chunks or more share the first bucket, and the order inside a
// bucket is whatever the LDS atomics give (it decides only which workgroups
// start first, never a result).
constexpr int kOrderBuckets = 1024;

__device__ __forceinline__ int order_bucket(int nch) {
  return (kOrderBuckets - 1) - min(nch, kOrderBuckets - 1);
}

__global__ __launch_bounds__(256) void gdn_chunk_map_kernel(const int64_t* __restrict__ cu, int N,
                                                            int T, int slots,
                                                            int4* __restrict__ cmap,
                                                            int* __restrict__ seq_slot,
                                                            int* __restrict__ seq_order) {
  __shared__ int64_t smax[256];
  __shared__ int ssum[256];
  __shared__ int hist[kOrderBuckets];
  __shared__ int64_t carry_b;
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  if (tid == 0) {
    carry_b = min(max(cu[0], (int64_t)0), (int64_t)T);
    carry_s = 0;
  }
  __syncthreads();
  for (int base = 0; base < N; base += 256) {
    const int n = base + tid;
    smax[tid] = (n < N) ? min(max(cu[n + 1], (int64_t)0), (int64_t)T) : (int64_t)0;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      int64_t y = tid >= off ? smax[tid - off] : (int64_t)0;
      __syncthreads();
      smax[tid] = max(smax[tid], y);
      __syncthreads();
    }
    const int64_t cb = carry_b;
    const int64_t e = max(smax[tid], cb);
    const int64_t b = tid == 0 ? cb : max(smax[tid - 1], cb);
    const int len = (n < N) ? (int)(e - b) : 0;
    const int nch = (len + kChunk - 1) / kChunk;
    ssum[tid] = nch;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      int y = tid >= off ? ssum[tid - off] : 0;
      __syncthreads();
      ssum[tid] += y;
      __syncthreads();
    }
    const int s0 = carry_s + ssum[tid] - nch;
    if (n < N) {
      seq_slot[n] = min(s0, slots);
      for (int c = 0; c < nch; ++c) {
        const int s = s0 + c;
        if (s < slots) cmap[s] = make_int4(n, (int)(b + (int64_t)kChunk * c), min(kChunk, len - kChunk * c), 0);
      }
    }
    __syncthreads();
    if (tid == 255) {
      carry_b = max(smax[255], cb);
      carry_s += ssum[255];
    }
    __syncthreads();
  }
  const int used = min(carry_s, slots);
  for (int s = used + tid; s < slots; s += 256) cmap[s] = make_int4(-1, 0, 0, 0);
  if (tid == 0) seq_slot[N] = used;

  // seq_order: bucket counts, their exclusive scan (thread t owns buckets
  // 4t .. 4t+3), then each sequence placed at its bucket's next position
  constexpr int PER = kOrderBuckets / 256;
  static_assert(kOrderBuckets % 256 == 0, "buckets split evenly over the threads");
  for (int i = tid; i < kOrderBuckets; i += 256) hist[i] = 0;
  __syncthreads();  // also makes every seq_slot entry visible to the workgroup
  for (int n = tid; n < N; n += 256) atomicAdd(&hist[order_bucket(seq_slot[n + 1] - seq_slot[n])], 1);
  __syncthreads();
  int mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += hist[PER * tid + i];
  ssum[tid] = mine;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int y = tid >= off ? ssum[tid - off] : 0;
    __syncthreads();
    ssum[tid] += y;
    __syncthreads();
  }
  int run = ssum[tid] - mine;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = hist[PER * tid + i];
    hist[PER * tid + i] = run;
    run += c;
  }
  __syncthreads();
  for (int n = tid; n < N; n += 256)
    seq_order[atomicAdd(&hist[order_bucket(seq_slot[n + 1] - seq_slot[n])], 1)] = n;
}

// Transposed K / V tiles in LDS ([K or V][64] rows, chunk index along a row)
// are stored with their 4-element column groups XOR-swizzled by row / 8, which
// makes the transposed 8-byte writes of a wave (rows 8 apart) bank-conflict
// free.  Readers apply the same swizzle; groups stay 4 contiguous elements.
__device__ __forceinline__ int tswz(int row) { return 4 * ((row >> 3) & 15); }

template <typename E>
__device__ __forceinline__ Frag<E> frag_from_trow(const E* tile, int row, int stride, int col0) {
  const int g = lane_id() >> 4, sw = tswz(row);
  const E* r = tile + row * stride;
  return frag_from_pieces(r + ((col0 + 4 * g) ^ sw), r + ((col0 + 16 + 4 * g) ^ sw));
}

// ---------------------------------------------------------------------------
// WY representation.  One workgroup (8 waves) per (chunk slot, value head).
//
// LDS: K natural [64][K] (later reused for A, then for V^T) and T (fp32
// [64][64]).  K and V wait in registers as loaded; once T has been read into
// the w / u operands, V^T [V][64] takes the region of K / A and K^T [K][64]
// (bf16; fp32 at K = 128 keeps an array of its own, staged at the start) the
// region of T.  Rows past the chunk end are zero.
//
// T = (I + A)^-1 is unit lower triangular.  Its 16x16 diagonal blocks are
// found by forward substitution (one lane per column, the rows of A read from
// LDS one ahead of their use), the off-diagonal blocks block-row by block-row:
// T_rc = -T_rr sum_{m=c}^{r-1} A_rm T_mc, on fp32 MFMAs.  The scaled factors
// T diag(beta e^G) and T diag(beta) are never stored: each wave builds its
// operand fragments for w and u from its own rows of T, scaled in registers.
//
// Outputs (fragment-major, dtype E):
//   wf  [hv][slot][ct<4][kb<K/32][lane]   A operand of  w H        (rows c, k over K)
//   ktf [hv][slot][mt<K/16][cb<2][lane]   A operand of  kd^T v_new (rows K, k over c)
//   uf  [hv][slot][vt<V/16][cp<2][lane][2] D tiles ct = 2cp, 2cp+1 of u (rows c, column v);
//                                         a lane's pair is one fragment-sized block
// Eight waves per WY workgroup.
constexpr int kWyThreads = 512;

// With STORE_T, T itself (lower triangular, in the call's dtype, [hv][slot][64][64]
// row-major, zeros above the diagonal) is also written to tmat, for the backward pass.
//
// With EMIT_P the workgroup also forms the chunk's intra-chunk output matrix
// P^T = (K Q^T) * [j <= i] * e^{G_i - G_j} (rows j: keys, columns i: queries;
// diagonal included), the intra-chunk term of the output stage, and stores it
// for the fused state-and-output pass as the B operands of v_new^T P^T:
//   pf [hv][slot][it<4][jb<2][lane]   k32 fragment over key rows 32jb.., query
//                                     column 16it + lane%16 (written for
//                                     jb <= it/2 only; the rest is all zero)
// Q is staged in the LDS of T, which is free until the diagonal blocks of T
// are solved.
// Eight consecutive elements of one row as loaded (16 bytes for bf16), and
// column j of four such rows stored as four consecutive elements.
template <typename E> struct Raw8;
template <> struct Raw8<bf16> {
  bf16x8 x;
  __device__ __forceinline__ void load(const bf16* p) { x = *reinterpret_cast<const bf16x8*>(p); }
  __device__ __forceinline__ void zero() { x = bf16x8{}; }
  __device__ __forceinline__ void store(bf16* p) const { *reinterpret_cast<bf16x8*>(p) = x; }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const f32x4*>(p)[0];
    b = reinterpret_cast<const f32x4*>(p)[1];
  }
  __device__ __forceinline__ void zero() { a = b = f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void store(float* p) const {
    reinterpret_cast<f32x4*>(p)[0] = a;
    reinterpret_cast<f32x4*>(p)[1] = b;
  }
};
__device__ __forceinline__ void raw_column(const Raw8<bf16> (&e)[4], int j, bf16* p) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{e[0].x[j], e[1].x[j], e[2].x[j], e[3].x[j]};
}
__device__ __forceinline__ void raw_column(const Raw8<float> (&e)[4], int j, float* p) {
  auto el = [&](int r) { return j < 4 ? e[r].a[j] : e[r].b[j - 4]; };
  *reinterpret_cast<f32x4*>(p) = f32x4{el(0), el(1), el(2), el(3)};
}

template <typename E, int K>
constexpr bool wy_q_fits() {
  return kChunk * (K + 16 / (int)sizeof(E)) * (int)sizeof(E) <= kChunk * (kChunk + 4) * 4;
}

// SPLIT (with EMIT_P, for grids that run in one round at two workgroups per
// CU): K and Q natural get LDS of their own (71 KB in all at K = V = 128), so
// that Q's loads go out after the first barrier, while K K^T is formed, and
// waves 4-7 form P^T while waves 0-3 solve the diagonal blocks of T, instead
// of both lengthening the phases before.
template <typename E, int K, int V, bool VARLEN, bool STORE_T = false, bool EMIT_P = false,
          bool SPLIT = false>
__global__ __launch_bounds__(kWyThreads) void gdn_wy_kernel(Geo geo, const E* __restrict__ kg,
                                                     const E* __restrict__ vg,
                                                     const float* __restrict__ g_raw,
                                                     const float* __restrict__ beta,
                                                     const float* __restrict__ A_log,
                                                     const float* __restrict__ dt_bias,
                                                     const int4* __restrict__ cmap,
                                                     float* __restrict__ gam,
                                                     float* __restrict__ bet,
                                                     Frag<E>* __restrict__ wf,
                                                     Frag<E>* __restrict__ ktf,
                                                     Quad<E>* __restrict__ uf,
                                                     E* __restrict__ tmat,
                                                     const E* __restrict__ qg,
                                                     Frag<E>* __restrict__ pf) {
  static_assert(!EMIT_P || wy_q_fits<E, K>(), "Q rows must fit the LDS of T");
  static_assert(!SPLIT || EMIT_P, "the split only moves the P^T work");
  constexpr int P = 16 / sizeof(E);  // 16 bytes of row padding
  constexpr int KS = K + P;          // K natural row stride
  constexpr int CSK = kChunk + 4;    // K^T row stride
  constexpr int CSV = kChunk + P;    // V^T row stride
  constexpr int FS = kChunk + 4;     // A, T row stride (fp32)
  // Region 0 holds K natural until the products of A are formed, then A
  // until T is formed, then V^T (bf16 at K = V = 128: 36.4 KB in all).
  constexpr int R0A = kChunk * KS * (int)sizeof(E), R0C = kChunk * FS * 4;
  constexpr int R0V = V * CSV * (int)sizeof(E);
  constexpr int R0 = R0A > R0C ? (R0A > R0V ? R0A : R0V) : (R0C > R0V ? R0C : R0V);
  __shared__ __align__(16) char r0[R0];
  // K^T too is staged late when it fits the LDS of T (bf16): T has then been
  // read into the w / u operands
  constexpr bool KT_LATE = K * CSK * (int)sizeof(E) <= kChunk * FS * 4;
  __shared__ __align__(16) E Kt_sep[KT_LATE ? 8 : K * CSK];
  __shared__ __align__(16) float Ts[kChunk * FS];
  E* const Kt = KT_LATE ? reinterpret_cast<E*>(Ts) : Kt_sep;
  __shared__ float sg[kChunk], sb[kChunk];
  __shared__ __align__(16) E KQ_sep[SPLIT ? 2 * kChunk * KS : 8];  // SPLIT: K, Q natural
  E* const Ks = SPLIT ? KQ_sep : reinterpret_cast<E*>(r0);
  E* const Vt = reinterpret_cast<E*>(r0);  // V^T, once T is formed
  float* const As = reinterpret_cast<float*>(r0);
  // EMIT_P: Q natural [64][KS], until T is formed (SPLIT: for the whole kernel)
  E* const Qs = SPLIT ? KQ_sep + kChunk * KS : reinterpret_cast<E*>(Ts);

  int hv, slot;
  xcd_slot_block(blockIdx.x, geo.H, geo.G, geo.slots, hv, slot);
  // Blocks in descending chunk order (fixed length: every sequence's last
  // chunk first; packed: the slots reversed), so the first chunks, which the
  // state pass reads first, are the most recently written when it starts
  // (still in the last-level cache when a step's intermediates exceed it).
  if constexpr (!VARLEN) {
    const int c = geo.NT - 1 - slot / geo.N, n = slot % geo.N;
    slot = n * geo.NT + c;
  } else {
    slot = geo.slots - 1 - slot;
  }
  int n, len;
  int64_t t0;
  if (!chunk_of_slot<VARLEN>(geo, cmap, slot, n, t0, len)) return;
  const int h = hv / geo.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, lc = lane & 15;
  const size_t hs = (size_t)hv * geo.slots + slot;

  // All global loads first (one memory latency for K, V and the gate inputs):
  // thread t < 256 owns the 4x8 micro-tile t of K, thread 256 + t that of V;
  // wave 0 also reads this head's 64 raw gates and betas (stride HV along T).
  float graw = 0.f, braw = 0.f;
  if (wave == 0 && lane < len) {
    graw = g_raw[(t0 + lane) * geo.HV + hv];
    braw = beta[(t0 + lane) * geo.HV + hv];
  }
  constexpr int NKM = 16 * (K / 8), NVM = 16 * (V / 8);  // micro-tiles (<= 256 each)
  const bool kside = tid < 256;
  const int mtile = tid & 255, W8 = (kside ? K : V) / 8;
  const int rb = 4 * (mtile / W8), c0 = 8 * (mtile % W8);
  const bool owns = mtile < (kside ? NKM : NVM);
  // the micro-tile as loaded (raw elements: few registers while it waits)
  Raw8<E> e[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (owns && rb + r < len) {
      if (kside) e[r].load(kg + ((t0 + rb + r) * geo.H + h) * K + c0);
      else e[r].load(vg + ((t0 + rb + r) * geo.HV + hv) * V + c0);
    } else {
      e[r].zero();
    }
  }
  // EMIT_P: thread t also loads 8-element pieces t and t + 512 of Q's rows
  // (SPLIT: after the first barrier).
  constexpr int NQP = EMIT_P ? (kChunk * (K / 8) + kWyThreads - 1) / kWyThreads : 0;
  Raw8<E> eq[NQP > 0 ? NQP : 1];  // as loaded
  auto load_q = [&]() {
#pragma unroll
    for (int it = 0; it < NQP; ++it) {
      const int m = tid + kWyThreads * it, row = m / (K / 8), qc = 8 * (m % (K / 8));
      if (row < kChunk && row < len) eq[it].load(qg + ((t0 + row) * geo.H + h) * K + qc);
      else eq[it].zero();
    }
  };
  auto stage_q = [&]() {
#pragma unroll
    for (int it = 0; it < NQP; ++it) {
      const int m = tid + kWyThreads * it, row = m / (K / 8), qc = 8 * (m % (K / 8));
      if (row < kChunk) eq[it].store(Qs + row * KS + qc);
    }
  };
  if constexpr (!SPLIT) load_q();
  if (owns && kside) {
#pragma unroll
    for (int r = 0; r < 4; ++r) e[r].store(Ks + (rb + r) * KS + c0);
    if constexpr (!KT_LATE) {
#pragma unroll
      for (int j = 0; j < 8; ++j) raw_column(e, j, Kt + (c0 + j) * CSK + (rb ^ tswz(c0 + j)));
    }
  }
  if constexpr (!SPLIT) stage_q();
  // Gate prologue (wave 0, lane = token): g in fp32 with the softplus
  // threshold of the KDA gate guide ("core computation logic"), the chunk-local
  // scan, and this head's stride-1 rows of the cumulative gate (times log2 e)
  // and beta for the state pass and the output.  Past the chunk end g = 0 (the
  // cumulative gate stays at its last value) and beta = 0.
  if (wave == 0) {
    float gv = 0.f;
    if (lane < len) {
      const float x = graw + (dt_bias ? dt_bias[hv] : 0.f);
      gv = -expf(A_log[hv]) * gate_softplus(x);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(gv, off, 64);
      if (lane >= off) gv += y;
    }
    gv *= kLog2e;
    sg[lane] = gv;
    sb[lane] = braw;
    gam[hs * kChunk + lane] = gv;
    bet[hs * kChunk + lane] = braw;
  }
  __syncthreads();
  if constexpr (SPLIT) load_q();  // in flight while K K^T is formed

  // EMIT_P: P^T fragment job j (0..5): query tile it, key rows 32jb..32jb+31
  // (key tiles 2jb, 2jb+1; a key tile past it is 0).  p_products forms it
  // from K and Q natural; p_store masks and decays it (sg) and stores it.
  auto p_tile = [](int j, int& pit, int& pjb) {
    pit = j < 1 ? 0 : j < 2 ? 1 : j < 4 ? 2 : 3;
    pjb = (j == 3 || j == 5) ? 1 : 0;
  };
  auto p_products = [&](int j, f32x4 (&pt)[2]) {
    int pit, pjb;
    p_tile(j, pit, pjb);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int jt = 2 * pjb + q;
      pt[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (jt <= pit) {
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb)
          mma_k32(pt[q], frag_from_row(Ks + (16 * jt + lc) * KS + 32 * kb),
                  frag_from_row(Qs + (16 * pit + lc) * KS + 32 * kb));
      }
    }
  };
  auto p_store = [&](int j, f32x4 (&pt)[2]) {
    int pit, pjb;
    p_tile(j, pit, pjb);
    const int i = 16 * pit + lc;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = 16 * (2 * pjb + q) + 4 * g + r;
        pt[q][r] = jj <= i ? pt[q][r] * fast_exp2(sg[i] - sg[jj]) : 0.f;
      }
    }
    pf[((hs * 4 + pit) * 2 + pjb) * 64 + lane] = frag_from_tiles<E>(pt[0], pt[1]);
  };

  // A = strictly_lower(beta_i (K K^T)_ij exp(G_i - G_j)).  The 10 tiles on or
  // below the diagonal go 2/2/1/1/1/1/1/1 to the waves; the products finish
  // before A overwrites K natural in region 0.
  {
    f32x4 acc[2];
    int ti[2], tj[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int t = wave + 8 * q;  // tile index in (0,0),(1,0),(1,1),(2,0),...
      const int it = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
      ti[q] = it;
      tj[q] = t - it * (it + 1) / 2;
      acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < 10) {
#pragma unroll
        for (int kb = 0; kb < K / 32; ++kb)
          mma_k32(acc[q], frag_from_row(Ks + (16 * ti[q] + lc) * KS + 32 * kb),
                  frag_from_row(Ks + (16 * tj[q] + lc) * KS + 32 * kb));
      }
    }
    // EMIT_P without SPLIT: fragment job j = wave - 2 (waves 2..7) of P^T
    // (p_products / p_store below), formed here next to K K^T.
    f32x4 pt[2];
    if constexpr (EMIT_P && !SPLIT) {
      if (wave >= 2) p_products(wave - 2, pt);
    }
    __syncthreads();
    if constexpr (EMIT_P && !SPLIT) {
      if (wave >= 2) p_store(wave - 2, pt);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (wave + 8 * q < 10) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * ti[q] + 4 * g + r, col = 16 * tj[q] + lc;
          As[row * FS + col] = col < row ? sb[row] * acc[q][r] * fast_exp2(sg[row] - sg[col]) : 0.f;
        }
      }
    }
  }
  if constexpr (SPLIT) stage_q();
  __syncthreads();

  // Diagonal blocks of T by forward substitution, lane j solving column j of
  // the block: row i of T_bb is e_i - sum_{m<i} A_bb[i][m] T_bb[m], with
  // A_bb's rows read from LDS (the same address in every lane: broadcast),
  // a row ahead of its use, so that few registers are live.  The blocks
  // above the diagonal are never written: T is lower triangular, and the
  // reads below take those blocks as zero.
  {
    const int b = wave;
    if constexpr (SPLIT) {
      // waves 4-7: the P^T jobs (4, 5 two each; 6, 7 one each)
      if (b >= 4) {
        f32x4 pt[2];
        p_products(b - 4, pt);
        p_store(b - 4, pt);
        if (b < 6) {
          p_products(b, pt);
          p_store(b, pt);
        }
      }
    }
    if (b < 4 && lane < 16) {
      const float* ab = As + 16 * b * FS + 16 * b;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == lane) ? 1.f : 0.f;
      f32x4 nxt[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) nxt[q] = reinterpret_cast<const f32x4*>(ab + FS)[q];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        f32x4 row[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) row[q] = nxt[q];
        if (i + 1 < 16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) nxt[q] = reinterpret_cast<const f32x4*>(ab + (i + 1) * FS)[q];
        }
        // A_bb[i][m] for m >= i is zero (strictly lower), so the later x[m]
        // (still e_j's entries) add nothing
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int m = 0; m < 16; m += 2) {
          if (m < i) s0 += row[m >> 2][m & 3] * x[m];
          if (m + 1 < i) s1 += row[(m + 1) >> 2][(m + 1) & 3] * x[m + 1];
        }
        x[i] -= s0 + s1;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) Ts[(16 * b + i) * FS + 16 * b + lane] = x[i];
    }
  }
  __syncthreads();

  // Off-diagonal blocks, one block row at a time.
  for (int r = 1; r < 4; ++r) {
    if (wave < r) {
      const int c = wave;
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
      for (int m = c; m < r; ++m)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          X = mfma_f32_4(As[(16 * r + lc) * FS + 16 * m + 4 * ks + g],
                         Ts[(16 * m + 4 * ks + g) * FS + 16 * c + lc], X);
      // Y = T_rr X, with X's D tile used directly as the B operand:
      // MFMA q reduces over k = 4*g + q for lane group g.
      f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) Y = mfma_f32_4(Ts[(16 * r + lc) * FS + 16 * r + 4 * g + q], X[q], Y);
#pragma unroll
      for (int q = 0; q < 4; ++q) Ts[(16 * r + 4 * g + q) * FS + 16 * c + lc] = -Y[q];
    }
    __syncthreads();
  }

  if constexpr (STORE_T) {
#pragma unroll
    for (int it = 0; it < kChunk * kChunk / 4 / kWyThreads; ++it) {
      const int e4 = tid + kWyThreads * it, i = e4 >> 4, j = (e4 & 15) << 2;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      // blocks right of the diagonal block were never written
      const f32x4 x = (j >> 4) <= (i >> 4) ? *reinterpret_cast<const f32x4*>(Ts + i * FS + j) : zero;
      *reinterpret_cast<Quad<E>*>(tmat + hs * kChunk * kChunk + i * kChunk + j) = make_quad<E>(x);
    }
  }

  // Waves w and w + 4 own chunk rows 16w..16w+15 (w < 4), each half of the
  // output tiles.  Their k32 fragments of T diag(beta e^G) and T diag(beta)
  // over the chunk index (row 16w + lane%16, columns 32cb + kslot(g, i)) are
  // formed from T in registers.
  // wave-uniform (scalar) values, so the zero-block test below is a scalar branch
  const int ct = __builtin_amdgcn_readfirstlane(wave & 3), half = __builtin_amdgcn_readfirstlane(wave >> 2);
  Frag<E> bw[2], bu[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    // Columns 32cb..32cb+15 (lo) and 32cb+16..32cb+31 (hi) lie in the 16-wide
    // column blocks 2cb and 2cb+1; a block right of the diagonal block ct is 0.
    const float* trow = Ts + (16 * ct + lc) * FS + 32 * cb;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 lo = 2 * cb <= ct ? *reinterpret_cast<const f32x4*>(trow + 4 * g) : zero;
    const f32x4 hi = 2 * cb + 1 <= ct ? *reinterpret_cast<const f32x4*>(trow + 16 + 4 * g) : zero;
    float sw[8], su[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 32 * cb + kslot(g, i);
      su[i] = sb[j];
      sw[i] = sb[j] * fast_exp2(sg[j]);
    }
    const Frag<float> tf = {lo, hi};
    bw[cb] = to_frag<E>(frag_scale(tf, sw));
    bu[cb] = to_frag<E>(frag_scale(tf, su));
  }

  // T has been read (w / u operands in registers): V^T takes region 0 (A is
  // no longer read either), K^T the LDS of T
  __syncthreads();
  if (owns && (!kside || KT_LATE)) {
    E* const tr = kside ? Kt : Vt;
    const int cs = kside ? CSK : CSV;
#pragma unroll
    for (int j = 0; j < 8; ++j) raw_column(e, j, tr + (c0 + j) * cs + (rb ^ tswz(c0 + j)));
  }
  __syncthreads();

  // w^T = K^T T_w^T: D tile (mt) holds w[16ct + lane%16][16mt + 4g + r], so
  // tile pairs are the state pass's A fragments.
  {
    constexpr int MTH = K / 32;  // row tiles of w^T per half
    f32x4 acc[MTH];
#pragma unroll
    for (int m = 0; m < MTH; ++m) {
      const int mt = half * MTH + m;
      acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      // T's column block cb is zero for the rows of tile ct < 2cb (right of
      // the diagonal block): that product is skipped, not multiplied by zero
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        if (2 * cb <= ct) mma_k32(acc[m], frag_from_trow(Kt, 16 * mt + lc, CSK, 32 * cb), bw[cb]);
    }
    Frag<E>* dst = wf + (hs * 4 + ct) * (K / 32) * 64;
#pragma unroll
    for (int b2 = 0; b2 < MTH / 2; ++b2)
      dst[(half * (MTH / 2) + b2) * 64 + lane] = frag_from_tiles<E>(acc[2 * b2], acc[2 * b2 + 1]);
  }
  // u = T_u V (A operand: this wave's rows of T_u; each half takes half of
  // the value tiles).
  {
    Quad<E>* dst = uf + hs * (V / 16) * 4 * 64;
#pragma unroll
    for (int m = 0; m < V / 32; ++m) {
      const int vt = half * (V / 32) + m;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        if (2 * cb <= ct) mma_k32(acc, bu[cb], frag_from_trow(Vt, 16 * vt + lc, CSV, 32 * cb));
      dst[((vt * 2 + (ct >> 1)) * 64 + lane) * 2 + (ct & 1)] = make_quad<E>(acc);
    }
  }
  // kd^T = (diag(e^{G_last - G}) K)^T as A fragments over the chunk index.
  {
    Frag<E>* dst = ktf + hs * (K / 16) * 2 * 64;
    const float gl = sg[kChunk - 1];
    for (int f = wave; f < (K / 16) * 2; f += kWyThreads / 64) {
      const int mt = f >> 1, cb = f & 1;
      float sc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sc[i] = fast_exp2(gl - sg[32 * cb + kslot(g, i)]);
      dst[f * 64 + lane] = frag_scale(frag_from_trow(Kt, 16 * mt + lc, CSK, 32 * cb), sc);
    }
  }
}

// ---------------------------------------------------------------------------
// Inter-chunk state pass.  One wave per (sequence, value head, 16 value
// columns); the K x 16 fp32 state lives in registers as K/16 D tiles
// (rows k, column v).  Per chunk, in order:
//   store H_c (the chunk-start state) for the output stage,
//   v_new = u - w H_c            (B operand: the state tiles, paired),
//   store v_new,
//   H <- e^{G_last} H + kd^T v_new (B operand: the v_new tiles, paired).
// A chunk's operands (w and kd^T fragments, the u tiles, e^{G_last}) are
// loaded in one batch, one chunk ahead of their use (two register buffers), so
// the loads of chunk c+1 are in flight while chunk c computes.
// Outputs (fragment-major, dtype E):
//   hcf [hv][slot][vt][kb<K/32][lane]  A operand of H_c^T q^T (rows v, k over K)
//   vnf [hv][slot][vt][cb<2][lane]     A operand of v_new^T P^T (rows v, k over c)
// State-pass modes.  CHAIN_FULL: the pass as described, storing H_c and v_new.
// CHAIN_END: the same arithmetic without those stores (only the end state is
// kept).  CHAIN_MAP: u taken as 0 and no stores; started from the identity
// (with V = K), the end state is the chunks' composed linear map M.
// CHAIN_PLAIN: the CHAIN_FULL arithmetic, storing H_c and v_new transposed in
// row-major layouts of the call's dtype instead (hcf, vnf then point at arrays
// [hv][slot][V][K] = H_c^T and [hv][slot][V][64] = v_new^T); the backward pass
// reads them.
enum { CHAIN_FULL = 0, CHAIN_END = 1, CHAIN_MAP = 2, CHAIN_PLAIN = 3 };

template <typename E, int K, int V, int MODE = CHAIN_FULL>
struct ChainStep {
  static constexpr int KB = K / 32, KT = K / 16, NV = V / 16;
  Frag<E> w[4][KB];
  Frag<E> kt[KT][2];
  Quad<E> u[4];
  float gl;  // lane l: entry l of the chunk's (log2-scaled) cumulative gate row

  __device__ __forceinline__ void load(const Frag<E>* __restrict__ wf,
                                       const Frag<E>* __restrict__ ktf,
                                       const Quad<E>* __restrict__ uf,
                                       const float* __restrict__ gam, size_t hs, int vt,
                                       int lane) {
    // Every lane loads one entry of the chunk's gate row (a vector load, issued
    // first so it is the oldest of the batch; a scalar load would make every
    // later LDS or scalar wait a full drain).  Lane 63 holds the last value.
    gl = gam[hs * kChunk + lane];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) w[ct][kb] = wf[((hs * 4 + ct) * KB + kb) * 64 + lane];
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) kt[mt][cb] = ktf[((hs * KT + mt) * 2 + cb) * 64 + lane];
    if constexpr (MODE == CHAIN_MAP) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) u[ct] = make_quad<E>(f32x4{0.f, 0.f, 0.f, 0.f});
    } else {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) u[ct] = uf[(((hs * NV + vt) * 2 + (ct >> 1)) * 64 + lane) * 2 + (ct & 1)];
    }
  }

  // First half of a chunk: emits H_c (the state on entry) and v_new = u - w H_c
  // through the sinks put_hc(kb, fragment) / put_vn(cb, fragment), and returns
  // v_new as the two B fragments of the state update.  Uses w and u.
  template <typename PutH, typename PutV, typename PutVF>
  __device__ __forceinline__ void vnew(const f32x4 (&Hs)[KT], Frag<E> (&vb)[2], PutH&& put_hc,
                                       PutV&& put_vn, PutVF&& put_vf) const {
    Frag<E> hb[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      hb[kb] = frag_from_tiles<E>(Hs[2 * kb], Hs[2 * kb + 1]);
      put_hc(kb, hb[kb]);
    }
    // by pairs of row tiles, so the first pair's conversion can overlap the
    // second pair's products
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        mma_k32(p0, w[2 * cb][kb], hb[kb]);
        mma_k32(p1, w[2 * cb + 1][kb], hb[kb]);
      }
      const f32x4 d0 = quad_f32(u[2 * cb]) - p0, d1 = quad_f32(u[2 * cb + 1]) - p1;
      vb[cb] = frag_from_tiles<E>(d0, d1);
      put_vn(cb, vb[cb]);
      put_vf(cb, d0, d1);
    }
  }

  // vnew with H_c and v_new stored straight to their fragment-major arrays
  // (CHAIN_FULL), in plain layouts (CHAIN_PLAIN), or not stored at all
  // (the other modes).
  __device__ __forceinline__ void vnew_global(const f32x4 (&Hs)[KT], Frag<E> (&vb)[2],
                                              Frag<E>* __restrict__ hcf, Frag<E>* __restrict__ vnf,
                                              size_t hs, int vt, int lane) const {
    auto none_f = [](int, const Frag<E>&) {};
    auto none_t = [](int, const f32x4&, const f32x4&) {};
    if constexpr (MODE == CHAIN_FULL) {
      Frag<E>* hc = hcf + (hs * NV + vt) * KB * 64 + lane;
      Frag<E>* vn = vnf + (hs * NV + vt) * 2 * 64 + lane;
      vnew(Hs, vb, [&](int kb, const Frag<E>& f) { hc[kb * 64] = f; },
           [&](int cb, const Frag<E>& f) { vn[cb * 64] = f; }, none_t);
    } else if constexpr (MODE == CHAIN_PLAIN) {
      // D tile element r of lane (lc, g) is row 4g + r of the tile, column lc:
      // four consecutive elements of row v of the transposed layouts.
      const int g = lane >> 4, v = 16 * vt + (lane & 15);
      Quad<E>* hp = reinterpret_cast<Quad<E>*>(reinterpret_cast<E*>(hcf) + hs * K * V + (size_t)v * K + 4 * g);
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) hp[4 * mt] = make_quad<E>(Hs[mt]);
      Quad<E>* vp = reinterpret_cast<Quad<E>*>(reinterpret_cast<E*>(vnf) + hs * kChunk * V + (size_t)v * kChunk + 4 * g);
      vnew(Hs, vb, none_f, none_f, [&](int cb, const f32x4& d0, const f32x4& d1) {
        vp[8 * cb] = make_quad<E>(d0);
        vp[8 * cb + 4] = make_quad<E>(d1);
      });
    } else {
      vnew(Hs, vb, none_f, none_f, none_t);
    }
  }

  // Second half: H += kd^T v_new, on a state already multiplied by e^{G_last}.
  // Uses kt.
  __device__ __forceinline__ void update(f32x4 (&Hs)[KT], const Frag<E> (&vb)[2]) const {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) mma_k32(Hs[mt], kt[mt][cb], vb[cb]);
  }

  // One chunk: consumes this step's operands, updates Hs, writes H_c and v_new.
  __device__ __forceinline__ void compute(f32x4 (&Hs)[KT], Frag<E>* __restrict__ hcf,
                                          Frag<E>* __restrict__ vnf, size_t hs, int vt,
                                          int lane) const {
    Frag<E> vb[2];
    vnew_global(Hs, vb, hcf, vnf, hs, vt, lane);
    // gl holds the chunk's gate row, one entry per lane; the decay uses the last.
    const float dec = fast_exp2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), kChunk - 1)));
#pragma unroll
    for (int mt = 0; mt < KT; ++mt) Hs[mt] *= dec;
    update(Hs, vb);
  }
};

// Initial state tiles (rows 16*mt + 4g + r, column v) from h0, or zero.
template <int K, int V>
__device__ __forceinline__ void load_state(f32x4 (&Hs)[K / 16], const float* __restrict__ h0,
                                           size_t sbase, int v, int g) {
  if (h0) {
#pragma unroll
    for (int mt = 0; mt < K / 16; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Hs[mt][r] = h0[sbase + (size_t)(16 * mt + 4 * g + r) * V + v];
  } else {
#pragma unroll
    for (int mt = 0; mt < K / 16; ++mt) Hs[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Initial state tiles (rows 16*mt + 4g + r, column v): the identity for
// CHAIN_MAP (V = K), else from h0, or zero.
template <int K, int V, int MODE>
__device__ __forceinline__ void init_state(f32x4 (&Hs)[K / 16], const float* __restrict__ h0,
                                           size_t sbase, int v, int g) {
  if constexpr (MODE == CHAIN_MAP) {
    static_assert(K == V, "the map is K x K");
#pragma unroll
    for (int mt = 0; mt < K / 16; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Hs[mt][r] = (16 * mt + 4 * g + r == v) ? 1.f : 0.f;
  } else {
    load_state<K, V>(Hs, h0, sbase, v, g);
  }
}

template <typename E, int K, int V, bool VARLEN, int MODE = CHAIN_FULL>
__global__ __launch_bounds__(64) void gdn_chain_kernel(Geo geo, const Frag<E>* __restrict__ wf,
                                                       const Frag<E>* __restrict__ ktf,
                                                       const Quad<E>* __restrict__ uf,
                                                       const float* __restrict__ gam,
                                                       const int* __restrict__ seq_slot,
                                                       const float* __restrict__ h0,
                                                       float* __restrict__ fin,
                                                       Frag<E>* __restrict__ hcf,
                                                       Frag<E>* __restrict__ vnf) {
  using Step = ChainStep<E, K, V, MODE>;
  constexpr int NV = V / 16, KT = K / 16;
  // Two register buffers when a step's operands fit in ~150 VGPRs.
  constexpr bool kDouble = sizeof(Step) <= 600;
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
  const int lane = lane_id(), g = lane >> 4, lc = lane & 15;
  const int v = 16 * vt + lc;
  const size_t sbase = ((size_t)n * geo.HV + hv) * K * V;
  const size_t hbase = (size_t)hv * geo.slots;

  f32x4 Hs[KT];
  init_state<K, V, MODE>(Hs, h0, sbase, v, g);

  if constexpr (kDouble) {
    // The next chunk's loads are issued unconditionally (the last chunk reloads
    // itself, in bounds), so the compiler's wait counts stay exact across the
    // loop instead of falling back to full drains at the join.
    Step A, B;
    const int last = s1 - 1;
    // The empty asm statements keep the compiler from sinking a prefetch batch
    // below the compute that should overlap it.
    if (s0 < s1) A.load(wf, ktf, uf, gam, hbase + s0, vt, lane);
    for (int s = s0; s < s1; s += 2) {
      B.load(wf, ktf, uf, gam, hbase + min(s + 1, last), vt, lane);
      asm volatile("" ::: "memory");
      A.compute(Hs, hcf, vnf, hbase + s, vt, lane);
      if (s + 1 >= s1) break;
      A.load(wf, ktf, uf, gam, hbase + min(s + 2, last), vt, lane);
      asm volatile("" ::: "memory");
      B.compute(Hs, hcf, vnf, hbase + s + 1, vt, lane);
    }
  } else {
    Step A;
    for (int s = s0; s < s1; ++s) {
      A.load(wf, ktf, uf, gam, hbase + s, vt, lane);
      A.compute(Hs, hcf, vnf, hbase + s, vt, lane);
    }
  }
  if (fin) {
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) fin[sbase + (size_t)(16 * mt + 4 * g + r) * V + v] = Hs[mt][r];
  }
}

// ---------------------------------------------------------------------------
// State pass, register variant with two value tiles per wave (bf16, CHAIN_FULL):
// one wave per (sequence, value head, 32 value columns).  The chunk's w and
// kd^T fragments are loaded once for both tiles (34 KB per chunk per wave, as
// for one tile), which halves the operand stream per value column of the
// one-tile register variant; used when the units are too many for the ring
// variant's workgroups to be resident at once.  The next chunk's operands are
// loaded one chunk ahead (two register sets).
template <typename E, int K, int V>
struct ChainStep2 {
  static constexpr int KB = K / 32, KT = K / 16, NV = V / 16;
  Frag<E> w[4][KB];
  Frag<E> kt[KT][2];
  Quad<E> u[2][4];
  float gl;  // lane l: entry l of the chunk's (log2-scaled) cumulative gate row

  __device__ __forceinline__ void load(const Frag<E>* __restrict__ wf,
                                       const Frag<E>* __restrict__ ktf,
                                       const Quad<E>* __restrict__ uf,
                                       const float* __restrict__ gam, size_t hs, int vt0,
                                       int lane) {
    gl = gam[hs * kChunk + lane];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) w[ct][kb] = wf[((hs * 4 + ct) * KB + kb) * 64 + lane];
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) kt[mt][cb] = ktf[((hs * KT + mt) * 2 + cb) * 64 + lane];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        u[t][ct] = uf[(((hs * NV + vt0 + t) * 2 + (ct >> 1)) * 64 + lane) * 2 + (ct & 1)];
  }

  // One chunk for both tiles: store H_c and v_new, then
  // H <- e^{G_last} H + kd^T v_new.
  __device__ __forceinline__ void compute(f32x4 (&Hs)[2][KT], Frag<E>* __restrict__ hcf,
                                          Frag<E>* __restrict__ vnf, size_t hs, int vt0,
                                          int lane) const {
    Frag<E> vb[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      Frag<E> hb[KB];
      Frag<E>* hc = hcf + (hs * NV + vt0 + t) * KB * 64 + lane;
      Frag<E>* vn = vnf + (hs * NV + vt0 + t) * 2 * 64 + lane;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        hb[kb] = frag_from_tiles<E>(Hs[t][2 * kb], Hs[t][2 * kb + 1]);
        hc[kb * 64] = hb[kb];
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          mma_k32(p0, w[2 * cb][kb], hb[kb]);
          mma_k32(p1, w[2 * cb + 1][kb], hb[kb]);
        }
        vb[t][cb] = frag_from_tiles<E>(quad_f32(u[t][2 * cb]) - p0, quad_f32(u[t][2 * cb + 1]) - p1);
        vn[cb * 64] = vb[t][cb];
      }
    }
    const float dec = fast_exp2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), kChunk - 1)));
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) Hs[t][mt] *= dec;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int t = 0; t < 2; ++t) mma_k32(Hs[t][mt], kt[mt][cb], vb[t][cb]);
  }
};

template <typename E, int K, int V, bool VARLEN>
__global__ __launch_bounds__(64) void gdn_chain2_kernel(Geo geo, const Frag<E>* __restrict__ wf,
                                                        const Frag<E>* __restrict__ ktf,
                                                        const Quad<E>* __restrict__ uf,
                                                        const float* __restrict__ gam,
                                                        const int* __restrict__ seq_slot,
                                                        const float* __restrict__ h0,
                                                        float* __restrict__ fin,
                                                        Frag<E>* __restrict__ hcf,
                                                        Frag<E>* __restrict__ vnf) {
  using Step = ChainStep2<E, K, V>;
  constexpr int NV = V / 16, KT = K / 16, NP = NV / 2;
  int hv, rest;
  head_major_block(blockIdx.x, geo.HV, geo.N * NP, hv, rest);
  const int n = rest / NP, vt0 = 2 * (rest - n * NP);
  int s0, s1;
  if constexpr (VARLEN) {
    s0 = seq_slot[n];
    s1 = seq_slot[n + 1];
  } else {
    s0 = n * geo.NT;
    s1 = s0 + geo.NT;
  }
  const int lane = lane_id(), g = lane >> 4, lc = lane & 15;
  const size_t sbase = ((size_t)n * geo.HV + hv) * K * V;
  const size_t hbase = (size_t)hv * geo.slots;
  f32x4 Hs[2][KT];
#pragma unroll
  for (int t = 0; t < 2; ++t) load_state<K, V>(Hs[t], h0, sbase, 16 * (vt0 + t) + lc, g);
  // The next chunk's loads are issued unconditionally (the last chunk reloads
  // itself, in bounds), so the compiler's wait counts stay exact across the loop.
  Step A, B;
  const int last = s1 - 1;
  if (s0 < s1) A.load(wf, ktf, uf, gam, hbase + s0, vt0, lane);
  for (int s = s0; s < s1; s += 2) {
    B.load(wf, ktf, uf, gam, hbase + min(s + 1, last), vt0, lane);
    asm volatile("" ::: "memory");
    A.compute(Hs, hcf, vnf, hbase + s, vt0, lane);
    if (s + 1 >= s1) break;
    A.load(wf, ktf, uf, gam, hbase + min(s + 2, last), vt0, lane);
    asm volatile("" ::: "memory");
    B.compute(Hs, hcf, vnf, hbase + s + 1, vt0, lane);
  }
  if (fin) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          fin[sbase + (size_t)(16 * mt + 4 * g + r) * V + 16 * (vt0 + t) + lc] = Hs[t][mt][r];
  }
}

// ---------------------------------------------------------------------------
// State pass, LDS-ring variant (used when its workgroups fit one per CU).
// Same arithmetic as gdn_chain_kernel; only the operand supply differs.  A
// workgroup is:
//   NC compute waves  -- NC 16-column tiles of one (sequence, value head); each
//                        stores its H_c and v_new fragments itself (staging
//                        them through LDS for another wave to store measured
//                        slower: the LDS traffic costs more than the stores);
//   two loader waves  -- stream each chunk's operands (w and kd^T fragments,
//                        shared by the compute waves, the tiles' u pairs and
//                        the gate row) into a D-stage LDS ring with
//                        global_load_lds (16 bytes per lane, written to LDS at
//                        lane*16 from the stage base), each issuing half of a
//                        chunk's loads and waiting for them by vmcnt alone.
// A compute wave takes in about 1 KB of operands per ~40 cycles whether from
// LDS or from memory, so its 34 KB of fragments per chunk, not the MFMAs,
// bound a chunk's time; the ring keeps that intake off memory latency and
// overlaps it with the products (below).
//
// The compute waves are software-pipelined across chunks: chunk i's w
// fragments are read into registers during chunk i-1's state update, and its
// kd^T, u and gate reads overlap its own v_new products.  One workgroup
// barrier per chunk, B_i, between the two halves of chunk i:
//   compute:  [reads of chunk i's kd^T, u, gate; v_new; all reads of stage
//             i % D complete]  B_i  [reads of chunk i+1's w; state update]
//   loaders:  [wait until chunk i+1 has landed]  B_i  [refill stage i % D,
//             which no compute wave reads again, with chunk i+D]
// B_{-1} (before the loop) certifies chunk 0.  The barrier is s_barrier
// between compiler-level memory fences; the explicit waits named above are
// the only ones it relies on.
template <typename E, int K, int V, int NC_, bool HAS_U = true, int RESERVE = 0>
struct RingCfg {
  static constexpr int FB = (int)sizeof(Frag<E>);      // bytes per lane per fragment
  static constexpr int KB = K / 32, KT = K / 16, NV = V / 16;
  static constexpr int NC = NC_;                       // compute waves (16-column tiles)
  static constexpr int WAVES = NC + 2;                 // compute waves, then two loaders
  static constexpr int FU = 4 * KB + 2 * KT;           // first u-pair fragment
  static constexpr int NFRAG = FU + (HAS_U ? 2 * NC : 0);  // w, kd^T, u-pair fragments per chunk
  static constexpr int SUB = FB / 16;                  // 1 KB blocks per fragment
  static constexpr int GOFF = NFRAG * 64 * FB;         // gate row (256 bytes) after the fragments
  static constexpr int STEP = GOFF + 256;              // bytes per ring stage
  static constexpr int NLOAD = NFRAG * SUB;            // 1 KB loads per chunk
  static constexpr int PER = NLOAD / 2;                // per loader wave; the first
                                                       // loader also loads the gate row
  static constexpr int D0 = (160 * 1024 - RESERVE) / STEP;  // RESERVE: other LDS of the kernel
  static constexpr int D = D0 > 6 ? 6 : D0;            // ring stages
  static constexpr int LDS = D * STEP;
  // fp32 fragments at K = 128 do not fit the pipelined registers in 256 VGPRs
  static constexpr bool FITS = FB == 16 || K <= 64;
  static_assert(NC == 1 || NC == 2, "one or two compute waves");
  static_assert(NV % NC == 0, "value tiles group evenly");
  static_assert(NLOAD % 2 == 0, "loads split evenly over the two loader waves");
  static_assert(D >= 2, "ring needs two stages");
  static_assert((D - 1) * (PER + 1) <= 63, "in-flight loads exceed vmcnt");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most ahead * PER of this wave's loads are outstanding.
template <int PER, int D>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if (ahead <= 0) wait_vmcnt<0>();
  else if constexpr (D > 2) {
    if (ahead == 1) wait_vmcnt<PER>();
    else if constexpr (D > 3) {
      if (ahead == 2) wait_vmcnt<2 * PER>();
      else if constexpr (D > 4) {
        if (ahead == 3) wait_vmcnt<3 * PER>();
        else if constexpr (D > 5) {
          wait_vmcnt<4 * PER>();
        }
      }
    }
  }
}

__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((global_void_t*)src, (lds_void_t*)lds_dst, 16, 0, 0);
}

// Fragment f of a ring stage (1 KB blocks, 16 bytes per lane).
__device__ __forceinline__ Frag<bf16> ring_frag(const char* stage, int f, int lane, bf16*) {
  return *reinterpret_cast<const Frag<bf16>*>(stage + f * 1024 + 16 * lane);
}
__device__ __forceinline__ Frag<float> ring_frag(const char* stage, int f, int lane, float*) {
  const char* b = stage + f * 2048 + 16 * lane;
  return {*reinterpret_cast<const f32x4*>(b), *reinterpret_cast<const f32x4*>(b + 1024)};
}
__device__ __forceinline__ void split_pair(const Frag<bf16>& f, Quad<bf16>& a, Quad<bf16>& b) {
  a.x = __builtin_shufflevector(f.x, f.x, 0, 1, 2, 3);
  b.x = __builtin_shufflevector(f.x, f.x, 4, 5, 6, 7);
}
__device__ __forceinline__ void split_pair(const Frag<float>& f, Quad<float>& a, Quad<float>& b) {
  a.x = f.lo;
  b.x = f.hi;
}

__device__ __forceinline__ void wait_lgkm0() {
  // gfx9 s_waitcnt with lgkmcnt = 0 and vmcnt / expcnt at their maxima
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Loader role of the LDS-ring state passes: loader lw (0 or 1) issues loads
// lw*PER .. lw*PER + PER-1 of each chunk (1 KB blocks of the fragments);
// loader 0 also loads the gate row.  It takes part in the ring's barriers
// B_{-1} .. B_{nsteps-1}, refilling stage i % D with chunk i + D after B_i.
template <typename R, typename E, int K, int V, int NC>
__device__ __forceinline__ void ring_loader(char* ring, int lw, const Geo& geo,
                                            const Frag<E>* __restrict__ wf,
                                            const Frag<E>* __restrict__ ktf,
                                            const Quad<E>* __restrict__ uf,
                                            const float* __restrict__ gam, size_t hbase, int vp,
                                            int nsteps) {
  constexpr int NV = V / 16, KB = K / 32, KT = K / 16, D = R::D;
  const int lane = threadIdx.x & 63;
  // Loader l issues loads l*PER .. l*PER + PER-1 of each chunk (1 KB blocks
  // of the fragments); loader 0 also loads the gate row.  Sources at chunk 0
  // (per lane); a chunk later every source has advanced by one slot of its
  // array.
  const int j0 = lw * R::PER;
  const char* src0[R::PER];
  size_t adv[R::PER];
#pragma unroll
  for (int jj = 0; jj < R::PER; ++jj) {
    const int j = j0 + jj;
    const int f = j / R::SUB, h = j - f * R::SUB;
    const char* base;
    if (f < 4 * KB) {
      const int ct = f / KB, kb = f - ct * KB;
      base = reinterpret_cast<const char*>(wf + ((hbase * 4 + ct) * KB + kb) * 64);
      adv[jj] = (size_t)4 * KB * 64 * R::FB;
    } else if (f < R::FU) {
      const int f2 = f - 4 * KB, mt = f2 >> 1, cb = f2 & 1;
      base = reinterpret_cast<const char*>(ktf + ((hbase * KT + mt) * 2 + cb) * 64);
      adv[jj] = (size_t)KT * 2 * 64 * R::FB;
    } else {
      const int q = f - R::FU, vt = NC * vp + (q >> 1), cp = q & 1;
      base = reinterpret_cast<const char*>(uf + ((hbase * NV + vt) * 2 + cp) * 64 * 2);
      adv[jj] = (size_t)NV * 2 * 64 * R::FB;
    }
    src0[jj] = base + lane * R::FB + 16 * h;
  }
  const float* gsrc0 = gam + hbase * kChunk + lane;
  auto issue = [&](int c) {
    char* stage = ring + (c % D) * R::STEP;
#pragma unroll
    for (int jj = 0; jj < R::PER; ++jj) dma16(src0[jj] + (size_t)c * adv[jj], stage + (j0 + jj) * 1024);
    if (lw == 0)
      __builtin_amdgcn_global_load_lds((global_void_t*)(gsrc0 + (size_t)c * kChunk),
                                       (lds_void_t*)(stage + R::GOFF), 4, 0, 0);
  };
  for (int c = 0; c < D - 1 && c < nsteps; ++c) issue(c);
  for (int i = -1; i < nsteps; ++i) {
    if (i + 1 < nsteps) {
      // chunk i+1 must have landed; chunks i+2 .. min(nsteps, i+D) - 1 may be in flight
      const int later = nsteps - 2 - i;
      const int ahead = later < D - 2 ? later : D - 2;
      if (lw == 0) wait_ahead<R::PER + 1, D>(ahead);  // also loads the gate row
      else wait_ahead<R::PER, D>(ahead);
    }
    ring_barrier();  // B_i
    if (i + D < nsteps) issue(i + D);
  }
}

template <typename E, int K, int V, bool VARLEN, int NC, int MODE = CHAIN_FULL>
__global__ __launch_bounds__((64 * RingCfg<E, K, V, NC>::WAVES)) void gdn_chain_ring_kernel(
    Geo geo, const Frag<E>* __restrict__ wf, const Frag<E>* __restrict__ ktf,
    const Quad<E>* __restrict__ uf, const float* __restrict__ gam,
    const int* __restrict__ seq_slot, const int* __restrict__ seq_order,
    const float* __restrict__ h0, float* __restrict__ fin, Frag<E>* __restrict__ hcf,
    Frag<E>* __restrict__ vnf) {
  using R = RingCfg<E, K, V, NC, MODE != CHAIN_MAP>;
  using Step = ChainStep<E, K, V, MODE>;
  constexpr int NV = V / 16, KB = K / 32, KT = K / 16, D = R::D;
  __shared__ __align__(16) char ring[R::LDS];
  // packed sequences with an order (the chunk map's seq_order): longest
  // first, for launches whose workgroups run in several rounds
  int hv, n, vp;
  if (VARLEN && seq_order != nullptr) {
    int r;
    rank_major_block(blockIdx.x, geo.HV, NV / NC, hv, r, vp);
    n = seq_order[r];
  } else {
    int rest;
    head_major_block(blockIdx.x, geo.HV, geo.N * (NV / NC), hv, rest);
    n = rest / (NV / NC);
    vp = rest - n * (NV / NC);
  }
  int s0, s1;
  if constexpr (VARLEN) {
    s0 = seq_slot[n];
    s1 = seq_slot[n + 1];
  } else {
    s0 = n * geo.NT;
    s1 = s0 + geo.NT;
  }
  const int nsteps = s1 - s0;
  // wave index made provably uniform, so the role branches and the LDS base
  // of global_load_lds stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const size_t hbase = (size_t)hv * geo.slots + s0;

  if (wave < NC) {
    const int vt = NC * vp + wave;
    const int g = lane >> 4, lc = lane & 15, v = 16 * vt + lc;
    const size_t sbase = ((size_t)n * geo.HV + hv) * K * V;
    f32x4 Hs[KT];
    init_state<K, V, MODE>(Hs, h0, sbase, v, g);
    Step st;
    auto read_w = [&](const char* stage) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) st.w[ct][kb] = ring_frag(stage, ct * KB + kb, lane, (E*)nullptr);
    };
    ring_barrier();  // B_{-1}
    if (nsteps > 0) read_w(ring);
    for (int i = 0; i < nsteps; ++i) {
      const char* stage = ring + (i % D) * R::STEP;
      // the chunk's last cumulative gate value, read by every lane (broadcast)
      const float glast = reinterpret_cast<const float*>(stage + R::GOFF)[kChunk - 1];
      if constexpr (MODE == CHAIN_MAP) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) st.u[ct] = make_quad<E>(f32x4{0.f, 0.f, 0.f, 0.f});
      } else {
#pragma unroll
        for (int cp = 0; cp < 2; ++cp)
          split_pair(ring_frag(stage, R::FU + 2 * wave + cp, lane, (E*)nullptr), st.u[2 * cp],
                     st.u[2 * cp + 1]);
      }
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          st.kt[mt][cb] = ring_frag(stage, 4 * KB + 2 * mt + cb, lane, (E*)nullptr);
      Frag<E> vb[2];
      st.vnew_global(Hs, vb, hcf, vnf, hbase + i, vt, lane);
      const float dec = fast_exp2(glast);
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
        Hs[mt] *= dec;
        // keep the decay ahead of the barrier, overlapping the products above
        asm volatile("" : "+v"(Hs[mt]));
      }
      wait_lgkm0();    // every read of stage i % D has completed
      ring_barrier();  // B_i
      if (i + 1 < nsteps) read_w(ring + ((i + 1) % D) * R::STEP);
      st.update(Hs, vb);
    }
    if (fin) {
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) fin[sbase + (size_t)(16 * mt + 4 * g + r) * V + v] = Hs[mt][r];
    }
  } else {
    ring_loader<R, E, K, V, NC>(ring, wave - NC, geo, wf, ktf, uf, gam, hbase, vp, nsteps);
  }
}

// ---------------------------------------------------------------------------
// State pass with the K rows split over K/32 waves (CHAIN_FULL): one workgroup
// per (sequence, value head, 16 value columns).  Wave q holds rows
// 32q .. 32q+31 of the K x 16 state (two D tiles) and reads only the w and
// kd^T fragments of those rows: a quarter of the one-wave variant's operand
// stream at K = 128, and a quarter of its products.  Per chunk:
//   store the wave's H_c fragment (k block q, the one-wave variant's layout);
//   partial products P_q = w[:, rows of q] H_c[rows of q], four 16-row tiles;
//   reduce-scatter through LDS: the wave owning chunk-row tile ct
//   (ct mod KB = q) forms v_new tile ct = u - (P_0 + P_1 + ...), summed in
//   wave order and rounded to the dtype;
//   exchange the v_new tiles, so every wave holds v_new; store v_new;
//   H[rows of q] <- e^{G_last} H[rows of q] + kd^T[rows of q] v_new.
// Two workgroup barriers per chunk.  Each wave loads its operands (about 65
// VGPRs per chunk for fp32 at K = 128) D chunks ahead into registers.  Used
// for fp32 operands, whose one-wave stream is twice the bf16 one.
template <typename E, int K, int V>
struct ChainKsStep {
  static constexpr int KB = K / 32, KT = K / 16, NV = V / 16, OWN = 4 / KB;
  Frag<E> w[4];      // w, chunk-row tile ct, k block q
  Frag<E> kt[2][2];  // kd^T, row tile 2q + j, chunk block cb
  Quad<E> u[OWN];    // u, chunk-row tiles q + KB j
  float gl;          // lane l: entry l of the chunk's gate row

  template <int Q>
  __device__ __forceinline__ void load(const Frag<E>* __restrict__ wf,
                                       const Frag<E>* __restrict__ ktf,
                                       const Quad<E>* __restrict__ uf,
                                       const float* __restrict__ gam, size_t hs, int vt,
                                       int lane) {
    gl = gam[hs * kChunk + lane];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) w[ct] = wf[((hs * 4 + ct) * KB + Q) * 64 + lane];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) kt[j][cb] = ktf[((hs * KT + 2 * Q + j) * 2 + cb) * 64 + lane];
#pragma unroll
    for (int j = 0; j < OWN; ++j) {
      const int ct = Q + KB * j;
      u[j] = uf[(((hs * NV + vt) * 2 + (ct >> 1)) * 64 + lane) * 2 + (ct & 1)];
    }
  }
};

__device__ __forceinline__ Frag<bf16> frag_join(const Quad<bf16>& a, const Quad<bf16>& b) {
  return {__builtin_shufflevector(a.x, b.x, 0, 1, 2, 3, 4, 5, 6, 7)};
}
__device__ __forceinline__ Frag<float> frag_join(const Quad<float>& a, const Quad<float>& b) {
  return {a.x, b.x};
}

template <typename E, int K, int V>
struct ChainKsLds {
  f32x4 part[K / 32][4][64];  // partial products, by wave and chunk-row tile
  Quad<E> vx[4][64];          // v_new tiles, rounded
};

// Wave Q's part of gdn_chain_ks_kernel (Q is the wave index, uniform).
template <typename E, int K, int V, int D, int Q>
__device__ __forceinline__ void chain_ks_wave(ChainKsLds<E, K, V>& sh, const Frag<E>* __restrict__ wf,
                                              const Frag<E>* __restrict__ ktf,
                                              const Quad<E>* __restrict__ uf,
                                              const float* __restrict__ gam, const float* __restrict__ h0,
                                              float* __restrict__ fin, Frag<E>* __restrict__ hcf,
                                              Frag<E>* __restrict__ vnf, int s0, int s1, size_t hbase,
                                              size_t sbase, int vt) {
  using Step = ChainKsStep<E, K, V>;
  constexpr int KB = Step::KB, NV = Step::NV, OWN = Step::OWN, HALF = KB / 2;
  const int lane = lane_id(), g = lane >> 4, v = 16 * vt + (lane & 15);
  f32x4 Hs[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Hs[j][r] = h0 ? h0[sbase + (size_t)(32 * Q + 16 * j + 4 * g + r) * V + v] : 0.f;

  auto chunk = [&](const Step& S, size_t hs) {
    const Frag<E> hb = frag_from_tiles<E>(Hs[0], Hs[1]);
    hcf[((hs * NV + vt) * KB + Q) * 64 + lane] = hb;
    f32x4 p[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      p[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      mma_k32(p[ct], S.w[ct], hb);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      if (ct % KB != Q) sh.part[Q][ct][lane] = p[ct];
    wait_lgkm0();
    ring_barrier();
    Quad<E> own[OWN];
#pragma unroll
    for (int j = 0; j < OWN; ++j) {
      const int ct = Q + KB * j;
      f32x4 acc = Q == 0 ? p[ct] : sh.part[0][ct][lane];
#pragma unroll
      for (int w2 = 1; w2 < KB; ++w2) acc += (w2 == Q ? p[ct] : sh.part[w2][ct][lane]);
      own[j] = make_quad<E>(quad_f32(S.u[j]) - acc);
      sh.vx[ct][lane] = own[j];
    }
    wait_lgkm0();
    ring_barrier();
    Quad<E> vq[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) vq[ct] = (ct % KB == Q) ? own[ct / KB] : sh.vx[ct][lane];
    Frag<E> vb[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) vb[cb] = frag_join(vq[2 * cb], vq[2 * cb + 1]);
    if constexpr (Q % HALF == HALF - 1) vnf[((hs * NV + vt) * 2 + Q / HALF) * 64 + lane] = vb[Q / HALF];
    const float dec = fast_exp2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(S.gl), kChunk - 1)));
    Hs[0] *= dec;
    Hs[1] *= dec;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 2; ++j) mma_k32(Hs[j], S.kt[j][cb], vb[cb]);
  };

  if (s0 < s1) {
    // The loads are issued unconditionally (clamped to the last chunk, in
    // bounds), so the compiler's wait counts stay exact around the loop; the
    // exit jumps past it.
    Step buf[D];
    const int last = s1 - 1;
#pragma unroll
    for (int j = 0; j < D; ++j) buf[j].template load<Q>(wf, ktf, uf, gam, hbase + min(s0 + j, last), vt, lane);
    for (int s = s0;; s += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (s + j >= s1) goto done;
        chunk(buf[j], hbase + s + j);
        buf[j].template load<Q>(wf, ktf, uf, gam, hbase + min(s + j + D, last), vt, lane);
        asm volatile("" ::: "memory");
      }
    }
  }
done:
  if (fin) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) fin[sbase + (size_t)(32 * Q + 16 * j + 4 * g + r) * V + v] = Hs[j][r];
  }
}

template <typename E, int K, int V, bool VARLEN, int D>
__global__ __launch_bounds__(64 * (K / 32)) void gdn_chain_ks_kernel(Geo geo, const Frag<E>* __restrict__ wf,
                                                                    const Frag<E>* __restrict__ ktf,
                                                                    const Quad<E>* __restrict__ uf,
                                                                    const float* __restrict__ gam,
                                                                    const int* __restrict__ seq_slot,
                                                                    const float* __restrict__ h0,
                                                                    float* __restrict__ fin,
                                                                    Frag<E>* __restrict__ hcf,
                                                                    Frag<E>* __restrict__ vnf) {
  static_assert(K == 64 || K == 128, "two or four waves");
  constexpr int NV = V / 16;
  __shared__ ChainKsLds<E, K, V> sh;
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
  const size_t sbase = ((size_t)n * geo.HV + hv) * K * V;
  const size_t hbase = (size_t)hv * geo.slots;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave == 0)
    chain_ks_wave<E, K, V, D, 0>(sh, wf, ktf, uf, gam, h0, fin, hcf, vnf, s0, s1, hbase, sbase, vt);
  else if (wave == 1)
    chain_ks_wave<E, K, V, D, 1>(sh, wf, ktf, uf, gam, h0, fin, hcf, vnf, s0, s1, hbase, sbase, vt);
  if constexpr (K == 128) {
    if (wave == 2)
      chain_ks_wave<E, K, V, D, 2>(sh, wf, ktf, uf, gam, h0, fin, hcf, vnf, s0, s1, hbase, sbase, vt);
    else if (wave == 3)
      chain_ks_wave<E, K, V, D, 3>(sh, wf, ktf, uf, gam, h0, fin, hcf, vnf, s0, s1, hbase, sbase, vt);
  }
}

// ---------------------------------------------------------------------------
// State pass with the output stage fused in (LDS-ring variant).  The chunk
// states never leave the CU: a workgroup is
//   NC compute waves -- as in gdn_chain_ring_kernel, except that H_c and v_new
//                       go to an LDS exchange (two buffers, by chunk parity)
//                       instead of memory;
//   NOUT output waves -- output wave ow owns query tiles TPW*ow ..
//                       TPW*ow + TPW-1 (TPW = 4 / NOUT) of every
//                       chunk: after B_i it takes chunk i's H_c and v_new
//                       fragments from the exchange and computes, for its
//                       tiles and the workgroup's NC value tiles,
//                         o^T = scale (e^{G_i} (H_c^T Q^T) + v_new^T P^T)
//                       with Q rows read from q and P^T from the WY stage
//                       (pf), both loaded into registers before the chunk's
//                       barrier (one register set: a second one, loading the
//                       next chunk during this one's products, measured
//                       slower);
//   two loader waves -- as in gdn_chain_ring_kernel.
// Exchange timing: compute writes buffer i%2 before B_i (its LDS writes have
// completed when it reaches the barrier); the output waves read it between B_i
// and B_{i+1} (completed before they reach B_{i+1}); compute writes it again
// only after B_{i+1}.  Every wave passes the same nsteps + 1 barriers.
template <typename E, int K, int V, int NC>
struct ChainOutCfg {
  static constexpr int FB = (int)sizeof(Frag<E>);
  static constexpr int XF = K / 32 + 2;                 // exchange fragments per compute wave
  static constexpr int XBYTES = 2 * NC * XF * 64 * FB;  // both buffers
  using R = RingCfg<E, K, V, NC, true, XBYTES>;
  static constexpr int NOUT = 4;                        // output waves
  static constexpr int TPW = 4 / NOUT;                  // query tiles per output wave
  static constexpr int WAVES = NC + NOUT + 2;           // compute, output, two loaders
  // the ring's registers hold bf16 fragments at any K, fp32 ones at K = 64
  static constexpr bool FITS = (FB == 16 || K <= 64) && wy_q_fits<E, K>();
};

template <typename E, int K, int V, bool VARLEN, int NC>
__global__ __launch_bounds__((64 * ChainOutCfg<E, K, V, NC>::WAVES)) void gdn_chain_out_kernel(
    Geo geo, const Frag<E>* __restrict__ wf, const Frag<E>* __restrict__ ktf,
    const Quad<E>* __restrict__ uf, const float* __restrict__ gam,
    const int* __restrict__ seq_slot, const int* __restrict__ seq_order,
    const int4* __restrict__ cmap, const float* __restrict__ h0, float* __restrict__ fin,
    const E* __restrict__ qg, const Frag<E>* __restrict__ pf, E* __restrict__ og) {
  using C = ChainOutCfg<E, K, V, NC>;
  static_assert(C::FITS, "fragments fit the ring's registers");
  using R = typename C::R;
  using Step = ChainStep<E, K, V, CHAIN_FULL>;
  constexpr int NV = V / 16, KB = K / 32, KT = K / 16, D = R::D, XF = C::XF;
  __shared__ __align__(16) char ring[R::LDS];
  __shared__ __align__(16) Frag<E> xch[2][NC][XF][64];
  // Beyond one workgroup per CU the workgroups run in rounds; packed
  // sequences are then taken longest first (seq_order), so that the longest
  // chains start in the first round.
  int hv, n, vp;
  if constexpr (VARLEN) {
    int r;
    rank_major_block(blockIdx.x, geo.HV, NV / NC, hv, r, vp);
    n = seq_order[r];
  } else {
    // a key head's value heads on one XCD: their output waves read the same q rows
    int rest;
    key_head_major_block(blockIdx.x, geo.H, geo.G, geo.N * (NV / NC), hv, rest);
    n = rest / (NV / NC);
    vp = rest - n * (NV / NC);
  }
  int s0, s1;
  if constexpr (VARLEN) {
    s0 = seq_slot[n];
    s1 = seq_slot[n + 1];
  } else {
    s0 = n * geo.NT;
    s1 = s0 + geo.NT;
  }
  const int nsteps = s1 - s0;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane >> 4, lc = lane & 15;
  const size_t hbase = (size_t)hv * geo.slots + s0;

  if (wave < NC) {
    const int vt = NC * vp + wave;
    const int v = 16 * vt + lc;
    const size_t sbase = ((size_t)n * geo.HV + hv) * K * V;
    f32x4 Hs[KT];
    init_state<K, V, CHAIN_FULL>(Hs, h0, sbase, v, g);
    Step st;
    auto read_w = [&](const char* stage) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) st.w[ct][kb] = ring_frag(stage, ct * KB + kb, lane, (E*)nullptr);
    };
    auto none_t = [](int, const f32x4&, const f32x4&) {};
    ring_barrier();  // B_{-1}
    if (nsteps > 0) read_w(ring);
    for (int i = 0; i < nsteps; ++i) {
      const char* stage = ring + (i % D) * R::STEP;
      const float glast = reinterpret_cast<const float*>(stage + R::GOFF)[kChunk - 1];
#pragma unroll
      for (int cp = 0; cp < 2; ++cp)
        split_pair(ring_frag(stage, R::FU + 2 * wave + cp, lane, (E*)nullptr), st.u[2 * cp],
                   st.u[2 * cp + 1]);
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          st.kt[mt][cb] = ring_frag(stage, 4 * KB + 2 * mt + cb, lane, (E*)nullptr);
      Frag<E> vb[2];
      Frag<E>* x = &xch[i & 1][wave][0][lane];
      // H_c goes to the exchange with k in natural order inside each k32
      // block (lane group g' holds k = 8g' .. 8g'+7), so that the output
      // waves' Q operands are single 16-byte runs of a q row.  The k order
      // of one product only has to agree between its two operands.  The
      // fragment's halves are the two D tiles (rows 4g .. 4g+3 of tiles 0
      // and 1 of the block): tile t's four values are k = 16t + 4g + r, that
      // is lane group 2t + g/2, elements 4(g%2) + r.
      char* xh = reinterpret_cast<char*>(&xch[i & 1][wave][0][0]);
      st.vnew(Hs, vb,
              [&](int kb, const Frag<E>& f) {
                // lane slot lc + 16 (2t + g/2), half g % 2 of its FB bytes
                constexpr int FB = C::FB;
                char* blk = xh + kb * 64 * FB + (lc + 16 * (g >> 1)) * FB + (g & 1) * (FB / 2);
                Quad<E> t0, t1;
                split_pair(f, t0, t1);
                *reinterpret_cast<Quad<E>*>(blk) = t0;
                *reinterpret_cast<Quad<E>*>(blk + 32 * FB) = t1;
              },
              [&](int cb, const Frag<E>& f) { x[(KB + cb) * 64] = f; }, none_t);
      const float dec = fast_exp2(glast);
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
        Hs[mt] *= dec;
        asm volatile("" : "+v"(Hs[mt]));
      }
      wait_lgkm0();    // stage i % D read, exchange i % 2 written
      ring_barrier();  // B_i
      if (i + 1 < nsteps) read_w(ring + ((i + 1) % D) * R::STEP);
      st.update(Hs, vb);
    }
    if (fin) {
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) fin[sbase + (size_t)(16 * mt + 4 * g + r) * V + v] = Hs[mt][r];
    }
  } else if (wave < NC + C::NOUT) {
    // output wave OW (0 .. NOUT-1, query tiles TPW*OW ..) as a compile-time
    // constant, so that every load count is fixed
    constexpr int TPW = C::TPW;
    auto role = [&](auto ow_c) {
      constexpr int OW = decltype(ow_c)::value;
      constexpr int it0 = TPW * OW;
      const int h = hv / geo.G;
      // the sequence's token range: chunk c covers bos + 64c .. min(bos + 64c + 64, eos)
      int64_t bos = 0, eos = 0;
      if (nsteps > 0) {
        if constexpr (VARLEN) {
          const int4 a = cmap[s0], b = cmap[s1 - 1];
          bos = a.y;
          eos = (int64_t)b.y + b.z;
        } else {
          bos = (int64_t)n * geo.T;
          eos = bos + geo.T;
        }
      }
      struct Ops {
        Frag<E> q[TPW][KB];  // Q rows of query tiles it0 + t (B operands over K)
        Frag<E> p[TPW][2];   // P^T fragments (it, jb), jb <= it/2
        float gq[TPW];       // cumulative gate (log2 units) of the lane's query in each tile
      };
      // Every load is unconditional (in bounds): a query row past the chunk's
      // end reads the chunk's last row instead; only output rows that are not
      // stored depend on it.  (A load skipped on some path would make the
      // compiler's wait counts fall back to draining every load.)
      auto load = [&](Ops& o, int c) {
        const int64_t t0 = bos + (int64_t)kChunk * c;
        const int len = (int)min((int64_t)kChunk, eos - t0);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const int it = it0 + t, row = 16 * it + lc;
          const E* qr = qg + ((t0 + min(row, len - 1)) * geo.H + h) * K + 8 * g;
          // k in natural order (see the exchange): one run of 8 elements each
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) o.q[t][kb] = *reinterpret_cast<const Frag<E>*>(qr + 32 * kb);
#pragma unroll
          for (int jb = 0; jb <= ((it0 + TPW - 1) >> 1); ++jb)
            if (jb <= ((it0 + t) >> 1)) o.p[t][jb] = pf[(((hbase + c) * 4 + it) * 2 + jb) * 64 + lane];
          o.gq[t] = gam[(hbase + c) * kChunk + row];
        }
      };
      auto out = [&](const Ops& o, int i) {
        const int64_t t0 = bos + (int64_t)kChunk * i;
        const int len = (int)min((int64_t)kChunk, eos - t0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const Frag<E>* x = &xch[i & 1][c][0][lane];
          Frag<E> hc[KB], vn[2];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) hc[kb] = x[kb * 64];
#pragma unroll
          for (int jb = 0; jb < 2; ++jb) vn[jb] = x[(KB + jb) * 64];
          const int vt = NC * vp + c;
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            const int it = it0 + t;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) mma_k32(acc, hc[kb], o.q[t][kb]);
            acc *= fast_exp2(o.gq[t]);
#pragma unroll
            for (int jb = 0; jb <= ((it0 + TPW - 1) >> 1); ++jb)
              if (jb <= ((it0 + t) >> 1)) mma_k32(acc, vn[jb], o.p[t][jb]);
            acc *= geo.scale;
            const int row = 16 * it + lc;
            if (row < len)
              st4(og + ((t0 + row) * geo.HV + hv) * V + 16 * vt + 4 * g, acc[0], acc[1], acc[2],
                  acc[3]);
          }
        }
      };
      // One register set: chunk i's operands are loaded at the top of its
      // step, before B_i, and consumed after it.
      ring_barrier();  // B_{-1}
      for (int i = 0; i < nsteps; ++i) {
        Ops cur;
        load(cur, i);
        ring_barrier();  // B_i
        out(cur, i);
        wait_lgkm0();    // exchange i % 2 read before B_{i+1}
      }
    };
    if (wave == NC) role(std::integral_constant<int, 0>{});
    else if (C::NOUT == 2 || wave == NC + 1) role(std::integral_constant<int, 1>{});
    else if constexpr (C::NOUT == 4) {
      if (wave == NC + 2) role(std::integral_constant<int, 2>{});
      else role(std::integral_constant<int, 3>{});
    }
  } else {
    ring_loader<R, E, K, V, NC>(ring, wave - NC - C::NOUT, geo, wf, ktf, uf, gam, hbase, vp, nsteps);
  }
}

// ---------------------------------------------------------------------------
// Segment table for the segment-parallel state pass.  Sequence n's chunks
// (slots s0 .. s1-1: seq_slot for packed input, n*NT .. (n+1)*NT-1 otherwise)
// are cut into ceil((s1 - s0) / L) segments of L chunks, numbered in sequence
// order.  seg_slot[j] = first slot of segment j; entries from the number of
// segments used up to nseg_max hold the end of the last sequence, so every
// segment j covers seg_slot[j] .. seg_slot[j+1]-1 (empty for unused j).
// seq_seg[n] = first segment of sequence n, seq_seg[N] = segments used.
// One workgroup (prefix sums over the sequences, 256 at a time).
template <bool VARLEN>
__global__ __launch_bounds__(256) void gdn_segment_map_kernel(const int* __restrict__ seq_slot,
                                                              int N, int NT, int L, int nseg_max,
                                                              int* __restrict__ seg_slot,
                                                              int* __restrict__ seq_seg) {
  __shared__ int ssum[256];
  __shared__ int carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < N; base += 256) {
    const int n = base + tid;
    int s0 = 0, s1 = 0;
    if (n < N) {
      s0 = VARLEN ? seq_slot[n] : n * NT;
      s1 = VARLEN ? seq_slot[n + 1] : (n + 1) * NT;
    }
    const int ns = (s1 - s0 + L - 1) / L;
    ssum[tid] = ns;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int y = tid >= off ? ssum[tid - off] : 0;
      __syncthreads();
      ssum[tid] += y;
      __syncthreads();
    }
    const int j0 = carry + ssum[tid] - ns;
    if (n < N) {
      seq_seg[n] = min(j0, nseg_max);
      for (int c = 0; c < ns; ++c)
        if (j0 + c < nseg_max) seg_slot[j0 + c] = s0 + c * L;
    }
    __syncthreads();
    if (tid == 255) carry += ssum[255];
    __syncthreads();
  }
  const int used = min(carry, nseg_max);
  const int end = N > 0 ? (VARLEN ? seq_slot[N] : N * NT) : 0;
  if (tid == 0) seq_seg[N] = used;
  for (int j = used + tid; j <= nseg_max; j += 256) seg_slot[j] = end;
}

// Level 2 of the segment-parallel state pass.  One workgroup of K/32 waves per
// (sequence, value head, 16 value columns) walks its sequence's segments in
// order:
//     seg_h[s] = H;   H <- M_s H + E_s,
// starting from h0 (or zero); the last H is the final state.  Wave q holds
// rows 32q .. 32q+31 of H (two fp32 D tiles) and forms those rows of M_s H on
// the MFMA: its rows of M_s as A fragments (converted from fp32), all of H as
// B fragments in the call's dtype, accumulating onto E_s's tiles in fp32.  H's
// k blocks pass between the waves through LDS (two buffers by segment parity,
// one barrier per segment).  Each wave loads its rows of M_s and E_s D
// segments ahead into registers, so a step costs the products and the
// exchange, not a memory round trip.
template <typename E>
__device__ __forceinline__ Frag<E> frag_from_f32_pieces(const f32x4& a, const f32x4& b);
template <>
__device__ __forceinline__ Frag<bf16> frag_from_f32_pieces<bf16>(const f32x4& a, const f32x4& b) {
  return frag_from_tiles<bf16>(a, b);
}
template <>
__device__ __forceinline__ Frag<float> frag_from_f32_pieces<float>(const f32x4& a, const f32x4& b) {
  return {a, b};
}

template <int K>
struct CombineStep {
  static constexpr int KB = K / 32;
  f32x4 m[2][KB][2];  // rows of M_s: row tile 2q + t, k block kb, the two 4-column pieces
  f32x4 e[2];         // E_s tiles (rows 32q + 16t + 4g + r, column v)

  __device__ __forceinline__ void load(const float* __restrict__ M, const float* __restrict__ Es,
                                       int q, int lane, int v, int V) {
    const int g = lane >> 4, lc = lane & 15;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float* row = M + (size_t)(32 * q + 16 * t + lc) * K;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        m[t][kb][0] = *reinterpret_cast<const f32x4*>(row + 32 * kb + 4 * g);
        m[t][kb][1] = *reinterpret_cast<const f32x4*>(row + 32 * kb + 16 + 4 * g);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) e[t][r] = Es[(size_t)(32 * q + 16 * t + 4 * g + r) * V + v];
    }
  }
};

template <typename E, int K, int V, int D, int Q>
__device__ __forceinline__ void combine_wave(Frag<E> (&xb)[2][K / 32][64], const Geo& geo, int n,
                                             int hv, int vt, const int* __restrict__ seq_seg,
                                             const float* __restrict__ seg_m,
                                             const float* __restrict__ seg_e,
                                             const float* __restrict__ h0, float* __restrict__ fin,
                                             float* __restrict__ seg_h) {
  constexpr int KB = K / 32;
  const int lane = lane_id(), g = lane >> 4, v = 16 * vt + (lane & 15);
  f32x4 Hs[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Hs[t][r] = h0 ? h0[((size_t)n * geo.HV + hv) * K * V + (size_t)(32 * Q + 16 * t + 4 * g + r) * V + v]
                    : 0.f;
  const int j0 = seq_seg[n], j1 = seq_seg[n + 1];
  auto mat = [&](int j) { return seg_m + ((size_t)j * geo.HV + hv) * K * K; };
  auto est = [&](int j) { return seg_e + ((size_t)j * geo.HV + hv) * K * V; };
  auto step = [&](const CombineStep<K>& S, int j, int par) {
    // this segment's start state: stored, and its k block shared
    float* hst = seg_h + ((size_t)j * geo.HV + hv) * K * V;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) hst[(size_t)(32 * Q + 16 * t + 4 * g + r) * V + v] = Hs[t][r];
    const Frag<E> own = frag_from_tiles<E>(Hs[0], Hs[1]);
    xb[par][Q][lane] = own;
    wait_lgkm0();
    ring_barrier();
    Frag<E> hb[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) hb[kb] = kb == Q ? own : xb[par][kb][lane];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 acc = S.e[t];
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const int kb = (Q + i) % KB;  // the wave's own block first: no LDS wait
        mma_k32(acc, frag_from_f32_pieces<E>(S.m[t][kb][0], S.m[t][kb][1]), hb[kb]);
      }
      Hs[t] = acc;
    }
  };
  if (j0 < j1) {
    // loads issued unconditionally (clamped to the last segment, in bounds), so
    // the compiler's wait counts stay exact around the loop
    CombineStep<K> buf[D];
    const int last = j1 - 1;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int jj = min(j0 + d, last);
      buf[d].load(mat(jj), est(jj), Q, lane, v, V);
    }
    for (int j = j0;; j += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (j + d >= j1) goto done;
        step(buf[d], j + d, (j + d - j0) & 1);
        const int jj = min(j + d + D, last);
        buf[d].load(mat(jj), est(jj), Q, lane, v, V);
        asm volatile("" ::: "memory");
      }
    }
  }
done:
  if (fin) {
    const size_t sbase = ((size_t)n * geo.HV + hv) * K * V;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) fin[sbase + (size_t)(32 * Q + 16 * t + 4 * g + r) * V + v] = Hs[t][r];
  }
}

// Grid: one workgroup of K/32 waves per (sequence, value head, 16 value columns).
template <typename E, int K, int V>
__global__ __launch_bounds__(64 * (K / 32)) void gdn_segment_combine_kernel(
    Geo geo, const int* __restrict__ seq_seg, const float* __restrict__ seg_m,
    const float* __restrict__ seg_e, const float* __restrict__ h0, float* __restrict__ fin,
    float* __restrict__ seg_h) {
  static_assert(K == 64 || K == 128, "two or four waves");
  constexpr int NV = V / 16, D = 2;
  __shared__ Frag<E> xb[2][K / 32][64];
  const int b = blockIdx.x;
  const int vt = b % NV, hv = (b / NV) % geo.HV, n = b / (NV * geo.HV);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave == 0)
    combine_wave<E, K, V, D, 0>(xb, geo, n, hv, vt, seq_seg, seg_m, seg_e, h0, fin, seg_h);
  else if (wave == 1)
    combine_wave<E, K, V, D, 1>(xb, geo, n, hv, vt, seq_seg, seg_m, seg_e, h0, fin, seg_h);
  if constexpr (K == 128) {
    if (wave == 2)
      combine_wave<E, K, V, D, 2>(xb, geo, n, hv, vt, seq_seg, seg_m, seg_e, h0, fin, seg_h);
    else if (wave == 3)
      combine_wave<E, K, V, D, 3>(xb, geo, n, hv, vt, seq_seg, seg_m, seg_e, h0, fin, seg_h);
  }
}

// ---------------------------------------------------------------------------
// Output.  One workgroup (4 waves) per (chunk slot, GS value heads of one key
// head), computing o^T (V x 64) so that the state and v_new fragments written
// by the chain are the A operands and rows of Q / P^T are the B operands:
//   S^T = K Q^T                               (wave w: token tile i = w; once)
//   P^T = S^T * [j <= i] * e^{G_i - G_j}      (per value head: its own G)
//   o^T = e^{G_i} (H_c^T Q^T) + v_new^T P^T, times scale  (wave w: value tiles w, w+4)
// With GS > 1 the Q and K rows are read and S formed once for the value heads
// hv0 .. hv0+GS-1 that share the key head (GS divides G).
template <typename E, int K, int V, bool VARLEN, int GS = 1>
__global__ __launch_bounds__(256) void gdn_output_kernel(Geo geo, const E* __restrict__ qg,
                                                         const E* __restrict__ kg,
                                                         const int4* __restrict__ cmap,
                                                         const float* __restrict__ gam,
                                                         const Frag<E>* __restrict__ hcf,
                                                         const Frag<E>* __restrict__ vnf,
                                                         E* __restrict__ og) {
  constexpr int P = 16 / sizeof(E), KS = K + P, NV = V / 16, KB = K / 32;
  static_assert(GS >= 1 && GS <= 4, "value heads per workgroup");
  __shared__ __align__(16) E Qs[kChunk * KS];
  __shared__ __align__(16) E Ks[kChunk * KS];
  __shared__ __align__(16) Frag<E> Pb[GS][4][2][64];
  __shared__ float sg[GS][kChunk];

  int hg, slot;
  head_major_block(blockIdx.x, geo.HV / GS, geo.slots, hg, slot);
  const int hv0 = hg * GS;
  int n, len;
  int64_t t0;
  if (!chunk_of_slot<VARLEN>(geo, cmap, slot, n, t0, len)) return;
  const int h = hv0 / geo.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, lc = lane & 15;

  // All global loads first: this wave's H_c and v_new fragments (value tiles
  // wave, wave+4, ..., of every value head), the gate rows, and the Q and K
  // rows of the chunk.
  constexpr int NVW = (NV + 3) / 4;  // value tiles per wave
  Frag<E> hc[GS][NVW][KB], vn[GS][NVW][2];
#pragma unroll
  for (int gi = 0; gi < GS; ++gi) {
    const size_t hs = (size_t)(hv0 + gi) * geo.slots + slot;
#pragma unroll
    for (int a = 0; a < NVW; ++a) {
      const int vt = wave + 4 * a;
      if (vt < NV) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) hc[gi][a][kb] = hcf[((hs * NV + vt) * KB + kb) * 64 + lane];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) vn[gi][a][jb] = vnf[((hs * NV + vt) * 2 + jb) * 64 + lane];
      }
    }
  }
  if (tid < kChunk * GS) {
    const int gi = tid / kChunk, c = tid - gi * kChunk;
    sg[gi][c] = gam[((size_t)(hv0 + gi) * geo.slots + slot) * kChunk + c];
  }
  constexpr int NIT = kChunk * (K / 8) / 256;  // 8-element pieces per thread
  Raw8<E> eq[NIT], ek[NIT];                      // as loaded
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int m = tid + 256 * it, row = m / (K / 8), c0 = 8 * (m % (K / 8));
    if (row < len) {
      eq[it].load(qg + ((t0 + row) * geo.H + h) * K + c0);
      ek[it].load(kg + ((t0 + row) * geo.H + h) * K + c0);
    } else {
      eq[it].zero();
      ek[it].zero();
    }
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int m = tid + 256 * it, row = m / (K / 8), c0 = 8 * (m % (K / 8));
    eq[it].store(Qs + row * KS + c0);
    ek[it].store(Ks + row * KS + c0);
  }
  __syncthreads();

  {
    const int it = wave;
    f32x4 st[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      st[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (jt <= it) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          mma_k32(st[jt], frag_from_row(Ks + (16 * jt + lc) * KS + 32 * kb),
                  frag_from_row(Qs + (16 * it + lc) * KS + 32 * kb));
      }
    }
    const int i = 16 * it + lc;
#pragma unroll
    for (int gi = 0; gi < GS; ++gi) {
      f32x4 pt[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * jt + 4 * g + r;
          pt[jt][r] = (jt <= it && j <= i) ? st[jt][r] * fast_exp2(sg[gi][i] - sg[gi][j]) : 0.f;
        }
      }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) Pb[gi][it][jb][lane] = frag_from_tiles<E>(pt[2 * jb], pt[2 * jb + 1]);
    }
  }
  __syncthreads();

#pragma unroll
  for (int gi = 0; gi < GS; ++gi) {
    const int hv = hv0 + gi;
#pragma unroll
    for (int a = 0; a < NVW; ++a) {
      const int vt = wave + 4 * a;
      if (vt >= NV) break;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          mma_k32(acc, hc[gi][a][kb], frag_from_row(Qs + (16 * it + lc) * KS + 32 * kb));
        acc *= fast_exp2(sg[gi][16 * it + lc]);
#pragma unroll
        for (int jb = 0; jb <= (it >> 1); ++jb) mma_k32(acc, vn[gi][a][jb], Pb[gi][it][jb][lane]);
        acc *= geo.scale;
        const int i = 16 * it + lc;
        if (i < len) {
          E* dst = og + ((t0 + i) * geo.HV + hv) * V + 16 * vt + 4 * g;
          st4(dst, acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
  }
}

}  // namespace gdn
