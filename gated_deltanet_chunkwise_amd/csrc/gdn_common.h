// gdn_common.h -- gfx950 device helpers shared by the GDN kernels.
//
// MFMA fragments.  All contractions use 16x16 output tiles.  An output tile
// ("D tile", f32x4 per lane) holds D[4*g + r][lane % 16] in element r, with
// g = lane / 16: four consecutive rows of one column.
//
// Reductions run over blocks of 32 indices ("k32 blocks").  A k32 operand
// fragment holds, per lane, 8 values at the k offsets
//     kslot(g, i) = 4*g + i          for i = 0..3
//                   16 + 4*g + (i-4) for i = 4..7
// of the block, for the lane's row (A operand: row lane%16) or column
// (B operand: column lane%16).  Any k order gives the same sum as long as the
// A and B fragments agree; this one has the property that two D tiles covering
// rows 0..15 and 16..31 of a block ARE a k32 fragment (element i<4 from the
// first tile, i>=4 from the second), so a product's output feeds the next
// product's reduction straight from registers with no LDS round trip.
//
//   bf16:  one v_mfma_f32_16x16x32_bf16 per k32 block (8 bf16 per lane).
//   fp32:  eight v_mfma_f32_16x16x4_f32, the s-th taking element s of both
//          fragments (k rows {kslot(g, s) : g = 0..3}, which are distinct).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;  // tokens per chunk
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

template <typename E> struct Frag;
template <> struct Frag<bf16> { bf16x8 x; };
template <> struct Frag<float> { f32x4 lo, hi; };

// Four consecutive elements (one D-tile lane's column segment), stored.
template <typename E> struct Quad;
template <> struct Quad<bf16> { bf16x4 x; };
template <> struct Quad<float> { f32x4 x; };

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  return __builtin_convertvector(v, bf16x4);
}
__device__ __forceinline__ f32x4 to_f32x4(bf16x4 v) { return __builtin_convertvector(v, f32x4); }

template <typename E> __device__ __forceinline__ Quad<E> make_quad(f32x4 v);
template <> __device__ __forceinline__ Quad<bf16> make_quad<bf16>(f32x4 v) { return {to_bf16x4(v)}; }
template <> __device__ __forceinline__ Quad<float> make_quad<float>(f32x4 v) { return {v}; }
__device__ __forceinline__ f32x4 quad_f32(const Quad<bf16>& q) { return to_f32x4(q.x); }
__device__ __forceinline__ f32x4 quad_f32(const Quad<float>& q) { return q.x; }

// Two D tiles (rows 0..15 and 16..31 of a k32 block) -> a k32 fragment.
template <typename E> __device__ __forceinline__ Frag<E> frag_from_tiles(f32x4 d0, f32x4 d1);
template <> __device__ __forceinline__ Frag<bf16> frag_from_tiles<bf16>(f32x4 d0, f32x4 d1) {
  bf16x4 a = to_bf16x4(d0), b = to_bf16x4(d1);
  return {__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7)};
}
template <> __device__ __forceinline__ Frag<float> frag_from_tiles<float>(f32x4 d0, f32x4 d1) {
  return {d0, d1};
}

// k32 fragment from its two 4-element pieces (k offsets 4g.. and 16+4g..).
__device__ __forceinline__ Frag<bf16> frag_from_pieces(const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  return {__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7)};
}
__device__ __forceinline__ Frag<float> frag_from_pieces(const float* p0, const float* p1) {
  return {*reinterpret_cast<const f32x4*>(p0), *reinterpret_cast<const f32x4*>(p1)};
}

// k32 fragment from a row-major matrix row: `row` points at element 32*kb of
// the lane's row (A operand) or column-as-row (B operand).  Works for LDS and
// global pointers; both 4-element pieces must be 8-byte (bf16) / 16-byte
// (fp32) aligned.
__device__ __forceinline__ Frag<bf16> frag_from_row(const bf16* row) {
  const int g = lane_id() >> 4;
  bf16x4 a = *reinterpret_cast<const bf16x4*>(row + 4 * g);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(row + 16 + 4 * g);
  return {__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7)};
}
__device__ __forceinline__ Frag<float> frag_from_row(const float* row) {
  const int g = lane_id() >> 4;
  return {*reinterpret_cast<const f32x4*>(row + 4 * g),
          *reinterpret_cast<const f32x4*>(row + 16 + 4 * g)};
}

// acc += A * B over one k32 block.
__device__ __forceinline__ void mma_k32(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.x, b.x, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_k32(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[s], b.lo[s], acc, 0, 0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[s], b.hi[s], acc, 0, 0, 0);
}

// Plain fp32 16x16x4 MFMA (A[m=lane%16][k=lane/16], B[k=lane/16][n=lane%16]).
__device__ __forceinline__ f32x4 mfma_f32_4(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// softplus(x) = log(1 + e^x), taken as x above 20 (the threshold of the KDA
// gate guide, "core computation logic"), in fp32.  log(1 + e^x) uses the
// hardware base-2 exp and log (v_exp_f32, v_log_f32; measured on gfx950 against
// fp64: at most 0.77 and 1.0 ulp for normal results, the log also just above 1)
// and Kahan's log1p correction (D. Goldberg, "What every computer scientist
// should know about floating-point arithmetic", 1991, Theorem 4): with y = e^x
// and u = fl(1 + y),
//     log1p(y) = log(u) * y / (u - 1)    (u != 1),   = y   (u == 1),
// which cancels the rounding of 1 + y.  v_exp_f32 flushes results below 2^-126,
// so for x log2(e) < -64 the exponent is shifted by 64 and the result scaled by
// 2^-64 (exact, one rounding into the subnormal range).  The error is a few ulp
// plus the |x| * 2^-24 that rounding x itself costs, in ~15 instructions where
// the device library's log1pf(expf(x)) takes ~140.
__device__ __forceinline__ float gate_softplus(float x) {
  if (x > 20.f) return x;
  const float t = x * kLog2e;
  const bool deep = t < -64.f;
  float y = __builtin_amdgcn_exp2f(deep ? t + 64.f : t);
  if (deep) y *= 0x1p-64f;
  const float u = 1.f + y;
  if (u == 1.f) return y;
  return __builtin_amdgcn_logf(u) * 0.693147180559945309f * (y * __builtin_amdgcn_rcpf(u - 1.f));
}

// Chunk geometry shared by all kernels (passed by value).
struct Geo {
  int B, T, H, HV, K, V, N;  // N = number of sequences
  int G;                     // HV / H: value heads per key head
  int NT;                    // chunks per sequence without cu_seqlens
  int slots;                 // chunk slots
  float scale;
};

// Chunk slot -> (sequence, absolute first token, length).  Returns false for
// an unused slot (packed sequences only).
template <bool VARLEN>
__device__ __forceinline__ bool chunk_of_slot(const Geo& geo, const int4* cmap, int slot,
                                              int& n, int64_t& t0, int& len) {
  if constexpr (VARLEN) {
    int4 e = cmap[slot];
    n = e.x;
    t0 = e.y;
    len = e.z;
    return e.z > 0;
  } else {
    n = slot / geo.NT;
    int c = slot - n * geo.NT;
    t0 = (int64_t)n * geo.T + (int64_t)c * kChunk;
    len = min(kChunk, geo.T - c * kChunk);
    return true;
  }
}

// Block id -> (value head, index within the head), such that every block of a
// head lands on one XCD when HV is a multiple of 8 (workgroups are dispatched
// to the 8 XCDs round-robin by id), keeping a head's intermediates in one L2.
// A bijection of [0, HV * per_head) in both branches.
__device__ __forceinline__ void head_major_block(int b, int HV, int per_head, int& hv, int& rest) {
  if ((HV & 7) == 0) {
    const int x = b & 7, j = b >> 3;
    const int hl = j / per_head;
    rest = j - hl * per_head;
    hv = x + 8 * hl;
  } else {
    hv = b / per_head;
    rest = b - hv * per_head;
  }
}

// Block id -> (value head, index within the head) like head_major_block, but
// with the XCD chosen by key head: with H a multiple of 8, key head h's value
// heads (hv = h G .. h G + G - 1) all go to XCD h % 8, so the query rows they
// share come through one L2.  With one value head per key head it is
// head_major_block's mapping.  A bijection of [0, H G per_head).
__device__ __forceinline__ void key_head_major_block(int b, int H, int G, int per_head, int& hv,
                                                     int& rest) {
  if ((H & 7) == 0) {
    const int x = b & 7, j = b >> 3;
    const int kl = j / (G * per_head), r2 = j - kl * (G * per_head);
    const int r = r2 / per_head;
    rest = r2 - r * per_head;
    hv = (x + 8 * kl) * G + r;
  } else {
    hv = b / per_head;
    rest = b - hv * per_head;
  }
}

// Block id -> (value head, sequence rank r, group of value tiles vp) for a
// state pass over packed sequences whose workgroups do not all fit on the
// device at once: rank-major, so the workgroups of the sequence of rank 0 (the
// longest, in the chunk map's order) are dispatched first, then rank 1, and so
// on.  With HV a multiple of 8 a value head keeps the XCD head_major_block
// gives it (hv % 8), so the workgroups of one (sequence, head) share that
// XCD's L2.  A bijection of [0, nseq * HV * groups).
__device__ __forceinline__ void rank_major_block(int b, int HV, int groups, int& hv, int& r,
                                                 int& vp) {
  if ((HV & 7) == 0) {
    const int x = b & 7, j = b >> 3, hl8 = HV >> 3;
    vp = j % groups;
    const int t = j / groups;
    r = t / hl8;
    hv = x + 8 * (t - r * hl8);
  } else {
    vp = b % groups;
    const int t = b / groups;
    r = t / HV;
    hv = t - r * HV;
  }
}

// Block id -> (value head, chunk slot) for the per-(chunk, value head) WY
// kernel.  With H a multiple of 8, key head h's value heads go to XCD h % 8,
// and on each XCD the blocks run slot-major over its value heads, so one
// chunk's workgroups for all of an XCD's value heads are dispatched together:
// they read the same K rows (the value heads of a key head) and the same gate
// and beta lines (the [T][HV] rows hold every head), which then come from that
// XCD's L2 once instead of once per value head.  Otherwise slot-major over all
// value heads.  A bijection of [0, HV * slots) in both branches; with one value
// head per key head and HV = 8 it is head_major_block's mapping.
__device__ __forceinline__ void xcd_slot_block(int b, int H, int G, int slots, int& hv, int& slot) {
  if ((H & 7) == 0) {
    const int x = b & 7, j = b >> 3;
    const int nh = (H >> 3) * G;  // value heads per XCD
    slot = j / nh;
    const int r = j - slot * nh;
    hv = (x + 8 * (r / G)) * G + r % G;
  } else {
    const int HV = H * G;
    slot = b / HV;
    hv = b - slot * HV;
  }
}

}  // namespace gdn
