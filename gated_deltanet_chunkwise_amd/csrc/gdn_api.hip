// gdn_api.hip -- host side of libgdn: argument validation, workspace layout
// and the launch sequence.  See include/gdn.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

#include "gdn.h"
#include "gdn_bwd.h"
#include "gdn_decode.h"
#include "gdn_kda.h"
#include "gdn_kernels.h"

namespace {

constexpr size_t kWsAlign = 256;
size_t align_up(size_t x) { return (x + kWsAlign - 1) & ~(kWsAlign - 1); }

struct Plan {
  gdn::Geo geo;
  gdn_workspace_layout_t lay;
  bool varlen;
  int64_t ntok;    // tokens in q/k/v/o
  int seg_chunks;  // chunks per segment of the segment-parallel state pass (0: off,
                   // GDN_SEG_AUTO: chosen at launch, see auto_seg_chunks)
};

// Smallest segment the automatic choice takes; the workspace of a
// GDN_SEG_AUTO call is sized for it, so it holds whatever the choice is.
constexpr int kAutoSegMin = 16;

// The automatic segment length for B fixed-length sequences of NT chunks and
// `units` (sequence, value head, 16-column) state-pass units on a device with
// `cus` compute units; 0 = the plain pass.  Cost model, measured on MI355X
// (256 CUs, bf16, K = V = 128, T = 65536): the segmented pass costs about
// three passes of L chunk steps at units * NS units (NS = NT / L segments) plus
// NS combine steps, the plain pass NT steps at `units` units; a step is
// cheapest at up to two units per CU.  The best L measured puts units * NS at
// two per CU: 16 units L = 32 (state pass 530 -> 225 us), 32 units L = 64
// (722 -> 326 us), 64 units L = 128 (772 -> 387 us).  With fewer than 8
// segments the three passes cost more than the one they replace (256 units,
// NS = 2: 1062 -> 1730 us at the best L), and below 16 chunks a segment is
// too short to amortise its start.
int auto_seg_chunks(int64_t units, int NT, int cus) {
  if (units <= 0 || cus <= 0) return 0;
  const int64_t ns = 2 * (int64_t)cus / units;
  if (ns < 8) return 0;
  const int64_t L = std::max<int64_t>((NT + ns - 1) / ns, kAutoSegMin);
  return NT / L >= 8 ? (int)L : 0;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The int a C caller passed for an enum-typed argument.  C lets any int
// through; loading an enum object that holds a value outside the enumerators'
// range is undefined in C++, so the bits are read instead of the enum.
template <typename Enum>
int enum_bits(const Enum& e) {
  static_assert(sizeof(Enum) == sizeof(int), "enum arguments are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

// Compute units of the current device (cached per device id; a benign race
// at worst stores the same value twice).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Shapes and sizes only (no pointers).
gdn_status_t make_plan(const gdn_params_t* p, bool varlen, Plan* out) {
  if (!p) return GDN_ERR_NULL;
  if (p->dtype != GDN_F32 && p->dtype != GDN_BF16) return GDN_ERR_DTYPE;
  if (p->B < 0 || p->T < 0 || p->H <= 0 || p->HV <= 0 || p->K <= 0 || p->V <= 0) return GDN_ERR_SHAPE;
  if (p->HV % p->H) return GDN_ERR_SHAPE;
  if ((p->K != 64 && p->K != 128) || (p->V != 64 && p->V != 128)) return GDN_ERR_UNSUPPORTED;
  if (varlen && (p->B != 1 || p->num_seqs < 0)) return GDN_ERR_SHAPE;
  // tokens but no sequence: cu_seqlens = {0} cannot end at T > 0, and every
  // per-chunk launch would read a chunk map that nothing wrote
  if (varlen && p->num_seqs == 0 && p->T > 0) return GDN_ERR_SHAPE;
  if (p->seg_chunks < 0 && p->seg_chunks != GDN_SEG_AUTO) return GDN_ERR_SHAPE;
  const int64_t N = varlen ? p->num_seqs : p->B;
  const int64_t NT = ((int64_t)p->T + gdn::kChunk - 1) / gdn::kChunk;
  const int64_t slots = varlen ? (int64_t)p->T / gdn::kChunk + N : (int64_t)p->B * NT;
  const int64_t ntok = varlen ? (int64_t)p->T : (int64_t)p->B * p->T;
  // Index arithmetic uses int32 for slots, units and tokens within a packed batch.
  const int64_t units = N * p->HV * (p->V / 16);
  if (slots > INT32_MAX / 2 || slots * p->HV > INT32_MAX || units > INT32_MAX || N + 1 > INT32_MAX)
    return GDN_ERR_UNSUPPORTED;

  Plan pl{};
  pl.varlen = varlen;
  pl.ntok = ntok;
  // packed input: the sequence lengths are on the device, so the automatic
  // choice is the plain pass
  pl.seg_chunks = (p->seg_chunks == GDN_SEG_AUTO && varlen) ? 0 : p->seg_chunks;
  gdn::Geo& g = pl.geo;
  g.B = p->B; g.T = p->T; g.H = p->H; g.HV = p->HV; g.K = p->K; g.V = p->V;
  g.N = (int)N; g.G = p->HV / p->H; g.NT = (int)NT; g.slots = (int)slots; g.scale = p->scale;

  const size_t esz = p->dtype == GDN_BF16 ? 2 : 4;
  const size_t hsl = (size_t)p->HV * (size_t)slots;  // (head, slot) pairs
  gdn_workspace_layout_t& L = pl.lay;
  size_t off = 0;
  L.gamma = off; off = align_up(off + hsl * gdn::kChunk * 4);
  L.beta = off;  off = align_up(off + hsl * gdn::kChunk * 4);
  L.w = off;     off = align_up(off + hsl * gdn::kChunk * p->K * esz);
  L.kt = off;    off = align_up(off + hsl * gdn::kChunk * p->K * esz);
  L.u = off;     off = align_up(off + hsl * gdn::kChunk * p->V * esz);
  L.hc = off;    off = align_up(off + hsl * (size_t)p->K * p->V * esz);
  L.vn = off;    off = align_up(off + hsl * gdn::kChunk * p->V * esz);
  L.pm = off;    off = align_up(off + hsl * gdn::kChunk * gdn::kChunk * esz);  // [4][2] k32 fragments
  L.chunk_map = off; off = align_up(off + (varlen ? (size_t)slots * 16 : 0));
  L.seq_slot = off;  off = align_up(off + (varlen ? (size_t)(N + 1) * 4 : 0));
  L.seq_order = off; off = align_up(off + (varlen ? (size_t)N * 4 : 0));
  // segments: at most ceil(c_n / L) per sequence, summing to <= slots / L + N
  int64_t nseg = 0;
  if (pl.seg_chunks != 0) {
    const int Lmin = pl.seg_chunks > 0 ? pl.seg_chunks : kAutoSegMin;  // GDN_SEG_AUTO: the bound
    nseg = varlen ? slots / Lmin + N : N * ((NT + Lmin - 1) / Lmin);
    if (nseg * p->HV * (p->V / 16) > INT32_MAX || nseg + 1 > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    const size_t per = (size_t)nseg * p->HV * p->K;
    L.seg_slot = off; off = align_up(off + (size_t)(nseg + 1) * 4);
    L.seq_seg = off;  off = align_up(off + (size_t)(N + 1) * 4);
    L.seg_e = off;    off = align_up(off + per * p->V * 4);
    L.seg_m = off;    off = align_up(off + per * p->K * 4);
    L.seg_h = off;    off = align_up(off + per * p->V * 4);
  }
  L.total = off;
  L.num_slots = (int32_t)slots;
  L.num_seqs = (int32_t)N;
  L.num_segs = (int32_t)nseg;
  *out = pl;
  return GDN_OK;
}

gdn_status_t check_all(const gdn_params_t* p, const void* q, const void* k, const void* v,
                       const float* g_raw, const float* beta, const float* A_log,
                       const float* dt_bias, const int64_t* cu_seqlens,
                       const float* initial_state, const void* o, const float* final_state,
                       const void* workspace, size_t workspace_bytes, Plan* plan) {
  if (!p) return GDN_ERR_NULL;
  gdn_status_t st = make_plan(p, cu_seqlens != nullptr, plan);
  if (st != GDN_OK) return st;
  const bool tokens = plan->ntok > 0;
  if (tokens && (!q || !k || !v || !g_raw || !beta || !A_log || !o)) return GDN_ERR_NULL;
  if (plan->lay.total > 0 && !workspace) return GDN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return GDN_ERR_ALIGN;
  if (!aligned(g_raw, 4) || !aligned(beta, 4) || !aligned(A_log, 4) || !aligned(dt_bias, 4) ||
      !aligned(initial_state, 4) || !aligned(final_state, 4))
    return GDN_ERR_ALIGN;
  if (!aligned(cu_seqlens, 8) || !aligned(workspace, kWsAlign)) return GDN_ERR_ALIGN;
  if (workspace_bytes < plan->lay.total) return GDN_ERR_WORKSPACE;
  return GDN_OK;
}

// hipLaunchKernel with the argument tuple converted to the kernel's own types.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t s, Args&&... args) {
  std::tuple<KArgs...> t(std::forward<Args>(args)...);
  return std::apply(
      [&](auto&... a) {
        void* argv[] = {(void*)&a...};
        return hipLaunchKernel((const void*)kern, grid, block, argv, 0, s);
      },
      t);
}

// The state pass in one mode, over geo.N pseudo-sequences whose slot ranges
// are seq_slot[n] .. seq_slot[n+1]-1 (VARLEN) or n*NT .. (n+1)*NT-1.  The
// LDS-ring variant when its workgroups fit one per CU: one compute wave (16
// columns) per workgroup when the units fit, two sharing the ring otherwise;
// beyond that many units share a CU and the register-buffered variant is used
// (also for fp32 at K = 128, whose pipelined operands do not fit the ring
// variant's registers), except in CHAIN_PLAIN mode, which keeps the two-wave
// ring.  seq_order (packed input, not segments): the ring's workgroups take
// the sequences longest first.
template <typename E, int K, int V, bool VARLEN, int MODE>
hipError_t launch_chain(const gdn::Geo& geo, hipStream_t s, const gdn::Frag<E>* wf,
                        const gdn::Frag<E>* ktf, const gdn::Quad<E>* uf, const float* gam,
                        const int* seq_slot, const float* h0, float* fin, gdn::Frag<E>* hcf,
                        gdn::Frag<E>* vnf, const int* seq_order = nullptr) {
  const int units = geo.N * geo.HV * (V / 16);
  if (units == 0) return hipSuccess;
  const int cus = device_cus();
  // fp32 operands, one unit per CU or fewer: the K rows split over K/32
  // waves, each reading a K/32-th of the chunk's (doubled-width) fragments.
  // Measured on MI355X: B=1, T=256, H=2, K=V=64 state pass 7.6 us against
  // 11.7 for the one-wave ring.  Not for bf16, whose one-wave operand stream
  // is half as wide: B=2, T=2048, H=8, K=V=128 took 27.0 us against 21.5,
  // the two barriers and LDS round trips per chunk outlasting the intake
  // they save.
  if constexpr (MODE == gdn::CHAIN_FULL && sizeof(E) == 4 && (K == 64 || K == 128)) {
    if (units <= cus)
      return launch(gdn::gdn_chain_ks_kernel<E, K, V, VARLEN, 2>, dim3(units),
                    dim3(64 * (K / 32)), s, geo, wf, ktf, uf, gam, seq_slot, h0, fin, hcf, vnf);
  }
  if constexpr (gdn::RingCfg<E, K, V, 1>::FITS) {
    if (units <= cus)
      return launch(gdn::gdn_chain_ring_kernel<E, K, V, VARLEN, 1, MODE>, dim3(units),
                    dim3(64 * gdn::RingCfg<E, K, V, 1>::WAVES), s, geo, wf, ktf, uf, gam, seq_slot,
                    seq_order, h0, fin, hcf, vnf);
    // CHAIN_PLAIN (the backward's recompute, row-major stores) keeps the ring at
    // any unit count, its workgroups then in rounds.  Measured on MI355X at
    // 12 packed sequences, T=32768, H=16 (1536 units): recompute 616 -> 535 us
    // against the register variant.
    if (units <= 2 * cus || MODE == gdn::CHAIN_PLAIN)
      return launch(gdn::gdn_chain_ring_kernel<E, K, V, VARLEN, 2, MODE>, dim3(units / 2),
                    dim3(64 * gdn::RingCfg<E, K, V, 2>::WAVES), s, geo, wf, ktf, uf, gam, seq_slot,
                    seq_order, h0, fin, hcf, vnf);
  }
  // bf16, beyond the ring variant: two value tiles per wave while the waves
  // (one per SIMD) are all resident at once
  if constexpr (MODE == gdn::CHAIN_FULL && sizeof(E) == 2 && (V / 16) % 2 == 0) {
    if (units <= 8 * cus)
      return launch(gdn::gdn_chain2_kernel<E, K, V, VARLEN>, dim3(units / 2), dim3(64), s, geo, wf,
                    ktf, uf, gam, seq_slot, h0, fin, hcf, vnf);
  }
  return launch(gdn::gdn_chain_kernel<E, K, V, VARLEN, MODE>, dim3(units), dim3(64), s, geo, wf,
                ktf, uf, gam, seq_slot, h0, fin, hcf, vnf);
}

// The segment length a call uses on the current device (0: the plain state
// pass) and its segment count: seg_chunks as given, or the automatic choice.
struct SegRun {
  int L, nseg;
};
SegRun seg_run(const Plan& pl) {
  if (pl.seg_chunks > 0) return {pl.seg_chunks, pl.lay.num_segs};
  if (pl.seg_chunks != GDN_SEG_AUTO) return {0, 0};
  const gdn::Geo& g = pl.geo;
  const int L = auto_seg_chunks((int64_t)g.N * g.HV * (g.V / 16), g.NT, device_cus());
  if (L == 0) return {0, 0};
  return {L, g.N * ((g.NT + L - 1) / L)};  // at most the workspace's bound (L >= kAutoSegMin)
}

// Whether the output stage runs fused into the state pass (see
// gdn_fwd_fuses_output): bf16 without segments, and fp32 at K = 64 beyond one
// unit per CU.  The fused workgroup holds
// one value tile when the units fit one per CU, two beyond that (in several
// rounds beyond two per CU).  Measured on MI355X, ms per forward step, fused
// against the state pass and output kernels: B=1, T=65536, H=16, HV=32 (256
// units) 1.86 against 2.09; B=2, T=2048, H=8 (128 units) 0.0489 against
// 0.0492; B=4, T=8192, H=16 (512 units) 0.50 against 0.58; B=8, T=4096,
// H=16 (1024 units) 0.51 against 0.57; 12 packed sequences, T=32768, H=16
// (1536 units) 0.56 against 0.61.  The fused kernel drops the chunk states'
// and v_new's round trip through memory.  With one value tile per workgroup
// it lost while the output waves' Q operands were two 8-byte pieces in the
// kslot order (B=2, T=2048, H=8: 45 us against 33 us for the state pass and
// output); since H_c reaches them with k in natural order, each is one
// 16-byte load.
template <typename E, int K, int V>
bool fuses_output(const Plan& pl) {
  if constexpr (!gdn::ChainOutCfg<E, K, V, 2>::FITS) {
    return false;
  } else {
    const int64_t units = (int64_t)pl.geo.N * pl.geo.HV * (V / 16);
    if (seg_run(pl).L != 0 || units <= 0) return false;
    // fp32 (K = 64): fused only beyond one unit per CU, where the two-tile
    // workgroups share the chunk operands.  Measured: B=4, T=2048, H=HV=32,
    // K=V=64 (512 units) 0.277 -> 0.252 ms; B=2, T=4096 (256 units) 0.286 ->
    // 0.296 ms fused (not used); B=1, T=256, H=2 (8 units) 24.6 -> 24.5 us.
    return sizeof(E) == 2 || units > device_cus();
  }
}

// Value heads per output workgroup: 2 (sharing the key head's Q and K loads
// and its Q K^T product) when an even number of value heads read each key
// head and the per-(chunk, value head) workgroups would fill the device at
// least eight times over; at fewer, the longer per-workgroup chain adds
// latency that the shared work does not repay.  Measured on MI355X at B=1,
// T=65536, H=16, HV=32: output 567 -> 499 us.  The same sharing in WY (K K^T
// once per key head) needs ~210 VGPRs, which halves its occupancy: 737 ->
// 1089 us, so WY stays one workgroup per (chunk, value head).
int heads_per_workgroup(const Plan& pl) {
  const int64_t wgs = (int64_t)pl.geo.slots * pl.geo.HV;
  return (pl.geo.G % 2 == 0 && wgs >= 8 * (int64_t)device_cus()) ? 2 : 1;
}

template <typename E, int K, int V, bool VARLEN>
gdn_status_t run(const Plan& pl, const void* q, const void* k, const void* v, const float* g_raw,
                 const float* beta, const float* A_log, const float* dt_bias,
                 const int64_t* cu_seqlens, const float* h0, void* o, float* fin, void* ws,
                 hipStream_t s, void* const* events, unsigned mask) {
  using gdn::Frag;
  using gdn::Quad;
  const gdn::Geo& geo = pl.geo;
  const gdn_workspace_layout_t& L = pl.lay;
  char* w = static_cast<char*>(ws);
  float* gam = reinterpret_cast<float*>(w + L.gamma);
  float* bet = reinterpret_cast<float*>(w + L.beta);
  Frag<E>* wf = reinterpret_cast<Frag<E>*>(w + L.w);
  Frag<E>* ktf = reinterpret_cast<Frag<E>*>(w + L.kt);
  Quad<E>* uf = reinterpret_cast<Quad<E>*>(w + L.u);
  Frag<E>* hcf = reinterpret_cast<Frag<E>*>(w + L.hc);
  Frag<E>* vnf = reinterpret_cast<Frag<E>*>(w + L.vn);
  int4* cmap = VARLEN ? reinterpret_cast<int4*>(w + L.chunk_map) : nullptr;
  int* seq_slot = VARLEN ? reinterpret_cast<int*>(w + L.seq_slot) : nullptr;
  int* seq_order = VARLEN ? reinterpret_cast<int*>(w + L.seq_order) : nullptr;
  const E* qe = static_cast<const E*>(q);
  const E* ke = static_cast<const E*>(k);
  const E* ve = static_cast<const E*>(v);
  E* oe = static_cast<E*>(o);

  hipError_t err = hipSuccess;
  auto ok = [&](hipError_t e) {
    if (e != hipSuccess && err == hipSuccess) err = e;
  };
  auto mark = [&](int i) {
    if (events) ok(hipEventRecord(static_cast<hipEvent_t>(events[i]), s));
  };
  mark(0);
  const bool work = geo.N > 0;
  if (VARLEN && work && (mask & GDN_STAGE_CHUNK_MAP))
    ok(launch(gdn::gdn_chunk_map_kernel, dim3(1), dim3(256), s, cu_seqlens, geo.N, geo.T,
              geo.slots, cmap, seq_slot, seq_order));
  mark(1);
  const bool fused = fuses_output<E, K, V>(pl);
  const int gs = fused ? 1 : heads_per_workgroup(pl);
  Frag<E>* pmf = reinterpret_cast<Frag<E>*>(w + L.pm);
  if (work && geo.slots > 0 && (mask & GDN_STAGE_WY)) {
    bool done = false;
    if constexpr (gdn::ChainOutCfg<E, K, V, 2>::FITS) {
      if (fused) {
        // all workgroups resident at two per CU: the LDS-rich split variant
        if ((int64_t)geo.slots * geo.HV <= 2 * (int64_t)device_cus())
          ok(launch(gdn::gdn_wy_kernel<E, K, V, VARLEN, false, true, true>, dim3(geo.slots * geo.HV),
                    dim3(gdn::kWyThreads), s, geo, ke, ve, g_raw, beta, A_log, dt_bias, cmap, gam,
                    bet, wf, ktf, uf, nullptr, qe, pmf));
        else
          ok(launch(gdn::gdn_wy_kernel<E, K, V, VARLEN, false, true>, dim3(geo.slots * geo.HV),
                    dim3(gdn::kWyThreads), s, geo, ke, ve, g_raw, beta, A_log, dt_bias, cmap, gam,
                    bet, wf, ktf, uf, nullptr, qe, pmf));
        done = true;
      }
    }
    if (!done)
      ok(launch(gdn::gdn_wy_kernel<E, K, V, VARLEN>, dim3(geo.slots * geo.HV), dim3(gdn::kWyThreads),
                s, geo, ke, ve, g_raw, beta, A_log, dt_bias, cmap, gam, bet, wf, ktf, uf, nullptr,
                nullptr, nullptr));
  }
  mark(2);
  const unsigned so = GDN_STAGE_STATE | GDN_STAGE_OUTPUT;
  if (fused && (mask & so) == so) {
    // the state pass with the output stage in the same workgroups
    if constexpr (gdn::ChainOutCfg<E, K, V, 2>::FITS) {
      const int units = geo.N * geo.HV * (V / 16);
      if (work && units > 0 && units <= device_cus())
        ok(launch(gdn::gdn_chain_out_kernel<E, K, V, VARLEN, 1>, dim3(units),
                  dim3(64 * gdn::ChainOutCfg<E, K, V, 1>::WAVES), s, geo, wf, ktf, uf, gam,
                  seq_slot, seq_order, cmap, h0, fin, qe, pmf, oe));
      else if (work && units > 0)
        ok(launch(gdn::gdn_chain_out_kernel<E, K, V, VARLEN, 2>, dim3(units / 2),
                  dim3(64 * gdn::ChainOutCfg<E, K, V, 2>::WAVES), s, geo, wf, ktf, uf, gam,
                  seq_slot, seq_order, cmap, h0, fin, qe, pmf, oe));
    }
    mark(3);
    mark(4);
    return err == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
  }
  if (work && (mask & GDN_STAGE_STATE)) {
    const SegRun seg = seg_run(pl);
    if (seg.L > 0) {
      // segment-parallel: E_s and M_s per segment, start states in order, then
      // the full pass per segment from its start state
      int* seg_slot = reinterpret_cast<int*>(w + L.seg_slot);
      int* seq_seg = reinterpret_cast<int*>(w + L.seq_seg);
      float* seg_e = reinterpret_cast<float*>(w + L.seg_e);
      float* seg_m = reinterpret_cast<float*>(w + L.seg_m);
      float* seg_h = reinterpret_cast<float*>(w + L.seg_h);
      ok(launch(gdn::gdn_segment_map_kernel<VARLEN>, dim3(1), dim3(256), s, seq_slot, geo.N,
                geo.NT, seg.L, seg.nseg, seg_slot, seq_seg));
      gdn::Geo gs = geo;
      gs.N = seg.nseg;
      ok(launch_chain<E, K, V, true, gdn::CHAIN_END>(gs, s, wf, ktf, uf, gam, seg_slot, nullptr,
                                                     seg_e, hcf, vnf));
      ok(launch_chain<E, K, K, true, gdn::CHAIN_MAP>(gs, s, wf, ktf, uf, gam, seg_slot, nullptr,
                                                     seg_m, hcf, vnf));
      ok(launch(gdn::gdn_segment_combine_kernel<E, K, V>, dim3(geo.N * geo.HV * (V / 16)),
                dim3(64 * (K / 32)), s, geo, seq_seg, seg_m, seg_e, h0, fin, seg_h));
      ok(launch_chain<E, K, V, true, gdn::CHAIN_FULL>(gs, s, wf, ktf, uf, gam, seg_slot, seg_h,
                                                      nullptr, hcf, vnf));
    } else {
      ok(launch_chain<E, K, V, VARLEN, gdn::CHAIN_FULL>(geo, s, wf, ktf, uf, gam, seq_slot, h0,
                                                        fin, hcf, vnf, seq_order));
    }
  }
  mark(3);
  if (work && geo.slots > 0 && (mask & GDN_STAGE_OUTPUT)) {
    if (gs == 2)
      ok(launch(gdn::gdn_output_kernel<E, K, V, VARLEN, 2>, dim3(geo.slots * geo.HV / 2), dim3(256), s,
                geo, qe, ke, cmap, gam, hcf, vnf, oe));
    else
      ok(launch(gdn::gdn_output_kernel<E, K, V, VARLEN>, dim3(geo.slots * geo.HV), dim3(256), s, geo,
                qe, ke, cmap, gam, hcf, vnf, oe));
  }
  mark(4);
  return err == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <typename E, int K, int V>
gdn_status_t run_v(const Plan& pl, const void* q, const void* k, const void* v, const float* g_raw,
                   const float* beta, const float* A_log, const float* dt_bias,
                   const int64_t* cu, const float* h0, void* o, float* fin, void* ws, hipStream_t s,
                   void* const* ev, unsigned m) {
  return pl.varlen ? run<E, K, V, true>(pl, q, k, v, g_raw, beta, A_log, dt_bias, cu, h0, o, fin, ws, s, ev, m)
                   : run<E, K, V, false>(pl, q, k, v, g_raw, beta, A_log, dt_bias, cu, h0, o, fin, ws, s, ev, m);
}

template <typename E>
gdn_status_t run_e(const Plan& pl, const void* q, const void* k, const void* v, const float* g_raw,
                   const float* beta, const float* A_log, const float* dt_bias,
                   const int64_t* cu, const float* h0, void* o, float* fin, void* ws, hipStream_t s,
                   void* const* ev, unsigned m) {
  const int K = pl.geo.K, V = pl.geo.V;
  if (K == 128 && V == 128) return run_v<E, 128, 128>(pl, q, k, v, g_raw, beta, A_log, dt_bias, cu, h0, o, fin, ws, s, ev, m);
  if (K == 128 && V == 64) return run_v<E, 128, 64>(pl, q, k, v, g_raw, beta, A_log, dt_bias, cu, h0, o, fin, ws, s, ev, m);
  if (K == 64 && V == 128) return run_v<E, 64, 128>(pl, q, k, v, g_raw, beta, A_log, dt_bias, cu, h0, o, fin, ws, s, ev, m);
  return run_v<E, 64, 64>(pl, q, k, v, g_raw, beta, A_log, dt_bias, cu, h0, o, fin, ws, s, ev, m);
}

}  // namespace

// ---- backward ----
namespace {

// Workspace of the backward pass: the forward layout (without segments), then
// the backward's intermediates (see gdn_bwd.h for each one's type).
struct BwdLayout {
  size_t tmat, hcp, vnp, wtf, kdf, bq, dvl, dhn, dvn, dqp, dkp, dwp, dgp, dAp, dbp, total;
};

gdn_status_t make_bwd_plan(const gdn_params_t* p, bool varlen, Plan* pl, BwdLayout* bl) {
  if (!p) return GDN_ERR_NULL;
  gdn_params_t q = *p;
  q.seg_chunks = 0;
  gdn_status_t st = make_plan(&q, varlen, pl);
  if (st != GDN_OK) return st;
  // the key-head sum's grid: one workgroup per (slot, key head, 256 pieces)
  if ((int64_t)pl->geo.slots * p->H * (gdn::kChunk * p->K / 1024) > INT32_MAX) return GDN_ERR_UNSUPPORTED;
  // the WY backward addresses a chunk's token rows with 32-bit offsets
  if ((int64_t)gdn::kChunk * p->HV * p->V > INT32_MAX || (int64_t)gdn::kChunk * p->H * p->K > INT32_MAX)
    return GDN_ERR_UNSUPPORTED;
  const size_t hsl = (size_t)p->HV * (size_t)pl->geo.slots, C = gdn::kChunk, K = p->K, V = p->V;
  size_t off = pl->lay.total;
  const size_t esz = p->dtype == GDN_BF16 ? 2 : 4;
  auto take_n = [&](size_t& field, size_t n, size_t bytes) {
    field = off;
    off = align_up(off + hsl * n * bytes);
  };
  auto take = [&](size_t& field, size_t floats) { take_n(field, floats, 4); };
  // in the call's dtype: T, H_c, v_new, dH, dv_new, dw (see gdn_bwd.h)
  auto take_e = [&](size_t& field, size_t elems) { take_n(field, elems, esz); };
  take_e(bl->tmat, C * C);
  take_e(bl->hcp, K * V);
  take_e(bl->vnp, C * V);
  take(bl->wtf, K * C);  // fp32 size: also holds the dtype's fragments
  take(bl->kdf, C * K);
  take(bl->bq, K * V);
  take(bl->dvl, C * V);
  take_e(bl->dhn, K * V);
  take_e(bl->dvn, C * V);
  take(bl->dqp, C * K);
  take(bl->dkp, C * K);
  take_e(bl->dwp, C * K);
  take(bl->dgp, C);
  take(bl->dAp, 1);
  take(bl->dbp, 1);
  bl->total = off;
  return GDN_OK;
}

struct BwdArgs {
  const void *q, *k, *v;
  const float *g_raw, *beta, *A_log, *dt_bias;
  const int64_t* cu;
  const float* h0;
  const void* d_o;
  const float* dht;
  void *dq, *dk, *dv;
  float *dg_raw, *dbeta, *dA_log, *ddt_bias, *dh0;
};

gdn_status_t check_bwd(const gdn_params_t* p, const BwdArgs& a, const void* ws, size_t ws_bytes,
                       Plan* pl, BwdLayout* bl) {
  if (!p) return GDN_ERR_NULL;
  gdn_status_t st = make_bwd_plan(p, a.cu != nullptr, pl, bl);
  if (st != GDN_OK) return st;
  const bool tokens = pl->ntok > 0;
  if (tokens && (!a.q || !a.k || !a.v || !a.g_raw || !a.beta || !a.A_log || !a.d_o || !a.dq ||
                 !a.dk || !a.dv || !a.dg_raw || !a.dbeta))
    return GDN_ERR_NULL;
  if (!a.dA_log) return GDN_ERR_NULL;
  if (bl->total > 0 && !ws) return GDN_ERR_NULL;
  for (const void* x : {a.q, a.k, a.v, a.d_o, (const void*)a.dq, (const void*)a.dk, (const void*)a.dv})
    if (!aligned(x, 16)) return GDN_ERR_ALIGN;
  for (const void* x : {(const void*)a.g_raw, (const void*)a.beta, (const void*)a.A_log,
                        (const void*)a.dt_bias, (const void*)a.h0, (const void*)a.dht,
                        (const void*)a.dg_raw, (const void*)a.dbeta, (const void*)a.dA_log,
                        (const void*)a.ddt_bias, (const void*)a.dh0})
    if (!aligned(x, 4)) return GDN_ERR_ALIGN;
  if (!aligned(a.cu, 8) || !aligned(ws, kWsAlign)) return GDN_ERR_ALIGN;
  if (ws_bytes < bl->total) return GDN_ERR_WORKSPACE;
  return GDN_OK;
}

template <typename E, int K, int V, bool VARLEN>
gdn_status_t run_bwd(const Plan& pl, const BwdLayout& bl, const BwdArgs& a, void* ws,
                     hipStream_t s, void* const* events) {
  using gdn::Frag;
  using gdn::Quad;
  const gdn::Geo& geo = pl.geo;
  const gdn_workspace_layout_t& L = pl.lay;
  char* w = static_cast<char*>(ws);
  auto F = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  float* gam = F(L.gamma);
  float* bet = F(L.beta);
  Frag<E>* wf = reinterpret_cast<Frag<E>*>(w + L.w);
  Frag<E>* ktf = reinterpret_cast<Frag<E>*>(w + L.kt);
  Quad<E>* uf = reinterpret_cast<Quad<E>*>(w + L.u);
  int4* cmap = VARLEN ? reinterpret_cast<int4*>(w + L.chunk_map) : nullptr;
  int* seq_slot = VARLEN ? reinterpret_cast<int*>(w + L.seq_slot) : nullptr;
  int* seq_order = VARLEN ? reinterpret_cast<int*>(w + L.seq_order) : nullptr;
  auto FE = [&](size_t off) { return reinterpret_cast<Frag<E>*>(w + off); };
  auto EP = [&](size_t off) { return reinterpret_cast<E*>(w + off); };
  const E* qe = static_cast<const E*>(a.q);
  const E* ke = static_cast<const E*>(a.k);
  const E* ve = static_cast<const E*>(a.v);
  const E* doe = static_cast<const E*>(a.d_o);

  hipError_t err = hipSuccess;
  auto ok = [&](hipError_t e) {
    if (e != hipSuccess && err == hipSuccess) err = e;
  };
  auto mark = [&](int i) {
    if (events) ok(hipEventRecord(static_cast<hipEvent_t>(events[i]), s));
  };
  const unsigned chunk_wgs = (unsigned)geo.slots * geo.HV;
  const unsigned units = (unsigned)geo.N * geo.HV * (V / 16);
  mark(0);
  if (VARLEN && geo.N > 0)
    ok(launch(gdn::gdn_chunk_map_kernel, dim3(1), dim3(256), s, a.cu, geo.N, geo.T, geo.slots,
              cmap, seq_slot, seq_order));
  if (chunk_wgs > 0)
    ok(launch(gdn::gdn_wy_kernel<E, K, V, VARLEN, true>, dim3(chunk_wgs), dim3(gdn::kWyThreads), s, geo, ke, ve,
              a.g_raw, a.beta, a.A_log, a.dt_bias, cmap, gam, bet, wf, ktf, uf, EP(bl.tmat),
              nullptr, nullptr));
  if (units > 0 && geo.slots > 0)
    ok(launch_chain<E, K, V, VARLEN, gdn::CHAIN_PLAIN>(
        geo, s, wf, ktf, uf, gam, seq_slot, a.h0, nullptr, reinterpret_cast<Frag<E>*>(F(bl.hcp)),
        reinterpret_cast<Frag<E>*>(F(bl.vnp)), seq_order));
  mark(1);
  if (chunk_wgs > 0)
    {
      if constexpr (std::is_same<E, gdn::bf16>::value)
        ok(launch(gdn::gdn_bwd_prep_bf16_kernel<K, V, VARLEN>, dim3(chunk_wgs), dim3(gdn::kBwdThreads), s, geo,
                  qe, ke, doe, cmap, gam, wf, FE(bl.wtf), FE(bl.kdf),
                  reinterpret_cast<gdn::Quad<E>*>(w + bl.bq), reinterpret_cast<gdn::f32x4*>(w + bl.dvl)));
      else
        ok(launch(gdn::gdn_bwd_prep_kernel<E, K, V, VARLEN>, dim3(chunk_wgs), dim3(gdn::kBwdThreads), s, geo, qe,
                  ke, doe, cmap, gam, wf, FE(bl.wtf), FE(bl.kdf), reinterpret_cast<gdn::Quad<E>*>(w + bl.bq),
                  reinterpret_cast<gdn::f32x4*>(w + bl.dvl)));
    }
  mark(2);
  if (units > 0 && (units <= device_cus() || sizeof(E) == 2))
    // the K rows split over K/32 waves: one unit per CU or fewer, and bf16 at
    // any unit count (about four workgroups per CU, in rounds beyond that,
    // packed sequences longest first).  Measured on MI355X beyond one unit
    // per CU against one wave per unit: 12 packed sequences, T=32768, H=16
    // 553 -> 486 us (index order); B=4, T=8192, H=16 428 -> 409 us.
    ok(launch(gdn::gdn_bwd_chain_ks_kernel<E, K, V, VARLEN, 2>, dim3(units), dim3(64 * (K / 32)), s, geo,
              FE(bl.kdf), reinterpret_cast<const gdn::f32x4*>(w + bl.dvl), FE(bl.wtf),
              reinterpret_cast<const gdn::Quad<E>*>(w + bl.bq), gam, seq_slot, seq_order, a.dht, a.dh0,
              EP(bl.dhn), EP(bl.dvn)));
  else if (units > 0)
    ok(launch(gdn::gdn_bwd_chain_kernel<E, K, V, VARLEN>, dim3(units), dim3(64), s, geo,
              FE(bl.kdf), reinterpret_cast<const gdn::f32x4*>(w + bl.dvl), FE(bl.wtf),
              reinterpret_cast<const gdn::Quad<E>*>(w + bl.bq), gam, seq_slot, a.dht, a.dh0,
              EP(bl.dhn), EP(bl.dvn)));
  mark(3);
  if (chunk_wgs > 0) {
    // bf16 calls take the bf16-MFMA variant, fp32 calls the fp32 one
    if constexpr (std::is_same<E, gdn::bf16>::value)
      ok(launch(gdn::gdn_bwd_dqk_bf16_kernel<K, V, VARLEN>, dim3(chunk_wgs), dim3(gdn::kBwdThreads), s, geo,
                qe, ke, doe, cmap, gam, EP(bl.vnp), EP(bl.dvn), EP(bl.hcp), EP(bl.dhn), F(bl.dqp),
                F(bl.dkp), EP(bl.dwp), F(bl.dgp), static_cast<E*>(a.dq)));
    else
      ok(launch(gdn::gdn_bwd_dqk_kernel<E, K, V, VARLEN>, dim3(chunk_wgs), dim3(gdn::kBwdThreads), s, geo, qe,
                ke, doe, cmap, gam, F(bl.vnp), F(bl.dvn), F(bl.hcp), F(bl.dhn), F(bl.dqp), F(bl.dkp),
                F(bl.dwp), F(bl.dgp), static_cast<E*>(a.dq)));
  }
  mark(4);
  if (chunk_wgs > 0) {
    if constexpr (std::is_same<E, gdn::bf16>::value)
      ok(launch(gdn::gdn_bwd_wy_bf16_kernel<K, V, VARLEN>, dim3(chunk_wgs), dim3(gdn::kBwdThreads), s,
                geo, ke, ve, a.g_raw, a.A_log, a.dt_bias, cmap, gam, bet, EP(bl.tmat), EP(bl.dwp),
                EP(bl.dvn), F(bl.dgp), F(bl.dkp), static_cast<E*>(a.dv), a.dbeta, a.dg_raw,
                F(bl.dAp), F(bl.dbp), static_cast<E*>(a.dk)));
    else
      ok(launch(gdn::gdn_bwd_wy_kernel<E, K, V, VARLEN>, dim3(chunk_wgs), dim3(gdn::kBwdThreads), s, geo, ke,
                ve, a.g_raw, a.A_log, a.dt_bias, cmap, gam, bet, F(bl.tmat), F(bl.dwp), F(bl.dvn),
                F(bl.dgp), F(bl.dkp), static_cast<E*>(a.dv), a.dbeta, a.dg_raw, F(bl.dAp),
                F(bl.dbp), static_cast<E*>(a.dk)));
  }
  mark(5);
  if (geo.slots > 0 && geo.G > 1)
    ok(launch(gdn::gdn_bwd_qk_sum_kernel<E, K, VARLEN>,
              dim3((unsigned)geo.slots * geo.H * gdn::qk_sum_parts<K>()), dim3(256), s, geo, cmap,
              F(bl.dqp), F(bl.dkp), static_cast<E*>(a.dq), static_cast<E*>(a.dk)));
  ok(launch(gdn::gdn_bwd_param_kernel, dim3(geo.HV), dim3(256), s, geo, F(bl.dAp), F(bl.dbp),
            a.dA_log, a.ddt_bias));
  mark(6);
  return err == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <typename E>
gdn_status_t run_bwd_e(const Plan& pl, const BwdLayout& bl, const BwdArgs& a, void* ws,
                       hipStream_t s, void* const* ev) {
  const int kv = pl.geo.K * 1000 + pl.geo.V;
  if (pl.varlen) {
    if (kv == 128128) return run_bwd<E, 128, 128, true>(pl, bl, a, ws, s, ev);
    if (kv == 128064) return run_bwd<E, 128, 64, true>(pl, bl, a, ws, s, ev);
    if (kv == 64128) return run_bwd<E, 64, 128, true>(pl, bl, a, ws, s, ev);
    return run_bwd<E, 64, 64, true>(pl, bl, a, ws, s, ev);
  }
  if (kv == 128128) return run_bwd<E, 128, 128, false>(pl, bl, a, ws, s, ev);
  if (kv == 128064) return run_bwd<E, 128, 64, false>(pl, bl, a, ws, s, ev);
  if (kv == 64128) return run_bwd<E, 64, 128, false>(pl, bl, a, ws, s, ev);
  return run_bwd<E, 64, 64, false>(pl, bl, a, ws, s, ev);
}

}  // namespace

namespace {
bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t elem_size(gdn_dtype_t t) { return t == GDN_F32 ? 4 : 2; }

template <typename TI, typename TO>
gdn_status_t kda_launch(const void* g, const float* A_log, const float* dt_bias, void* yg,
                        int64_t T, int H, int D, hipStream_t s) {
  const TI* gi = static_cast<const TI*>(g);
  TO* yo = static_cast<TO*>(yg);
  const int64_t rows = T * H;
  const int64_t cap = (int64_t)device_cus() * 32;  // grid-stride beyond ~32 workgroups per CU
  hipError_t e;
  if (D % 8 == 0 && D <= 8 * 256 && aligned_to(g, 16) && aligned_to(yg, 16) &&
      (!dt_bias || aligned_to(dt_bias, 16))) {
    const int rows_per_wg = 256 / (D / 8);
    const int64_t blocks = std::min<int64_t>((rows + rows_per_wg - 1) / rows_per_wg, cap);
    e = launch(gdn::gdn_kda_gate_vec_kernel<TI, TO>, dim3((unsigned)blocks), dim3(256), s, gi,
               A_log, dt_bias, yo, rows, H, D);
  } else {
    const int64_t n = rows * D;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, cap);
    e = launch(gdn::gdn_kda_gate_scalar_kernel<TI, TO>, dim3((unsigned)blocks), dim3(256), s, gi,
               A_log, dt_bias, yo, n, H, D);
  }
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <typename TI>
gdn_status_t kda_out(const void* g, const float* A_log, const float* dt_bias, void* yg,
                     gdn_dtype_t yt, int64_t T, int H, int D, hipStream_t s) {
  if (yt == GDN_F32) return kda_launch<TI, float>(g, A_log, dt_bias, yg, T, H, D, s);
  if (yt == GDN_BF16) return kda_launch<TI, gdn::bf16>(g, A_log, dt_bias, yg, T, H, D, s);
  return kda_launch<TI, gdn::f16>(g, A_log, dt_bias, yg, T, H, D, s);
}
}  // namespace

extern "C" {

size_t gdn_fwd_workspace_size(const gdn_params_t* p, int packed) {
  Plan pl;
  if (!p) return 0;
  return make_plan(p, packed != 0, &pl) == GDN_OK ? pl.lay.total : 0;
}

gdn_status_t gdn_fwd_workspace_layout(const gdn_params_t* p, int packed,
                                      gdn_workspace_layout_t* out) {
  if (!p || !out) return GDN_ERR_NULL;
  Plan pl;
  gdn_status_t st = make_plan(p, packed != 0, &pl);
  if (st == GDN_OK) *out = pl.lay;
  return st;
}

gdn_status_t gdn_fwd_fuses_output(const gdn_params_t* p, int packed, int32_t* fused) {
  if (!p || !fused) return GDN_ERR_NULL;
  Plan pl;
  gdn_status_t st = make_plan(p, packed != 0, &pl);
  if (st != GDN_OK) return st;
  bool f;
  const bool bf = p->dtype == GDN_BF16;
  if (p->K == 128 && p->V == 128) f = bf ? fuses_output<gdn::bf16, 128, 128>(pl) : fuses_output<float, 128, 128>(pl);
  else if (p->K == 128 && p->V == 64) f = bf ? fuses_output<gdn::bf16, 128, 64>(pl) : fuses_output<float, 128, 64>(pl);
  else if (p->K == 64 && p->V == 128) f = bf ? fuses_output<gdn::bf16, 64, 128>(pl) : fuses_output<float, 64, 128>(pl);
  else f = bf ? fuses_output<gdn::bf16, 64, 64>(pl) : fuses_output<float, 64, 64>(pl);
  *fused = f ? 1 : 0;
  return GDN_OK;
}

gdn_status_t gdn_fwd_seg_chunks(const gdn_params_t* p, int packed, int32_t* seg_chunks) {
  if (!p || !seg_chunks) return GDN_ERR_NULL;
  Plan pl;
  gdn_status_t st = make_plan(p, packed != 0, &pl);
  if (st != GDN_OK) return st;
  *seg_chunks = seg_run(pl).L;
  return GDN_OK;
}

gdn_status_t gdn_fwd_check(const gdn_params_t* p, const void* q, const void* k, const void* v,
                           const float* g_raw, const float* beta, const float* A_log,
                           const float* dt_bias, const int64_t* cu_seqlens,
                           const float* initial_state, const void* o, const float* final_state,
                           const void* workspace, size_t workspace_bytes) {
  Plan pl;
  return check_all(p, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, o,
                   final_state, workspace, workspace_bytes, &pl);
}

namespace {
gdn_status_t fwd_entry(const gdn_params_t* p, const void* q, const void* k, const void* v,
                       const float* g_raw, const float* beta, const float* A_log,
                       const float* dt_bias, const int64_t* cu_seqlens, const float* initial_state,
                       void* o, float* final_state, void* workspace, size_t workspace_bytes,
                       void* stream, void* const* events, unsigned mask) {
  Plan pl;
  gdn_status_t st = check_all(p, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state,
                              o, final_state, workspace, workspace_bytes, &pl);
  if (st != GDN_OK) return st;
  if (mask & ~GDN_STAGE_ALL) return GDN_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->dtype == GDN_BF16)
    return run_e<gdn::bf16>(pl, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, o,
                            final_state, workspace, s, events, mask);
  return run_e<float>(pl, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, o,
                      final_state, workspace, s, events, mask);
}
}  // namespace

gdn_status_t gdn_fwd_timed(const gdn_params_t* p, const void* q, const void* k, const void* v,
                           const float* g_raw, const float* beta, const float* A_log,
                           const float* dt_bias, const int64_t* cu_seqlens,
                           const float* initial_state, void* o, float* final_state,
                           void* workspace, size_t workspace_bytes, void* stream,
                           void* const* events) {
  return fwd_entry(p, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, o,
                   final_state, workspace, workspace_bytes, stream, events, GDN_STAGE_ALL);
}

gdn_status_t gdn_fwd_stages(const gdn_params_t* p, const void* q, const void* k, const void* v,
                            const float* g_raw, const float* beta, const float* A_log,
                            const float* dt_bias, const int64_t* cu_seqlens,
                            const float* initial_state, void* o, float* final_state,
                            void* workspace, size_t workspace_bytes, unsigned stage_mask,
                            void* stream) {
  return fwd_entry(p, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, o,
                   final_state, workspace, workspace_bytes, stream, nullptr, stage_mask);
}

gdn_status_t gdn_fwd(const gdn_params_t* p, const void* q, const void* k, const void* v,
                     const float* g_raw, const float* beta, const float* A_log,
                     const float* dt_bias, const int64_t* cu_seqlens, const float* initial_state,
                     void* o, float* final_state, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return gdn_fwd_timed(p, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, o,
                       final_state, workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

// Workspace of gdn_fwd_noalloc: one static array per device, loaded with the
// code object and held until the process ends.  Host code must never pass the
// name `scratch` itself to a kernel or a copy (in host code it is only a
// stand-in, not a device address): it uses the per-device address that
// hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[GDN_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mu;

// The device address of the current device's scratch array, looked up once
// per device (with that device current) and cached; nullptr on failure.
void* current_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = scratch_addr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  ptr = scratch_addr[dev].load(std::memory_order_relaxed);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  scratch_addr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

extern "C" {

gdn_status_t gdn_fwd_noalloc(const gdn_params_t* p, const void* q, const void* k, const void* v,
                             const float* g_raw, const float* beta, const float* A_log,
                             const float* dt_bias, const int64_t* cu_seqlens,
                             const float* initial_state, void* o, float* final_state,
                             void* stream) {
  Plan pl;
  if (!p) return GDN_ERR_NULL;
  gdn_status_t st = make_plan(p, cu_seqlens != nullptr, &pl);
  if (st != GDN_OK) return st;
  if (pl.lay.total > (size_t)GDN_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
  // the remaining argument checks, with a stand-in for the workspace (aligned,
  // large enough; never dereferenced) so that nothing touches the GPU before
  // every argument has passed
  st = check_all(p, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, o,
                 final_state, reinterpret_cast<const void*>(uintptr_t{kWsAlign}),
                 GDN_SCRATCH_BYTES, &pl);
  if (st != GDN_OK) return st;
  void* ws = current_scratch();
  if (!ws) return GDN_ERR_LAUNCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->dtype == GDN_BF16)
    return run_e<gdn::bf16>(pl, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, o,
                            final_state, ws, s, nullptr, GDN_STAGE_ALL);
  return run_e<float>(pl, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, o,
                      final_state, ws, s, nullptr, GDN_STAGE_ALL);
}

gdn_status_t gdn_decode(const gdn_params_t* p, const void* q, const void* k, const void* v,
                        const float* g_raw, const float* beta, const float* A_log,
                        const float* dt_bias, float* state, void* o, void* stream) {
  if (!p) return GDN_ERR_NULL;
  if (p->num_seqs != 0) return GDN_ERR_SHAPE;
  Plan pl;
  gdn_status_t st = make_plan(p, false, &pl);
  if (st != GDN_OK) return st;
  if (!state) return GDN_ERR_NULL;
  const bool tokens = (int64_t)p->B * p->T > 0;
  if (tokens && (!q || !k || !v || !g_raw || !beta || !A_log || !o)) return GDN_ERR_NULL;
  if (!aligned_to(q, 16) || !aligned_to(k, 16) || !aligned_to(v, 16) || !aligned_to(o, 16) ||
      !aligned_to(g_raw, 4) || !aligned_to(beta, 4) || !aligned_to(A_log, 4) ||
      !aligned_to(dt_bias, 4) || !aligned_to(state, 4))
    return GDN_ERR_ALIGN;
  if (!tokens) return GDN_OK;
  const gdn::Geo& geo = pl.geo;
  const dim3 grid((unsigned)((int64_t)p->B * p->HV * (p->V / 64)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  auto go = [&](auto kern, auto* tag) {
    using E = std::remove_pointer_t<decltype(tag)>;
    return launch(kern, grid, dim3(256), s, geo, static_cast<const E*>(q),
                  static_cast<const E*>(k), static_cast<const E*>(v), g_raw, beta, A_log, dt_bias,
                  state, static_cast<E*>(o));
  };
  const int kv = p->K * 1000 + p->V;
  if (p->dtype == GDN_BF16) {
    gdn::bf16* tag = nullptr;
    e = kv == 128128 ? go(gdn::gdn_decode_kernel<gdn::bf16, 128, 128>, tag)
      : kv == 128064 ? go(gdn::gdn_decode_kernel<gdn::bf16, 128, 64>, tag)
      : kv == 64128  ? go(gdn::gdn_decode_kernel<gdn::bf16, 64, 128>, tag)
                     : go(gdn::gdn_decode_kernel<gdn::bf16, 64, 64>, tag);
  } else {
    float* tag = nullptr;
    e = kv == 128128 ? go(gdn::gdn_decode_kernel<float, 128, 128>, tag)
      : kv == 128064 ? go(gdn::gdn_decode_kernel<float, 128, 64>, tag)
      : kv == 64128  ? go(gdn::gdn_decode_kernel<float, 64, 128>, tag)
                     : go(gdn::gdn_decode_kernel<float, 64, 64>, tag);
  }
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status_t gdn_kda_gate(const void* g, gdn_dtype_t g_dtype_arg, const float* A_log,
                          const float* dt_bias, void* yg, gdn_dtype_t yg_dtype_arg, int64_t T,
                          int32_t H, int32_t D, void* stream) {
  if (T < 0 || H < 1 || D < 1) return GDN_ERR_SHAPE;
  if ((int64_t)H * D > INT64_MAX / (T > 0 ? T : 1)) return GDN_ERR_SHAPE;
  auto known = [](int t) { return t == GDN_F32 || t == GDN_BF16 || t == GDN_F16; };
  if (!known(enum_bits(g_dtype_arg)) || !known(enum_bits(yg_dtype_arg))) return GDN_ERR_DTYPE;
  const gdn_dtype_t g_dtype = g_dtype_arg, yg_dtype = yg_dtype_arg;  // now in range
  if (T == 0) return GDN_OK;
  if (!g || !A_log || !yg) return GDN_ERR_NULL;
  if (!aligned_to(g, elem_size(g_dtype)) || !aligned_to(yg, elem_size(yg_dtype)) ||
      !aligned_to(A_log, 4) || (dt_bias && !aligned_to(dt_bias, 4)))
    return GDN_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g_dtype == GDN_F32) return kda_out<float>(g, A_log, dt_bias, yg, yg_dtype, T, H, D, s);
  if (g_dtype == GDN_BF16) return kda_out<gdn::bf16>(g, A_log, dt_bias, yg, yg_dtype, T, H, D, s);
  return kda_out<gdn::f16>(g, A_log, dt_bias, yg, yg_dtype, T, H, D, s);
}

size_t gdn_bwd_workspace_size(const gdn_params_t* p, int packed) {
  Plan pl;
  BwdLayout bl;
  if (!p) return 0;
  return make_bwd_plan(p, packed != 0, &pl, &bl) == GDN_OK ? bl.total : 0;
}

gdn_status_t gdn_bwd_timed(const gdn_params_t* p, const void* q, const void* k, const void* v,
                           const float* g_raw, const float* beta, const float* A_log,
                           const float* dt_bias, const int64_t* cu_seqlens,
                           const float* initial_state, const void* d_o,
                           const float* d_final_state, void* dq, void* dk, void* dv,
                           float* dg_raw, float* dbeta, float* dA_log, float* ddt_bias,
                           float* d_initial_state, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* events) {
  const BwdArgs a{q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, d_o,
                  d_final_state, dq, dk, dv, dg_raw, dbeta, dA_log, ddt_bias, d_initial_state};
  Plan pl;
  BwdLayout bl;
  gdn_status_t st = check_bwd(p, a, workspace, workspace_bytes, &pl, &bl);
  if (st != GDN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->dtype == GDN_BF16) return run_bwd_e<gdn::bf16>(pl, bl, a, workspace, s, events);
  return run_bwd_e<float>(pl, bl, a, workspace, s, events);
}

gdn_status_t gdn_bwd(const gdn_params_t* p, const void* q, const void* k, const void* v,
                     const float* g_raw, const float* beta, const float* A_log,
                     const float* dt_bias, const int64_t* cu_seqlens, const float* initial_state,
                     const void* d_o, const float* d_final_state, void* dq, void* dk, void* dv,
                     float* dg_raw, float* dbeta, float* dA_log, float* ddt_bias,
                     float* d_initial_state, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return gdn_bwd_timed(p, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, d_o,
                       d_final_state, dq, dk, dv, dg_raw, dbeta, dA_log, ddt_bias,
                       d_initial_state, workspace, workspace_bytes, stream, nullptr);
}

const char* gdn_status_string(gdn_status_t s) {
  switch (enum_bits(s)) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "invalid shape";
    case GDN_ERR_DTYPE: return "unsupported dtype";
    case GDN_ERR_UNSUPPORTED: return "unsupported size (K and V must be 64 or 128)";
    case GDN_ERR_ALIGN: return "misaligned pointer";
    case GDN_ERR_WORKSPACE: return "workspace too small";
    case GDN_ERR_LAUNCH: return "kernel launch failed";
    case GDN_ERR_SCRATCH: return "problem too large for the static scratch (GDN_SCRATCH_BYTES)";
  }
  return "unknown status";
}

}  // extern "C"
