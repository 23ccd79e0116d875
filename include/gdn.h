/*
 * gdn.h -- C ABI of libgdn, the MI355X (gfx950) Gated DeltaNet chunkwise
 * forward pass.
 *
 * The operation.  For every sequence and value head the library evaluates the
 * gated delta rule (the "stateful linear recurrent layer" of the Ascend GDN
 * blog, section "GDN sequence structure and Triton introduction": linear
 * attention + gating + the delta rule, one fixed-size state per head updated
 * token by token):
 *
 *     g_t = -exp(A_log[hv]) * softplus(g_raw_t + dt_bias[hv])
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * The gate is the per-head scalar case of the KDA gate guide (MindSpeed-Ops
 * issue page, "core computation logic"), softplus(x) = x for x > 20 and
 * log(1 + exp(x)) otherwise, evaluated in fp32 ("numerical stability": fp32
 * inside, cast at the output).  The state S_t (V x K) is exposed as its
 * transpose H = S^T: initial_state / final_state are [N][HV][K][V] fp32 with
 * element [n][hv][i][j] = S[j][i].
 *
 * It is computed chunkwise (chunks of 64 tokens, aligned to every sequence
 * start, last chunk of a sequence possibly shorter) by three gfx950 kernels
 * on the caller's stream: the per-chunk WY representation, which first runs
 * the gate prologue and chunk-local cumsum and writes them stride-1 along T
 * (the layout fix of the G_T_CONTIG page, "fix: host transpose + stride-1
 * pointer", done inside the kernel instead of on the host), the sequential
 * inter-chunk state pass, and the chunk output.  For bf16 without segments
 * (and fp32 at K = 64 with many units) the output runs inside the state-pass
 * kernel (gdn_fwd_fuses_output), so a call is two kernels.  One more kernel
 * builds the chunk map when cu_seqlens is given.
 *
 * Segment-parallel state pass (seg_chunks > 0).  The chunk update is affine in
 * the state, H_next = M_c H + B_c (M_c = e^{G_last} I - kd^T w), so a run of
 * L = seg_chunks chunks composes to H_end = M_s H_start + E_s.  With segments,
 * the state pass runs in three levels:
 *   1. for every segment of every sequence, in parallel, E_s (its end state
 *      from a zero start) and M_s (its K x K linear map, the same pass run
 *      with u = 0 from the identity);
 *   2. per sequence, in segment order, H_start(s+1) = M_s H_start(s) + E_s,
 *      from the initial state; the last one is the final state;
 *   3. every segment again from its true start state, writing the chunk
 *      states the output kernel reads.
 * It does about three times the state-pass work, in sequential runs L chunks
 * long instead of a whole sequence: worth it only when a few long sequences
 * leave most CUs idle.  Measured on MI355X at B=1, T=65536, K=V=128 bf16, with
 * U (sequence, value head, 16-column) units: U = 16, L = 32: state pass 530 ->
 * 225 us; U = 32, L = 64: 722 -> 326 us; U = 64, L = 128: 772 -> 387 us.  At
 * U = 256 (HV = 32) and at B=2, T=2048, HV=8 it is slower than the plain pass.
 * Same results as the plain pass up to rounding; M_s H is evaluated with
 * operands in the call's dtype (bf16 for bf16 calls).
 *
 * seg_chunks = GDN_SEG_AUTO chooses per call, from the shape and the current
 * device's compute-unit count (CUs): with NS = floor(2 CUs / U) (two units per
 * CU in the segment passes), segments of L = max(ceil(NT / NS), 16) chunks
 * (NT = chunks per sequence) when NS >= 8 and NT / L >= 8, else the plain pass
 * (also for packed sequences, whose lengths are not known on the host).  The
 * workspace is sized for the shortest segment it may choose (16 chunks);
 * gdn_fwd_seg_chunks reports the choice.
 *
 * Layouts (all contiguous, row-major, device memory):
 *   q, k           [B][T][H][K]   dtype (GDN_BF16 or GDN_F32)
 *   v              [B][T][HV][V]  dtype
 *   g_raw, beta    [B][T][HV]     fp32 (beta already in (0,1); no activation applied)
 *   A_log          [HV]           fp32
 *   dt_bias        [HV]           fp32, may be NULL (treated as 0)
 *   cu_seqlens     [N+1]          int64, may be NULL; see below
 *   initial_state  [N][HV][K][V]  fp32, may be NULL (zero state)
 *   o              [B][T][HV][V]  dtype (written)
 *   final_state    [N][HV][K][V]  fp32, may be NULL (written)
 *   workspace      gdn_fwd_workspace_size() bytes, 256-byte aligned
 * Value head hv reads query/key head hv / (HV/H).
 *
 * Packed sequences (the G_T_CONTIG page, "varlen checklist"): with cu_seqlens
 * given, B must be 1, T is the packed total, and sequence n covers tokens
 * cu_seqlens[n] .. cu_seqlens[n+1]-1.  Offsets are int64.  Precondition
 * (not checked, to avoid a device-to-host sync): cu_seqlens[0] == 0,
 * cu_seqlens[N] == T, non-decreasing.  Offsets that break it are clamped on the
 * device so that no access leaves the buffers; the results are then undefined.
 * Empty sequences are allowed (final state = initial state).  N = 0 is
 * allowed only with T = 0 (GDN_ERR_SHAPE otherwise: tokens with no sequence to
 * hold them).
 *
 * Ownership.  The caller owns every buffer.  The library never allocates,
 * frees or synchronizes; gdn_fwd only enqueues kernels on `stream` (a
 * hipStream_t, NULL = default stream) and returns.  It keeps no global mutable
 * state and may be called concurrently on different streams with different
 * workspaces.  Outputs and workspace must not overlap any input.
 *
 * Errors.  gdn_fwd validates every argument on the host first (the same checks
 * as gdn_fwd_check); on failure it returns the status and enqueues nothing.
 * A failed kernel launch returns GDN_ERR_LAUNCH.  Nothing is printed, thrown
 * or aborted across the ABI.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL */
  GDN_ERR_SHAPE = 2,       /* negative size, HV % H != 0, cu_seqlens with B != 1, seg_chunks < 0, ... */
  GDN_ERR_DTYPE = 3,       /* dtype not supported by the entry point */
  GDN_ERR_UNSUPPORTED = 4, /* K or V not in {64, 128}, or a size beyond the int32 index range */
  GDN_ERR_ALIGN = 5,       /* a pointer is not aligned as required below */
  GDN_ERR_WORKSPACE = 6,   /* workspace smaller than gdn_fwd_workspace_size() */
  GDN_ERR_LAUNCH = 7,      /* a kernel launch failed */
  GDN_ERR_SCRATCH = 8      /* gdn_fwd_noalloc: workspace beyond GDN_SCRATCH_BYTES */
} gdn_status_t;

/* Element types.  gdn_fwd takes GDN_F32 or GDN_BF16; the KDA gate takes all three. */
typedef enum { GDN_F32 = 0, GDN_BF16 = 1, GDN_F16 = 2 } gdn_dtype_t;

typedef struct {
  int32_t B;        /* sequences (fixed length), or 1 with cu_seqlens */
  int32_t T;        /* tokens per sequence, or the packed total with cu_seqlens */
  int32_t H;        /* query/key heads */
  int32_t HV;       /* value heads, a multiple of H */
  int32_t K;        /* key/query head dim: 64 or 128 */
  int32_t V;        /* value head dim: 64 or 128 */
  int32_t num_seqs; /* N with cu_seqlens; ignored (N = B) without */
  int32_t dtype;    /* gdn_dtype_t of q, k, v and o */
  float scale;      /* multiplies every o_t; 1.0 gives o_t = S_t q_t */
  int32_t seg_chunks; /* 0: plain state pass; L > 0: segments of L chunks;
                         GDN_SEG_AUTO: chosen per call (see above) */
} gdn_params_t;

/* seg_chunks value: let the library choose the segment length (see above). */
#define GDN_SEG_AUTO (-1)

/* Byte offsets of the intermediates inside the workspace, for inspection.
 * Every per-chunk buffer is indexed by a chunk slot: slot = n*ceil(T/64) + c
 * without cu_seqlens, or the position of the chunk in sequence order with
 * cu_seqlens (num_slots = floor(T/64) + N is an upper bound there).
 *   gamma [HV][num_slots][64] fp32  chunk-local cumsum of g, times log2(e)
 *   beta  [HV][num_slots][64] fp32  beta in the same layout (0 past a chunk's end)
 *   w, kt, u, hc, vn, pm             MFMA-fragment-ordered dtype tensors (see
 *                                    the kernel sources for the lane order);
 *                                    pm holds the masked, decayed Q K^T of every
 *                                    chunk, written only when the output stage is
 *                                    fused into the state pass (below), which then
 *                                    leaves hc and vn unwritten
 *   chunk_map [num_slots] int32x4, seq_slot [N+1] int32, seq_order [N] int32
 *                                    (cu_seqlens only; seq_order: the sequences
 *                                    by decreasing chunk count, the order in
 *                                    which the fused state pass starts them)
 * With seg_chunks > 0 (num_segs = an upper bound on the segment count):
 *   seg_slot [num_segs+1] int32    first slot of each segment, sequence order
 *   seq_seg  [N+1] int32           first segment of each sequence
 *   seg_e, seg_h [num_segs][HV][K][V] fp32   E_s, and the start states
 *   seg_m    [num_segs][HV][K][K] fp32        M_s
 * (their offsets are 0 and num_segs is 0 without segments). */
typedef struct {
  size_t gamma, beta, w, kt, u, hc, vn, pm, chunk_map, seq_slot, seq_order;
  size_t seg_slot, seq_seg, seg_e, seg_m, seg_h, total;
  int32_t num_slots;
  int32_t num_seqs;
  int32_t num_segs;
} gdn_workspace_layout_t;

/* Workspace bytes gdn_fwd needs for these parameters (0 if they are invalid).
 * `packed` != 0 for a call that will pass cu_seqlens.  Pure host function. */
size_t gdn_fwd_workspace_size(const gdn_params_t *p, int packed);

/* Fill *out with the workspace layout (`packed` as above).  Pure host function. */
gdn_status_t gdn_fwd_workspace_layout(const gdn_params_t *p, int packed,
                                      gdn_workspace_layout_t *out);

/* Validate a gdn_fwd call without touching the GPU or dereferencing any device
 * pointer: sizes, dtype, NULL-ness and alignment (q, k, v, o: 16 bytes;
 * g_raw, beta, A_log, dt_bias, initial_state, final_state: 4 bytes;
 * cu_seqlens: 8 bytes; workspace: 256 bytes) and workspace_bytes.  These are
 * the checks the KDA gate guide's API layer makes with asserts on ndim, shape
 * and element count before it dispatches (MindSpeed-Ops issue page, "API
 * layer"), returned here as status codes; the packed-sequence rules are those
 * of the G_T_CONTIG page, "varlen checklist".  gdn_fwd runs the same checks
 * first and enqueues nothing when one fails. */
gdn_status_t gdn_fwd_check(const gdn_params_t *p, const void *q, const void *k,
                           const void *v, const float *g_raw, const float *beta,
                           const float *A_log, const float *dt_bias,
                           const int64_t *cu_seqlens, const float *initial_state,
                           const void *o, const float *final_state,
                           const void *workspace, size_t workspace_bytes);

/* The forward pass (see the top of this file).  Enqueues the kernels on
 * `stream` (hipStream_t) and returns without waiting. */
gdn_status_t gdn_fwd(const gdn_params_t *p, const void *q, const void *k, const void *v,
                     const float *g_raw, const float *beta, const float *A_log,
                     const float *dt_bias, const int64_t *cu_seqlens,
                     const float *initial_state, void *o, float *final_state,
                     void *workspace, size_t workspace_bytes, void *stream);

/* ---- Forward pass without any allocation -------------------------------------
 * For callers that cannot allocate device memory at all (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): gdn_fwd with
 * the same arguments and results (the same kernels, bit for bit), but without
 * a workspace argument.  Its intermediates live in a static device array of
 * GDN_SCRATCH_BYTES per GPU, part of the library's code object: every GPU the
 * library runs on holds it until the process ends.  Its device address is
 * looked up on the first call on each device (hipGetSymbolAddress, with that
 * device current); the call itself allocates and frees nothing.
 *   Limit: gdn_fwd_workspace_size(p, cu_seqlens != NULL) <= GDN_SCRATCH_BYTES
 *   (64 MiB: e.g. B=2, T=2048, H=HV=8, K=V=128 bf16 needs 52.25 MiB); a larger
 *   problem returns GDN_ERR_SCRATCH and enqueues nothing.
 *   Sharing: all calls on one GPU use that GPU's one array, and each call
 *   leaves its intermediates there.  No part of it needs to start zeroed (each
 *   call writes every intermediate before reading it).  Calls that overlap in
 *   time on one GPU (on different streams, or from different host threads
 *   without ordering) race on it and give undefined results; serialize them,
 *   e.g. on one stream.
 * Errors: those of gdn_fwd (checked before anything is enqueued), plus
 * GDN_ERR_SCRATCH, and GDN_ERR_LAUNCH when the array's address cannot be
 * obtained. */
#define GDN_SCRATCH_BYTES (64u << 20)

gdn_status_t gdn_fwd_noalloc(const gdn_params_t *p, const void *q, const void *k,
                             const void *v, const float *g_raw, const float *beta,
                             const float *A_log, const float *dt_bias,
                             const int64_t *cu_seqlens, const float *initial_state, void *o,
                             float *final_state, void *stream);

/* The segment length gdn_fwd uses for these parameters on the current device:
 * p->seg_chunks itself, or with GDN_SEG_AUTO the automatic choice (0 = the
 * plain state pass).  *seg_chunks is set.  Queries the device's compute-unit
 * count (no GPU work); GDN_ERR_NULL / the gdn_fwd_check shape errors. */
gdn_status_t gdn_fwd_seg_chunks(const gdn_params_t *p, int packed, int32_t *seg_chunks);

/* Whether gdn_fwd, for these parameters on the current device, runs the output
 * stage fused into the state pass (one kernel) instead of as a kernel of its
 * own.  It does so for bf16 without segments, and for fp32 with K = 64 and
 * more units than compute units (below that, separate kernels measured
 * faster in fp32): each state-pass workgroup
 * holds one (sequence, value head, 16-column) unit when they fit one per
 * compute unit, two beyond that (beyond twice the compute units its
 * workgroups run in several rounds).  Each chunk's start state and v_new
 * then pass from the state-pass waves to
 * the output waves of the same workgroup through LDS instead of memory, and WY
 * also emits the chunk's masked, decayed Q K^T (the intra-chunk term of the
 * output).  For bf16 the results are bit-identical either way: the same
 * products in the same order and rounding.  For fp32 the final state is, while
 * o's fp32 MFMA sums group the reduction index differently (four at a time),
 * so o agrees up to fp32 rounding.  *fused is set to 1 or 0.  No GPU work (for fp32,
 * and with seg_chunks = GDN_SEG_AUTO, it queries the device's compute-unit
 * count, as gdn_fwd_seg_chunks does); GDN_ERR_NULL / the gdn_fwd_check shape
 * errors. */
gdn_status_t gdn_fwd_fuses_output(const gdn_params_t *p, int packed, int32_t *fused);

/* Number of stages gdn_fwd_timed brackets with events: chunk map, WY (with
 * the gate prologue), state pass, output.  With the output fused into the
 * state pass (gdn_fwd_fuses_output), the state-pass event follows the fused
 * kernel and the output event is recorded right after it. */
#define GDN_NUM_STAGES 4

/* gdn_fwd that also records timing events on `stream`, for profiling:
 * events[0] before the first kernel and events[i] right after stage i
 * (1..GDN_NUM_STAGES, order as above; a stage that does not run for these
 * arguments, e.g. the chunk map without cu_seqlens, records its event at the
 * same point as the previous one).  `events` holds GDN_NUM_STAGES + 1 hipEvent_t
 * created by the caller; NULL makes this identical to gdn_fwd.  Same
 * validation and errors as gdn_fwd; a failed event record returns
 * GDN_ERR_LAUNCH. */
gdn_status_t gdn_fwd_timed(const gdn_params_t *p, const void *q, const void *k,
                           const void *v, const float *g_raw, const float *beta,
                           const float *A_log, const float *dt_bias,
                           const int64_t *cu_seqlens, const float *initial_state, void *o,
                           float *final_state, void *workspace, size_t workspace_bytes,
                           void *stream, void *const *events);

/* Stage bits for gdn_fwd_stages, in the order the pass runs them. */
#define GDN_STAGE_CHUNK_MAP 1u /* packed sequences only */
#define GDN_STAGE_WY 2u        /* with the gate prologue */
#define GDN_STAGE_STATE 4u
#define GDN_STAGE_OUTPUT 8u
#define GDN_STAGE_ALL 15u

/* gdn_fwd restricted to the stages whose bits are set in `stage_mask`, for
 * timing or profiling one kernel on its own.  Each stage reads what the
 * earlier ones left in the workspace, so a partial mask reproduces gdn_fwd's
 * results only on a workspace that already holds a full call with the same
 * arguments; the stages are deterministic, so re-running any subset on such a
 * workspace leaves o, final_state and the workspace as they were.
 * GDN_STAGE_ALL is gdn_fwd.  When the output is fused into the state pass,
 * a mask with both GDN_STAGE_STATE and GDN_STAGE_OUTPUT runs the fused kernel;
 * either bit alone runs the unfused kernel of that stage (the state pass then
 * writes the chunk states hc and v_new vn, which the unfused output reads).
 * Same validation and errors as gdn_fwd, plus GDN_ERR_UNSUPPORTED for bits
 * outside GDN_STAGE_ALL.  Precondition with cu_seqlens: a mask without
 * GDN_STAGE_CHUNK_MAP takes the chunk map, seq_slot and seq_order from the
 * workspace as addresses, so the workspace must hold those a call with the
 * same cu_seqlens wrote; on any other workspace the kernels can read and
 * write outside the buffers.  (gdn_fwd, gdn_fwd_noalloc and gdn_bwd always
 * write them first.) */
gdn_status_t gdn_fwd_stages(const gdn_params_t *p, const void *q, const void *k,
                            const void *v, const float *g_raw, const float *beta,
                            const float *A_log, const float *dt_bias,
                            const int64_t *cu_seqlens, const float *initial_state, void *o,
                            float *final_state, void *workspace, size_t workspace_bytes,
                            unsigned stage_mask, void *stream);

/* ---- Backward pass ------------------------------------------------------------
 * Gradients of the forward pass for the scalar
 *     L = sum_t <d_o_t, o_t> + <d_final_state, final_state>,
 * i.e. given d_o = dL/do and d_final_state = dL/d(final state), returns
 * dL/dq, dL/dk, dL/dv, dL/dg_raw, dL/dbeta, dL/dA_log, dL/ddt_bias and
 * dL/d(initial state).  The pages list the kernels of this pass (per-chunk dv,
 * dq/dk/dw/dg, dg, the WY backward and the state recurrence's dh/du: the Ascend
 * GDN blog, "Ascend-affine tiling", and the G_T_CONTIG page, "fix" and
 * "correctness gates", which checks it against automatic differentiation);
 * their formulas are the derivative of the chunk form of the forward pass.  It
 * recomputes the forward intermediates (WY, the state pass) and then runs, on
 * `stream`: the per-chunk dv_local and operand preparation, the state-gradient
 * pass backwards over each sequence's chunks, the per-chunk dq/dk/dw/dg, the
 * WY backward with the gate backward, and the per-key-head dq/dk sums and
 * per-head dA_log/ddt_bias sums.  Arithmetic: fp32 calls multiply on the fp32
 * MFMA; bf16 calls multiply every product (recompute, dv_local preparation,
 * state-gradient pass, dq/dk, WY backward) on the bf16 MFMA with fp32
 * accumulation, their operands rounded to bf16 once (the per-chunk dO term of
 * the state gradient included); the gate backward and the sums are fp32.
 *   p, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state:
 *            exactly as for gdn_fwd (p->seg_chunks is not used: both state
 *            passes here run sequentially over each sequence)
 *   d_o            [B][T][HV][V]   dtype
 *   d_final_state  [N][HV][K][V]   fp32, or NULL (zero)
 *   dq, dk         [B][T][H][K]    dtype, written (sums over the value heads
 *                                  that read each key head)
 *   dv             [B][T][HV][V]   dtype, written
 *   dg_raw, dbeta  [B][T][HV]      fp32, written
 *   dA_log         [HV]            fp32, written
 *   ddt_bias       [HV]            fp32, written, or NULL (not computed); with
 *                                  dt_bias NULL it is the gradient at a zero bias
 *   d_initial_state [N][HV][K][V]  fp32, written, or NULL (not computed)
 *   workspace      gdn_bwd_workspace_size() bytes, 256-byte aligned
 * Alignment: q, k, v, d_o, dq, dk, dv 16 bytes; fp32 arrays 4 bytes;
 * cu_seqlens 8; workspace 256.  Errors as for gdn_fwd (GDN_ERR_NULL also for
 * d_o, dq, dk, dv, dg_raw, dbeta with tokens present, and for dA_log), all
 * checked before anything is enqueued.  Outputs must not overlap inputs or
 * each other.  Partial sums inside the workgroups use LDS atomics, so the low
 * bits of the fp32 results may differ between runs.  Enqueued on `stream`
 * (hipStream_t); returns without waiting; allocates nothing. */
size_t gdn_bwd_workspace_size(const gdn_params_t *p, int packed);

gdn_status_t gdn_bwd(const gdn_params_t *p, const void *q, const void *k, const void *v,
                     const float *g_raw, const float *beta, const float *A_log,
                     const float *dt_bias, const int64_t *cu_seqlens,
                     const float *initial_state, const void *d_o,
                     const float *d_final_state, void *dq, void *dk, void *dv,
                     float *dg_raw, float *dbeta, float *dA_log, float *ddt_bias,
                     float *d_initial_state, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Stages gdn_bwd_timed brackets with events: forward recompute (chunk map, WY,
 * state pass), dv_local preparation, backward state pass, dq/dk, WY backward,
 * sums. */
#define GDN_BWD_NUM_STAGES 6

/* gdn_bwd recording events[0] before the first kernel and events[i] after
 * stage i (GDN_BWD_NUM_STAGES + 1 hipEvent_t created by the caller; NULL makes
 * it gdn_bwd). */
gdn_status_t gdn_bwd_timed(const gdn_params_t *p, const void *q, const void *k,
                           const void *v, const float *g_raw, const float *beta,
                           const float *A_log, const float *dt_bias,
                           const int64_t *cu_seqlens, const float *initial_state,
                           const void *d_o, const float *d_final_state, void *dq, void *dk,
                           void *dv, float *dg_raw, float *dbeta, float *dA_log,
                           float *ddt_bias, float *d_initial_state, void *workspace,
                           size_t workspace_bytes, void *stream, void *const *events);

/* ---- Recurrent step (decode) ---------------------------------------------------
 * The state updated token by token, as the Ascend GDN blog describes the
 * recurrence ("GDN sequence structure and Triton introduction": one state per
 * head, updated as each token arrives).  For each of p->B sequences and each of
 * its p->T new tokens, in order (T = 1: one decode step):
 *     g = -exp(A_log[hv]) * softplus(g_raw + dt_bias[hv]),   a = e^g,
 *     p = H^T k;   H <- a H + beta k (v - a p)^T;   o = scale * H^T q,
 * with H = S^T the [K][V] fp32 state of each (sequence, value head), exactly
 * the recurrence gdn_fwd computes chunkwise.
 *   p        B, T, H, HV, K, V, dtype and scale as for gdn_fwd; num_seqs = 0
 *            (fixed-length sequences only)
 *   q, k     [B][T][H][K]; v [B][T][HV][V] (dtype); g_raw, beta [B][T][HV] fp32
 *   A_log    [HV] fp32; dt_bias [HV] fp32 or NULL
 *   state    [B][HV][K][V] fp32, required: read as the state before the tokens
 *            and overwritten with the state after them (gdn_fwd's
 *            initial_state / final_state layout, so a prefill's final state
 *            continues here)
 *   o        [B][T][HV][V] (dtype)
 * Same sizes, dtypes, alignment and status codes as gdn_fwd (GDN_ERR_SHAPE for
 * num_seqs != 0); no workspace.  B = 0 or T = 0 enqueues nothing.  Enqueued on
 * `stream` (hipStream_t); returns without waiting. */
gdn_status_t gdn_decode(const gdn_params_t *p, const void *q, const void *k, const void *v,
                        const float *g_raw, const float *beta, const float *A_log,
                        const float *dt_bias, float *state, void *o, void *stream);

/* ---- KDA per-channel gate --------------------------------------------------
 * The KDA gate guide (MindSpeed-Ops issue page, "core computation logic"):
 *     yg[t,h,d] = -exp(A_log[h]) * softplus(g[t,h,d] + dt_bias[h*D + d]),
 *     softplus(x) = x for x > 20, else log(1 + e^x),
 * evaluated in fp32 (log(1 + e^x) as log1p(exp(x))) and rounded to yg_dtype
 * with round-to-nearest-even.
 *   g       [T][H][D] contiguous, g_dtype (leading dimensions flattened into T)
 *   A_log   [H] fp32
 *   dt_bias [H*D] fp32 (the guide's [H, D] bias), or NULL for no bias
 *   yg      [T][H][D] contiguous, yg_dtype; written, never read.  yg may be
 *           the same buffer as g when the dtypes are equal (in place); any
 *           other overlap is undefined.
 * dtypes: GDN_F32, GDN_BF16 or GDN_F16, independently for g and yg.
 * Alignment: g and yg to their element size, A_log and dt_bias to 4 bytes.
 * Errors (checked before anything is enqueued): GDN_ERR_SHAPE for T < 0, H < 1,
 * D < 1 or T*H*D beyond int64; GDN_ERR_DTYPE; GDN_ERR_NULL for g, A_log or yg
 * NULL with T > 0; GDN_ERR_ALIGN; GDN_ERR_LAUNCH.  T = 0 enqueues nothing.
 * Enqueued on `stream` (hipStream_t); returns without waiting.  The caller
 * owns every buffer; nothing is allocated. */
gdn_status_t gdn_kda_gate(const void *g, gdn_dtype_t g_dtype, const float *A_log,
                          const float *dt_bias, void *yg, gdn_dtype_t yg_dtype, int64_t T,
                          int32_t H, int32_t D, void *stream);

/* Static description of a status code. */
const char *gdn_status_string(gdn_status_t s);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
