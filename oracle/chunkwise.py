"""fp64 chunkwise (WY) reformulation of the Gated DeltaNet forward pass.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The token oracle (gdn_oracle.c) applies the gated delta rule one token at a
time.  This module computes the same map chunk by chunk, the way the pages'
chunk kernels split it (Ascend GDN blog, "discrete-to-contiguous access":
the hidden state is iterated over T in blocks; the G_T_CONTIG page names the
stages: the WY representation in wy_fast.py, the state pass in
chunk_delta_h.py and the output stage chunk_fwd_o).  The pages do not print
the chunk equations; they follow from the recurrence by induction over the
tokens of a chunk.  With H_0 the state (H = S^T, K x V) at the chunk start,
G the chunk-local cumulative sum of g (restarting at each chunk start) and
delta_r = beta_r (v_r - exp(g_r) H_{r-1}^T k_r):

    H_r = exp(G_r) H_0 + sum_{j<=r} exp(G_r - G_j) k_j delta_j^T

which gives, for the chunk's rows (C tokens):

    A      = strictly_lower( beta_i (k_i . k_j) exp(G_i - G_j) )      (C x C)
    Tinv   = (I + A)^-1                                                (unit lower)
    w      = Tinv diag(beta exp(G)) K                                  (C x K)
    u      = Tinv diag(beta) V                                         (C x V)
    v_new  = u - w H_0                                                 (= delta)
    o      = scale [ diag(exp(G)) Q H_0 + (Q K^T * [j<=i] * exp(G_i - G_j)) v_new ]
    H_next = exp(G_last) H_0 + (diag(exp(G_last - G)) K)^T v_new

Chunks start at every sequence start; the last chunk of a sequence may be
shorter than C.  Decay factors exp(G_i - G_j) are formed from the difference
and only for j <= i.  g = -inf makes G_i - G_j undefined here; callers use a
large finite negative g instead (the token oracle takes -inf directly).
"""
import numpy as np


def _seq_bounds(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(n * T, (n + 1) * T) for n in range(B)]
    cu = [int(x) for x in cu_seqlens]
    return [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def chunk_step(Qc, Kc, Vc, gc, bc, H0, scale=1.0):
    """One chunk of the WY form.  Returns (o_c, H_next, intermediates dict)."""
    C = Kc.shape[0]
    G = np.cumsum(gc)
    # decay D[i, j] = exp(G_i - G_j) for j <= i, 0 above the diagonal
    diff = G[:, None] - G[None, :]
    lower_incl = np.tril(np.ones((C, C), dtype=bool))
    D = np.zeros((C, C))
    D[lower_incl] = np.exp(diff[lower_incl])
    strict = np.tril(np.ones((C, C), dtype=bool), -1)
    A = np.where(strict, bc[:, None] * (Kc @ Kc.T) * D, 0.0)
    Tinv = np.linalg.solve(np.eye(C) + A, np.eye(C))
    w = Tinv @ ((bc * np.exp(G))[:, None] * Kc)
    u = Tinv @ (bc[:, None] * Vc)
    v_new = u - w @ H0
    P = (Qc @ Kc.T) * D
    o_c = scale * ((np.exp(G)[:, None] * Qc) @ H0 + P @ v_new)
    Gl = G[-1]
    H_next = np.exp(Gl) * H0 + (np.exp(Gl - G)[:, None] * Kc).T @ v_new
    inter = dict(G=G, A=A, Tinv=Tinv, w=w, u=u, v_new=v_new, P=P, H0=H0.copy(),
                 kdecay=np.exp(Gl - G)[:, None] * Kc)
    return o_c, H_next, inter


def fwd(q, k, v, g, beta, cu_seqlens=None, h0=None, chunk=64, scale=1.0,
        keep=False, units=None):
    """Chunkwise forward pass in fp64.

    q, k: [B,T,H,K]; v: [B,T,HV,V]; g (log-decay), beta: [B,T,HV];
    cu_seqlens: None or N+1 offsets (B == 1); h0: None or [N,HV,K,V].
    keep=True also returns {(n, hv): [per-chunk intermediates]}.
    units: optional iterable of n*HV+hv to compute (others stay zero).
    """
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    qf, kf = q.reshape(B * T, H, K), k.reshape(B * T, H, K)
    vf, gf, bf = v.reshape(B * T, HV, V), g.reshape(B * T, HV), beta.reshape(B * T, HV)
    bounds = _seq_bounds(B, T, cu_seqlens)
    N = len(bounds)
    o = np.zeros((B * T, HV, V))
    fin = np.zeros((N, HV, K, V))
    kept = {}
    todo = range(N * HV) if units is None else units
    for unit in todo:
        n, hv = divmod(int(unit), HV)
        h = hv // G
        bos, eos = bounds[n]
        Hs = np.zeros((K, V)) if h0 is None else np.array(h0[n, hv], np.float64)
        steps = []
        for s in range(bos, eos, chunk):
            e = min(s + chunk, eos)
            o_c, Hs, inter = chunk_step(qf[s:e, h], kf[s:e, h], vf[s:e, hv],
                                        gf[s:e, hv], bf[s:e, hv], Hs, scale)
            o[s:e, hv] = o_c
            if keep:
                inter["start"] = s
                steps.append(inter)
        fin[n, hv] = Hs
        if keep:
            kept[(n, hv)] = steps
    o = o.reshape(B, T, HV, V)
    return (o, fin, kept) if keep else (o, fin)


def chunk_transition(Kc, gc, bc):
    """The chunk's state map H_next = M H + B, linear part only:
    M = exp(G_last) I - (diag(exp(G_last - G)) K)^T w, from chunk_step's own
    w and decayed keys (so M H equals chunk_step's H_next with V = 0)."""
    K = Kc.shape[1]
    _, _, inter = chunk_step(np.zeros_like(Kc), Kc, np.zeros((Kc.shape[0], 1)), gc, bc,
                             np.zeros((K, 1)))
    Gl = inter["G"][-1]
    return np.exp(Gl) * np.eye(K) - inter["kdecay"].T @ inter["w"]


def segment_scan(q, k, v, g, beta, cu_seqlens=None, h0=None, chunk=64, seg_chunks=4,
                 scale=1.0):
    """Two-level (segment-parallel) form of fwd, in fp64.

    Each sequence's chunks are cut into segments of seg_chunks chunks.  The
    chunk update is affine in the state, H_next = M_c H + B_c, so a segment
    composes to H_end = M_s H_start + E_s with M_s the ordered product of its
    chunks' M_c and E_s its end state from a zero start.  Level 1 forms
    (M_s, E_s) for every segment independently; level 2 walks the segments of
    a sequence in order, H_start(s+1) = M_s H_start(s) + E_s; level 3 reruns
    each segment from its true start state for the outputs.  Same results as
    fwd up to rounding.  Returns (o, fin)."""
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    qf, kf = q.reshape(B * T, H, K), k.reshape(B * T, H, K)
    vf, gf, bf = v.reshape(B * T, HV, V), g.reshape(B * T, HV), beta.reshape(B * T, HV)
    bounds = _seq_bounds(B, T, cu_seqlens)
    o = np.zeros((B * T, HV, V))
    fin = np.zeros((len(bounds), HV, K, V))
    for n, (bos, eos) in enumerate(bounds):
        starts = list(range(bos, eos, chunk))
        segs = [starts[i:i + seg_chunks] for i in range(0, len(starts), seg_chunks)]
        for hv in range(HV):
            h = hv // G
            # level 1: per segment, from a zero state and as a linear map
            ME = []
            for seg in segs:
                M, E = np.eye(K), np.zeros((K, V))
                for s in seg:
                    e = min(s + chunk, eos)
                    Mc = chunk_transition(kf[s:e, h], gf[s:e, hv], bf[s:e, hv])
                    _, E, _ = chunk_step(qf[s:e, h], kf[s:e, h], vf[s:e, hv], gf[s:e, hv],
                                         bf[s:e, hv], E, scale)
                    M = Mc @ M
                ME.append((M, E))
            # level 2: start states in order
            Hs = np.zeros((K, V)) if h0 is None else np.array(h0[n, hv], np.float64)
            starts_state = []
            for M, E in ME:
                starts_state.append(Hs)
                Hs = M @ Hs + E
            fin[n, hv] = Hs
            # level 3: outputs from the true start states
            for seg, Hstart in zip(segs, starts_state):
                Hc = Hstart
                for s in seg:
                    e = min(s + chunk, eos)
                    o_c, Hc, _ = chunk_step(qf[s:e, h], kf[s:e, h], vf[s:e, hv], gf[s:e, hv],
                                            bf[s:e, hv], Hc, scale)
                    o[s:e, hv] = o_c
    return o.reshape(B, T, HV, V), fin
