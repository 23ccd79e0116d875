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


# ---------------------------------------------------------------------------
# Backward.  The derivative of the chunk form above for
# L = sum <do, o> + <dht, H_final>, chunk by chunk (a second derivation,
# independent of the token oracle's reverse sweep).  Per chunk, with
# M the causal mask j <= i, P = (Q K^T) * M * e^{dG}, kd = diag(e^{G_last - G}) K:
#   dv_local = scale P^T do;      dv_new = dv_local + kd dH_{c+1}
#   dH_c     = e^{G_last} dH_{c+1} + scale (e^G * Q)^T do - w^T dv_new
#   dPm      = scale (do v_new^T) * M * e^{dG}
#   dq       = scale e^G * (do H_c^T) + dPm K
#   dk       = dPm^T Q + e^{G_last - G} * (v_new dH_{c+1}^T) + [WY terms]
#   dw       = -dv_new H_c^T;  dT = dw (diag(beta e^G) K)^T + dv_new (diag(beta) V)^T
#   dv       = beta * (Tinv^T dv_new)
#   dA       = -strictly_lower(Tinv^T dT Tinv^T)
# and dG collects every exp(G) factor's derivative; dg is its reversed
# chunk-local cumsum.  Returns the gradients with respect to q, k, v, beta and
# the log-decay g (not g_raw), and dh0.

def chunk_step_bwd(Qc, Kc, Vc, gc, bc, H0, dO, dHn, scale=1.0):
    """Gradients of one chunk.  dHn is dL/dH_next.  Returns
    (dq, dk, dv, dbeta, dg, dH0) for the chunk's rows and its start state."""
    C = Kc.shape[0]
    G = np.cumsum(gc)
    diff = G[:, None] - G[None, :]
    lower_incl = np.tril(np.ones((C, C), dtype=bool))
    strict = np.tril(np.ones((C, C), dtype=bool), -1)
    E = np.zeros((C, C))
    E[lower_incl] = np.exp(diff[lower_incl])
    S = Kc @ Kc.T
    A = np.where(strict, bc[:, None] * S * E, 0.0)
    Tinv = np.linalg.solve(np.eye(C) + A, np.eye(C))
    eG = np.exp(G)
    Gl = G[-1]
    w = Tinv @ ((bc * eG)[:, None] * Kc)
    u = Tinv @ (bc[:, None] * Vc)
    v_new = u - w @ H0
    kd = np.exp(Gl - G)[:, None] * Kc
    QK = Qc @ Kc.T
    P = QK * E
    # state pass (reverse)
    dv_new = scale * P.T @ dO + kd @ dHn
    dH0 = np.exp(Gl) * dHn + scale * (eG[:, None] * Qc).T @ dO - w.T @ dv_new
    # output and state-update terms
    dPm = scale * (dO @ v_new.T) * E
    R = dPm * QK
    dG = R.sum(1) - R.sum(0)
    dq_inter = scale * eG[:, None] * (dO @ H0.T)
    dG += np.sum(Qc * dq_inter, 1)
    dq = dq_inter + dPm @ Kc
    dk_kd = np.exp(Gl - G)[:, None] * (v_new @ dHn.T)
    x = np.sum(Kc * dk_kd, 1)
    dG -= x
    dG[-1] += x.sum() + np.exp(Gl) * np.sum(dHn * H0)
    dk = dPm.T @ Qc + dk_kd
    # WY terms
    dw = -dv_new @ H0.T
    dT = dw @ ((bc * eG)[:, None] * Kc).T + dv_new @ (bc[:, None] * Vc).T
    Xw = Tinv.T @ dw
    Xu = Tinv.T @ dv_new
    dk += (bc * eG)[:, None] * Xw
    dbeta = eG * np.sum(Kc * Xw, 1) + np.sum(Vc * Xu, 1)
    dG += bc * eG * np.sum(Kc * Xw, 1)
    dv = bc[:, None] * Xu
    dA = -np.where(strict, Tinv.T @ dT @ Tinv.T, 0.0)
    dS = dA * bc[:, None] * E
    dk += (dS + dS.T) @ Kc
    dbeta += np.sum(dA * E * S, 1)
    Z = dA * A
    dG += Z.sum(1) - Z.sum(0)
    dg = np.cumsum(dG[::-1])[::-1]
    return dq, dk, dv, dbeta, dg, dH0


def bwd(q, k, v, g, beta, do, dht=None, cu_seqlens=None, h0=None, chunk=64, scale=1.0):
    """Chunkwise backward from a given log-decay g [B,T,HV] (fp64).  Returns a
    dict: dq, dk [B,T,H,K]; dv [B,T,HV,V]; dbeta, dg [B,T,HV]; dh0 [N,HV,K,V]."""
    q, k, v, g, beta, do = (np.asarray(x, np.float64) for x in (q, k, v, g, beta, do))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    G = HV // H
    bounds = _seq_bounds(B, T, cu_seqlens)
    N = len(bounds)
    flat = lambda x: x.reshape((B * T,) + x.shape[2:])  # noqa: E731
    qf, kf, vf, gf, bf, df = (flat(x) for x in (q, k, v, g, beta, do))
    out = dict(dq=np.zeros((B * T, H, K)), dk=np.zeros((B * T, H, K)),
               dv=np.zeros((B * T, HV, V)), dbeta=np.zeros((B * T, HV)),
               dg=np.zeros((B * T, HV)), dh0=np.zeros((N, HV, K, V)))
    for n, (s, e) in enumerate(bounds):
        if cu_seqlens is None:
            s, e = n * T, (n + 1) * T
        for hv in range(HV):
            h = hv // G
            Hs = [np.zeros((K, V)) if h0 is None else np.asarray(h0[n, hv], np.float64)]
            cs = list(range(s, e, chunk))
            for c0 in cs:  # forward, keeping each chunk's start state
                c1 = min(c0 + chunk, e)
                _, Hn, _ = chunk_step(qf[c0:c1, h], kf[c0:c1, h], vf[c0:c1, hv], gf[c0:c1, hv],
                                      bf[c0:c1, hv], Hs[-1], scale)
                Hs.append(Hn)
            dH = np.zeros((K, V)) if dht is None else np.asarray(dht[n, hv], np.float64)
            for ci in reversed(range(len(cs))):
                c0 = cs[ci]
                c1 = min(c0 + chunk, e)
                dq, dk, dv, db, dg, dH = chunk_step_bwd(
                    qf[c0:c1, h], kf[c0:c1, h], vf[c0:c1, hv], gf[c0:c1, hv], bf[c0:c1, hv],
                    Hs[ci], df[c0:c1, hv], dH, scale)
                out["dq"][c0:c1, h] += dq
                out["dk"][c0:c1, h] += dk
                out["dv"][c0:c1, hv] = dv
                out["dbeta"][c0:c1, hv] = db
                out["dg"][c0:c1, hv] = dg
            out["dh0"][n, hv] = dH
    for key in ("dq", "dk", "dv", "dbeta", "dg"):
        out[key] = out[key].reshape((B, T) + out[key].shape[1:])
    return out
