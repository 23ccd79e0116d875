"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle on
the same (rounded) inputs, compare."""
import sys

import numpy as np
import torch

import gated_deltanet_chunkwise_amd as gdn
import oracle

# Tolerances: fp32 workloads rel-L2 <= 1e-4; bf16 workloads rel-L2 <= 1e-2 and
# max-abs <= 2e-2, on o and on the final state.
TOL = {torch.float32: dict(rel_l2=1e-4, max_abs=None),
       torch.bfloat16: dict(rel_l2=1e-2, max_abs=2e-2)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(inp, plan_out=None, ws_fill=None, seg_chunks=0):
    """Run the library on `inp` (CPU GdnInputs); returns (o, final) as fp64 numpy.
    ws_fill: a byte value the workspace is filled with first."""
    d = inp.to("cuda")
    s = inp.shape
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype, d.q.device,
                          num_seqs=None if d.cu_seqlens is None else s["N"], scale=d.scale,
                          seg_chunks=seg_chunks)
    # NaN-fill the outputs so that any element the kernels fail to write shows up
    plan.o.fill_(float("nan"))
    plan.final_state.fill_(float("nan"))
    if ws_fill is not None:
        plan.workspace.fill_(ws_fill)
    o, fin = plan(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0)
    torch.cuda.synchronize()
    if plan_out is not None:
        plan_out.append(plan)
    return f64(o), f64(fin)


def run_oracle(inp, units=None):
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    return oracle.fwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.g_raw), f64(inp.beta),
                      f64(inp.A_log), f64(inp.dt_bias), cu_seqlens=cu, h0=f64(inp.h0),
                      scale=inp.scale, units=units)


def unit_slices(inp, n, hv):
    """Inputs of one (sequence, value head) unit as a B=1, H=HV=1 problem."""
    s = inp.shape
    G = s["HV"] // s["H"]
    h = hv // G
    if inp.cu_seqlens is None:
        b, sl = n, slice(None)
    else:
        cu = inp.cu_seqlens.tolist()
        b, sl = 0, slice(cu[n], cu[n + 1])
    one = lambda t, i: t[b:b + 1, sl, i:i + 1]  # noqa: E731
    return dict(q=one(inp.q, h), k=one(inp.k, h), v=one(inp.v, hv), g_raw=one(inp.g_raw, hv),
                beta=one(inp.beta, hv), A_log=inp.A_log[hv:hv + 1],
                dt_bias=inp.dt_bias[hv:hv + 1],
                h0=None if inp.h0 is None else inp.h0[n:n + 1, hv:hv + 1]), (b, sl)


def oracle_unit(inp, n, hv):
    u, _ = unit_slices(inp, n, hv)
    o, fin = oracle.fwd(f64(u["q"]), f64(u["k"]), f64(u["v"]), f64(u["g_raw"]), f64(u["beta"]),
                        f64(u["A_log"]), f64(u["dt_bias"]), h0=f64(u["h0"]), scale=inp.scale)
    return o[0, :, 0], fin[0, 0]


def metrics(x, r):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    d = x - r
    nr = np.linalg.norm(r)
    return dict(rel_l2=float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d)),
                max_abs=float(np.max(np.abs(d))) if d.size else 0.0)


def assert_close(x, r, dtype, what):
    m = metrics(x, r)
    tol = TOL[dtype]
    say("  %-28s rel_l2=%.3e max_abs=%.3e" % (what, m["rel_l2"], m["max_abs"]))
    assert np.all(np.isfinite(x)), what + ": non-finite values"
    assert m["rel_l2"] <= tol["rel_l2"], (what, m)
    if tol["max_abs"] is not None:
        assert m["max_abs"] <= tol["max_abs"], (what, m)
    return m


def _sub_problem(inp, b, h_lo, h_hi):
    """Inputs restricted to batch row b (None: all rows, packed input) and key
    heads [h_lo, h_hi) with the value heads that read them: the same GQA
    structure on fewer heads."""
    s = inp.shape
    G = s["HV"] // s["H"]
    hv_lo, hv_hi = h_lo * G, h_hi * G
    rows = slice(None) if b is None else slice(b, b + 1)
    kh = lambda t: t[rows, :, h_lo:h_hi]  # noqa: E731
    vh = lambda t: t[rows, :, hv_lo:hv_hi]  # noqa: E731
    if inp.h0 is None:
        h0 = None
    else:
        n_rows = slice(None) if b is None else slice(b, b + 1)
        h0 = inp.h0[n_rows, hv_lo:hv_hi]
    return dict(q=kh(inp.q), k=kh(inp.k), v=vh(inp.v), g_raw=vh(inp.g_raw), beta=vh(inp.beta),
                A_log=inp.A_log[hv_lo:hv_hi], dt_bias=inp.dt_bias[hv_lo:hv_hi], h0=h0), \
        (rows, slice(hv_lo, hv_hi))


def full_oracle_metrics(inp, o, fin, heads_per_batch=None):
    """rel-L2 and max-abs of the GPU outputs (o [B,T,HV,V], fin [N,HV,K,V], fp64
    numpy) against the oracle over EVERY element, each tensor as a whole.  The
    oracle runs in batches (one sequence of a fixed-length batch, or the whole
    packed batch, times a group of key heads) so that host memory stays bounded;
    the sums of squares and the maximum are accumulated across batches."""
    s = inp.shape
    H = s["H"]
    hb = heads_per_batch or H
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    acc = {"o": [0.0, 0.0, 0.0], "final": [0.0, 0.0, 0.0]}
    rows = [None] if cu is not None else list(range(s["B"]))
    for b in rows:
        for h_lo in range(0, H, hb):
            sub, (rsl, hsl) = _sub_problem(inp, b, h_lo, min(H, h_lo + hb))
            o_r, f_r = oracle.fwd(f64(sub["q"]), f64(sub["k"]), f64(sub["v"]), f64(sub["g_raw"]),
                                  f64(sub["beta"]), f64(sub["A_log"]), f64(sub["dt_bias"]),
                                  cu_seqlens=cu, h0=f64(sub["h0"]), scale=inp.scale)
            n_rows = slice(None) if b is None else slice(b, b + 1)
            for key, x, r in (("o", o[rsl, :, hsl], o_r), ("final", fin[n_rows, hsl], f_r)):
                d = x - r
                a = acc[key]
                a[0] += float(np.sum(d * d))
                a[1] += float(np.sum(r * r))
                a[2] = max(a[2], float(np.max(np.abs(d))) if d.size else 0.0)
    out = {}
    for key, (dd, rr, mx) in acc.items():
        out[key] = dict(rel_l2=float(np.sqrt(dd / rr)) if rr > 0 else float(np.sqrt(dd)),
                        max_abs=mx)
    return out


def assert_metrics(m, dtype, what):
    tol = TOL[dtype]
    say("  %-28s rel_l2=%.3e max_abs=%.3e" % (what, m["rel_l2"], m["max_abs"]))
    assert m["rel_l2"] <= tol["rel_l2"], (what, m)
    if tol["max_abs"] is not None:
        assert m["max_abs"] <= tol["max_abs"], (what, m)
