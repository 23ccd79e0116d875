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


def run_gpu(inp, plan_out=None):
    """Run the library on `inp` (CPU GdnInputs); returns (o, final) as fp64 numpy."""
    d = inp.to("cuda")
    s = inp.shape
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype, d.q.device,
                          num_seqs=None if d.cu_seqlens is None else s["N"], scale=d.scale)
    # NaN-fill the outputs so that any element the kernels fail to write shows up
    plan.o.fill_(float("nan"))
    plan.final_state.fill_(float("nan"))
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
