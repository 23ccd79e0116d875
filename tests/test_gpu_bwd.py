"""Backward pass (gdn_bwd) vs the fp64 oracle's reverse-mode derivative, on the
same rounded inputs and output gradients.

Tolerances per gradient tensor: fp32 rel-L2 <= 1e-4; bf16 rel-L2 <= 1e-2 and
max-abs <= 2e-2 relative to max(1, max |reference|) (gradients are not O(1) in
scale the way o is).  dA_log[hv] and ddt_bias[hv] are sums over every token of
the head, whose terms cancel: their error is bounded against the sum of the
terms' magnitudes (the sum's condition), at the same relative tolerances.
Outputs are NaN-filled before each call, so any element the kernels fail to
write fails the comparison.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_chunkwise_amd as gdn
import oracle
from gated_deltanet_chunkwise_amd.inputs import make_grads, make_inputs, workload_inputs
from gpu_helpers import f64, metrics, say

pytestmark = pytest.mark.gpu

BF, F32 = "bf16", "fp32"
TOL = {torch.float32: (1e-4, None), torch.bfloat16: (1e-2, 2e-2)}
NAMES = ("dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "ddt_bias", "dh0")


def run_gpu_bwd(inp, d_o, dht):
    d = inp.to("cuda")
    s = inp.shape
    plan = gdn.GdnBackward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype,
                           d.q.device, num_seqs=None if d.cu_seqlens is None else s["N"],
                           scale=d.scale)
    for t in plan.grads().values():
        t.fill_(float("nan"))
    out = plan(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d_o.cuda(),
               None if dht is None else dht.cuda(), d.cu_seqlens, d.h0)
    torch.cuda.synchronize()
    return {n: f64(t) for n, t in out.items()}


def run_oracle_bwd(inp, d_o, dht, units=None):
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    # without dt_bias the library returns the gradient at a zero bias
    bias = f64(inp.dt_bias) if inp.dt_bias is not None else np.zeros(inp.shape["HV"])
    return oracle.bwd(f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.g_raw), f64(inp.beta),
                      f64(inp.A_log), bias, f64(d_o), f64(dht), cu_seqlens=cu,
                      h0=f64(inp.h0), scale=inp.scale, units=units)


def param_term_scale(inp, ref):
    """Per value head, the sums of |terms| of dA_log and ddt_bias.  Per token
    ddt_bias gathers dg_raw and dA_log gathers dg g = dg_raw softplus(x) /
    softplus'(x) (x = g_raw + dt_bias), from the oracle's dg_raw."""
    HV = inp.shape["HV"]
    x = f64(inp.g_raw).reshape(-1, HV)
    if inp.dt_bias is not None:
        x = x + f64(inp.dt_bias)[None, :]
    sp = np.where(x > 20, x, np.log1p(np.exp(np.minimum(x, 20))))
    slope = np.where(x > 20, 1.0, 1.0 / (1.0 + np.exp(-x)))
    dgr = np.asarray(ref["dg_raw"]).reshape(-1, HV)
    return dict(dA_log=np.sum(np.abs(dgr * sp / slope), 0), ddt_bias=np.sum(np.abs(dgr), 0))


def compare(got, ref, dtype, tag, names=NAMES, term_scale=None):
    """Every gradient is reported before the first failure is raised."""
    rel, mab = TOL[dtype]
    bad = []
    for n in names:
        x, r = np.asarray(got[n]), np.asarray(ref[n])
        if not np.all(np.isfinite(x)):
            bad.append((n, "non-finite values", int(np.sum(~np.isfinite(x)))))
            continue
        if term_scale is not None and n in term_scale:
            err = np.max(np.abs(x - r) / np.maximum(term_scale[n], 1e-30))
            say("  %-34s err/sum|terms|=%.3e" % (tag + " " + n, err))
            if err > rel:
                bad.append((n, float(err)))
            continue
        m = metrics(x, r)
        scale = max(1.0, float(np.max(np.abs(r)))) if r.size else 1.0
        say("  %-34s rel_l2=%.3e max_abs/scale=%.3e" % (tag + " " + n, m["rel_l2"],
                                                        m["max_abs"] / scale))
        if m["rel_l2"] > rel or (mab is not None and m["max_abs"] > mab * scale):
            bad.append((n, m))
    assert not bad, (tag, bad)


def check_full(inp, tag, seed, dht=True):
    say("case", tag, inp.shape)
    d_o, d_ht = make_grads(inp, seed, final_state_grad=dht)
    got = run_gpu_bwd(inp, d_o, d_ht)
    ref = run_oracle_bwd(inp, d_o, d_ht)
    compare(got, ref, inp.q.dtype, tag, term_scale=param_term_scale(inp, ref))


def test_tiny_fp32_workload():
    check_full(workload_inputs("tiny_fp32", h0=True), "bwd tiny_fp32", 501)


@pytest.mark.parametrize("dtype", [BF, F32])
@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_ragged_gqa_h0(dtype, K, V):
    # 300 = 4 full chunks + a 44-token tail; 2 value heads per key head
    inp = make_inputs(B=2, T=300, H=2, HV=4, K=K, V=V, dtype=dtype, seed=600 + K + V, h0=True,
                      scale=0.75)
    check_full(inp, "bwd ragged_gqa_%s_K%d_V%d" % (dtype, K, V), 700 + K + V)


@pytest.mark.parametrize("dtype", [BF, F32])
def test_packed_with_empty_sequence(dtype):
    # lengths with an empty sequence, a 1-token one and ragged tails
    inp = make_inputs(B=1, T=600, H=1, HV=2, K=128, V=128, dtype=dtype, seed=611, h0=True,
                      lengths=[130, 0, 1, 64, 305, 100])
    check_full(inp, "bwd packed_%s" % dtype, 612)


@pytest.mark.parametrize("dtype", [BF, F32])
def test_no_state_no_bias(dtype):
    # zero initial state, no final-state gradient, no dt_bias
    inp = make_inputs(B=1, T=200, H=2, HV=2, K=64, V=64, dtype=dtype, seed=621)
    inp.dt_bias = None
    check_full(inp, "bwd plain_%s" % dtype, 622, dht=False)


@pytest.mark.parametrize("dtype", [BF, F32])
def test_pages_workload_sampled_heads(dtype):
    """The pages' shape (B=2, T=2048, H=HV=8, K=V=128; bf16 as benchmarked, and
    fp32), every gradient of two sampled value heads (all sequences, so
    dA_log/ddt_bias are complete)."""
    inp = workload_inputs("pages_bf16", dtype=dtype)
    s = inp.shape
    d_o, dht = make_grads(inp, 631)
    got = run_gpu_bwd(inp, d_o, dht)
    for hv in (2, 7):
        units = [n * s["HV"] + hv for n in range(s["N"])]
        ref = run_oracle_bwd(inp, d_o, dht, units=units)
        ts = {k: v[hv:hv + 1] for k, v in param_term_scale(inp, ref).items()}
        sub = lambda d: dict(  # noqa: E731
            dq=d["dq"][:, :, hv], dk=d["dk"][:, :, hv], dv=d["dv"][:, :, hv],
            dg_raw=d["dg_raw"][:, :, hv], dbeta=d["dbeta"][:, :, hv],
            dA_log=d["dA_log"][hv:hv + 1], ddt_bias=d["ddt_bias"][hv:hv + 1],
            dh0=d["dh0"][:, hv])
        compare(sub(got), sub(ref), inp.q.dtype, "bwd pages %s hv=%d" % (dtype, hv),
                term_scale=ts)


def test_repeat_calls_agree():
    """Two calls on one plan (workspace reused) give the same gradients up to
    the order of the in-workgroup fp32 atomics."""
    inp = make_inputs(B=1, T=256, H=1, HV=1, K=64, V=64, dtype=F32, seed=641, h0=True)
    d_o, dht = make_grads(inp, 642)
    a = run_gpu_bwd(inp, d_o, dht)
    b = run_gpu_bwd(inp, d_o, dht)
    for n in NAMES:
        m = metrics(a[n], b[n])
        assert m["rel_l2"] <= 1e-6, (n, m)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129])
def test_chunk_edges(T):
    # one token, a chunk minus one, exactly one chunk, one past, two chunks + 1
    inp = make_inputs(B=2, T=T, H=1, HV=1, K=64, V=128, dtype=F32, seed=650 + T, h0=True)
    check_full(inp, "bwd edge_T%d" % T, 660 + T)


def test_wide_gqa_group():
    # four value heads per key head, bf16 (dq, dk summed by the key-head kernel)
    inp = make_inputs(B=1, T=256, H=2, HV=8, K=128, V=128, dtype=BF, seed=671, h0=True)
    check_full(inp, "bwd gqa4", 672)


def test_packed_mostly_empty():
    inp = make_inputs(B=1, T=70, H=1, HV=2, K=64, V=64, dtype=F32, seed=681, h0=True,
                      lengths=[0, 0, 70, 0])
    check_full(inp, "bwd packed_mostly_empty", 682)


def test_long_gqa_sampled_key_head():
    """A long sequence (T=16384, 256 chunks) with two value heads per key head,
    bf16: every gradient of key head 1's two value heads (the oracle keeps each
    unit's 16384 states, 2 GiB per unit)."""
    inp = make_inputs(B=1, T=16384, H=2, HV=4, K=128, V=128, dtype=BF, seed=691, h0=True)
    d_o, dht = make_grads(inp, 692)
    got = run_gpu_bwd(inp, d_o, dht)
    ref = run_oracle_bwd(inp, d_o, dht, units=[2, 3])
    ts = {k: v[2:4] for k, v in param_term_scale(inp, ref).items()}
    sub = lambda d: dict(  # noqa: E731
        dq=d["dq"][:, :, 1], dk=d["dk"][:, :, 1], dv=d["dv"][:, :, 2:4],
        dg_raw=d["dg_raw"][:, :, 2:4], dbeta=d["dbeta"][:, :, 2:4],
        dA_log=d["dA_log"][2:4], ddt_bias=d["ddt_bias"][2:4], dh0=d["dh0"][:, 2:4])
    compare(sub(got), sub(ref), inp.q.dtype, "bwd long_gqa", term_scale=ts)


@pytest.mark.parametrize("dtype", [BF, F32])
def test_many_units_one_wave_state_pass(dtype):
    """More (sequence, head, 16-column) units than compute units on the 256-CU
    device: the fp32 backward state pass runs one wave per unit; the bf16 one
    keeps the K rows split over waves, its workgroups beyond the resident ones
    in a second round."""
    inp = make_inputs(B=9, T=130, H=2, HV=4, K=128, V=128, dtype=dtype, seed=701, h0=True)
    s = inp.shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = s["N"] * s["HV"] * (s["V"] // 16)
    say("case bwd one_wave_state_pass", s, "units", units, "cus", cus)
    assert units > cus or cus != 256
    check_full(inp, "bwd many_units_%s" % dtype, 702)


@pytest.mark.parametrize("dtype,K,V", [(BF, 128, 128), (F32, 64, 64)])
def test_many_units_ring_recompute(dtype, K, V):
    """Packed sequences with more (sequence, head, 16-column) units than two per
    compute unit on the 256-CU device: the forward recompute's state pass keeps
    the two-wave LDS ring, its workgroups in rounds, longest sequences first."""
    lengths = [1, 63, 64, 65, 130, 0, 200, 3, 300, 129]
    inp = make_inputs(B=1, T=sum(lengths), H=8, HV=16, K=K, V=V, dtype=dtype, seed=720 + K,
                      lengths=lengths, h0=True)
    s = inp.shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = s["N"] * s["HV"] * (s["V"] // 16)
    say("case bwd ring_recompute", s, "units", units, "cus", cus)
    assert units > 2 * cus or cus != 256
    check_full(inp, "bwd ring_recompute_%s_K%d" % (dtype, K), 721)


@pytest.mark.parametrize("dtype,packed", [(BF, False), (F32, True)])
def test_autograd_op(dtype, packed):
    """gated_delta_rule as a torch op: the gradients loss.backward() leaves on
    every input, for loss = <d_o, o> + <d_final, final state>, against the
    oracle's reverse sweep (the same tolerances as a direct gdn_bwd call)."""
    if packed:
        inp = make_inputs(B=1, T=333, H=2, HV=4, K=64, V=128, dtype=dtype, seed=651, h0=True,
                          lengths=[100, 0, 64, 169])
    else:
        inp = make_inputs(B=2, T=150, H=2, HV=4, K=128, V=128, dtype=dtype, seed=652, h0=True,
                          scale=0.8)
    say("case autograd_op", dtype, "packed" if packed else "fixed", inp.shape)
    d_o, dht = make_grads(inp, 653)
    d = inp.to("cuda")
    leaves = {n: getattr(d, n).detach().clone().requires_grad_(True)
              for n in ("q", "k", "v", "g_raw", "beta", "A_log", "dt_bias", "h0")}
    o, fin = gdn.gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g_raw"],
                                  leaves["beta"], leaves["A_log"], leaves["dt_bias"],
                                  cu_seqlens=d.cu_seqlens, initial_state=leaves["h0"],
                                  scale=d.scale)
    loss = (o.float() * d_o.cuda().float()).sum() + (fin * dht.cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    got = dict(dq=leaves["q"].grad, dk=leaves["k"].grad, dv=leaves["v"].grad,
               dg_raw=leaves["g_raw"].grad, dbeta=leaves["beta"].grad,
               dA_log=leaves["A_log"].grad, ddt_bias=leaves["dt_bias"].grad,
               dh0=leaves["h0"].grad)
    got = {n: f64(t) for n, t in got.items()}
    ref = run_oracle_bwd(inp, d_o, dht)
    compare(got, ref, inp.q.dtype, "autograd %s" % dtype, term_scale=param_term_scale(inp, ref))


def test_autograd_op_output_only():
    """Only o enters the loss (no final-state gradient) and the inputs take no
    dt_bias or initial state: those gradients are None, the rest match a
    direct call with d_final_state = NULL."""
    inp = make_inputs(B=1, T=200, H=1, HV=2, K=64, V=64, dtype=BF, seed=661)
    inp.dt_bias = None
    d_o, _ = make_grads(inp, 662, final_state_grad=False)
    d = inp.to("cuda")
    q = d.q.detach().clone().requires_grad_(True)
    g_raw = d.g_raw.detach().clone().requires_grad_(True)
    o, _ = gdn.gated_delta_rule(q, d.k, d.v, g_raw, d.beta, d.A_log, scale=d.scale)
    (o.float() * d_o.cuda().float()).sum().backward()
    torch.cuda.synchronize()
    ref = run_oracle_bwd(inp, d_o, None)
    compare(dict(dq=f64(q.grad), dg_raw=f64(g_raw.grad)), ref, inp.q.dtype,
            "autograd o only", names=("dq", "dg_raw"))


@pytest.mark.parametrize("H,HV,packed", [(8, 32, False), (1, 8, True)])
def test_wide_gqa_groups(H, HV, packed):
    """Four and eight value heads per key head: the backward's block-to-head
    maps and the key-head sums of dq and dk over the group."""
    if packed:
        inp = make_inputs(B=1, T=300, H=H, HV=HV, K=64, V=64, dtype=BF, seed=681, h0=True,
                          lengths=[130, 0, 64, 106])
    else:
        inp = make_inputs(B=1, T=200, H=H, HV=HV, K=64, V=64, dtype=BF, seed=682, h0=True)
    check_full(inp, "bwd gqa_groups_H%d_HV%d%s" % (H, HV, "_packed" if packed else ""), 683)


@pytest.mark.parametrize("dtype", [F32, BF])
def test_extreme_decay(dtype):
    """The backward at A_log in [4, 5] (gates of about -100 per token): every
    gradient finite, and q, k, v, beta and initial-state gradients within the
    usual bounds.  The gate gradients are not held to them here: the chunk form
    gets a token's dg as the reversed in-chunk sum of the cumulative-gate
    gradients, whose O(1) terms cancel to ~0 for a token that cuts the state
    (e^g ~ 1e-44), leaving an fp32 rounding floor (measured ~5e-6 in dg_raw
    against true values below 1e-38) that the per-head sums dA_log and ddt_bias
    gather over the chunk."""
    inp = make_inputs(B=1, T=150, H=2, HV=4, K=64, V=64, dtype=dtype, seed=691, h0=True,
                      A_log_range=(4.0, 5.0))
    d_o, dht = make_grads(inp, 692)
    got = run_gpu_bwd(inp, d_o, dht)
    for n in NAMES:
        assert np.all(np.isfinite(got[n])), n
    ref = run_oracle_bwd(inp, d_o, dht)
    compare(got, ref, inp.q.dtype, "bwd extreme_decay_%s" % dtype,
            names=("dq", "dk", "dv", "dbeta", "dh0"))
    # the floor is small against the largest gate gradient: within the bf16
    # max-abs bound (2e-2) of it for bf16 calls, 1e-3 of it for fp32 calls
    err = np.max(np.abs(got["dg_raw"] - ref["dg_raw"]))
    say("  dg_raw max |err| / max |ref| = %.3e" % (err / np.max(np.abs(ref["dg_raw"]))))
    assert err <= (2e-2 if dtype == BF else 1e-3) * np.max(np.abs(ref["dg_raw"]))
