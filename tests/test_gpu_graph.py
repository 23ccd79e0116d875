"""HIP-graph capture of every entry point.

One call is captured on a side stream and the graph is replayed three times.
Between replays the test copies new input values into the captured tensors,
runs the same entry point eagerly on a second set of outputs (and, where it
has one, its own workspace) and synchronises the device. Every replay must
then equal that eager call:
* bit for bit for the forward (every path: ring, K-split, fused output,
  shared-key-head output, packed, segments, the static scratch), decode and
  the KDA gate;
* to 1e-3 of each gradient's norm for the backward, whose chunk-local row and
  column sums use LDS float atomics (their order, and so the low bits, can
  differ between runs).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_chunkwise_amd as gdn
from gated_deltanet_chunkwise_amd.inputs import make_grads, make_inputs
from gpu_helpers import say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def capture(make_launch):
    """make_launch(stream) -> zero-argument launcher on that stream.  Runs it
    once eagerly on the capture stream, then captures one call."""
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        launch = make_launch(cap)
        launch()
    cap.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        launch()
    torch.cuda.synchronize()
    return graph


def refill(dst, src):
    """Copy the tensors of input set `src` into the captured tensors `dst`."""
    for name in ("q", "k", "v", "g_raw", "beta", "A_log", "dt_bias", "h0"):
        a, b = getattr(dst, name), getattr(src, name)
        if a is not None:
            a.copy_(b.to(a.device))


FWD = {
    # output inside the state pass, one value tile per workgroup, h0, GQA
    "fixed_bf16": dict(B=2, T=300, H=2, HV=4, K=128, V=128, dtype="bf16", h0=True),
    # K split over waves, fp32
    "fixed_fp32_k64": dict(B=1, T=200, H=2, HV=2, K=64, V=64, dtype="fp32", h0=True),
    # packed, ragged, with an empty sequence
    "packed_bf16": dict(B=1, H=2, HV=4, K=128, V=128, dtype="bf16", h0=True,
                        lengths=[1, 63, 64, 65, 130, 0, 200, 3]),
    # output inside the state pass (units between one and two per CU)
    "fused_bf16": dict(B=5, T=300, H=4, HV=8, K=128, V=128, dtype="bf16", h0=True),
    # fp32 at K = 128 (never fused): the state pass, then one output workgroup
    # for both value heads of a key head (2048 workgroups)
    "shared_key_head_fp32": dict(B=1, T=8192, H=8, HV=16, K=128, V=128, dtype="fp32"),
    # fp32 at K = 64 beyond one unit per CU: output inside the state pass
    "fused_fp32_k64": dict(B=3, T=300, H=16, HV=32, K=64, V=64, dtype="fp32", h0=True),
}


def _inputs(kw, seed):
    kw = dict(kw)
    if "lengths" in kw:
        kw["T"] = sum(kw["lengths"])
    return make_inputs(seed=seed, **kw)


def _fwd_plan(s, dtype, packed, scale, seg_chunks=0):
    return gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], dtype, "cuda",
                          num_seqs=s["N"] if packed else None, scale=scale,
                          seg_chunks=seg_chunks)


def _check_forward_replays(case, seg_chunks=0):
    kw = FWD[case]
    d = _inputs(kw, 900).to("cuda")
    s = d.shape
    packed = d.cu_seqlens is not None
    say("case graph fwd", case, s, "seg_chunks", seg_chunks)
    g_plan = _fwd_plan(s, d.q.dtype, packed, d.scale, seg_chunks)
    e_plan = _fwd_plan(s, d.q.dtype, packed, d.scale, seg_chunks)
    fused = gdn.fuses_output(g_plan.params, packed)
    say("  output fused into the state pass:", fused)
    if case.startswith("fused") and seg_chunks == 0:
        assert fused
    if case == "shared_key_head_fp32":
        assert not fused
    args = (d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0)
    graph = capture(lambda st: g_plan.bind(*args, stream=st))
    for r in range(REPLAYS):
        refill(d, _inputs(kw, 901 + r))
        e_plan(*args)
        torch.cuda.synchronize()
        g_plan.o.fill_(float("nan"))
        g_plan.final_state.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_plan.o, e_plan.o), "replay %d: o differs" % r
        assert torch.equal(g_plan.final_state, e_plan.final_state), "replay %d: state" % r


@pytest.mark.parametrize("case", sorted(FWD))
def test_forward_graph_replays(case):
    _check_forward_replays(case)


def test_segmented_forward_graph_replays():
    _check_forward_replays("packed_bf16", seg_chunks=2)


def test_noalloc_graph_replays():
    """gdn_fwd_noalloc captured (its workspace is the library's static scratch)
    against gdn_fwd with a workspace of its own."""
    kw = FWD["packed_bf16"]
    d = _inputs(kw, 910).to("cuda")
    s = d.shape
    say("case graph fwd_noalloc", s)
    o = torch.empty((s["B"], s["T"], s["HV"], s["V"]), dtype=d.q.dtype, device="cuda")
    fin = torch.empty((s["N"], s["HV"], s["K"], s["V"]), dtype=torch.float32, device="cuda")
    e_plan = _fwd_plan(s, d.q.dtype, True, d.scale)

    def make(st):
        return lambda: gdn.fwd_noalloc(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, o,
                                       dt_bias=d.dt_bias, cu_seqlens=d.cu_seqlens,
                                       initial_state=d.h0, final_state=fin, scale=d.scale,
                                       stream=st)
    graph = capture(make)
    for r in range(REPLAYS):
        refill(d, _inputs(kw, 911 + r))
        e_plan(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0)
        torch.cuda.synchronize()
        o.fill_(float("nan"))
        fin.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, e_plan.o) and torch.equal(fin, e_plan.final_state), r


def _rel(a, b):
    a, b = a.double(), b.double()
    n = torch.linalg.vector_norm(b).item()
    return torch.linalg.vector_norm(a - b).item() / max(n, 1e-30)


@pytest.mark.parametrize("case", ["packed_bf16", "fixed_fp32_k64"])
def test_backward_graph_replays(case):
    kw = FWD[case]
    inp = _inputs(kw, 920)
    d = inp.to("cuda")
    s = d.shape
    packed = d.cu_seqlens is not None
    say("case graph bwd", case, s)

    def plan():
        return gdn.GdnBackward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype,
                               "cuda", num_seqs=s["N"] if packed else None, scale=d.scale)
    g_plan, e_plan = plan(), plan()
    d_o, dht = make_grads(inp, 921)
    d_o, dht = d_o.cuda(), dht.cuda()
    args = (d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d_o, dht, d.cu_seqlens, d.h0)
    graph = capture(lambda st: g_plan.bind(*args, stream=st))
    for r in range(REPLAYS):
        new = _inputs(kw, 922 + r)
        refill(d, new)
        n_o, n_ht = make_grads(new, 930 + r)
        d_o.copy_(n_o.cuda())
        dht.copy_(n_ht.cuda())
        e_plan(*args)
        torch.cuda.synchronize()
        for t in g_plan.grads().values():
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for name, g in g_plan.grads().items():
            e = e_plan.grads()[name]
            assert torch.isfinite(g).all(), "replay %d: %s not written" % (r, name)
            assert _rel(g, e) <= 1e-3, "replay %d: %s differs (%.3e)" % (r, name, _rel(g, e))


def test_decode_graph_replays():
    inp = make_inputs(B=3, T=4, H=2, HV=4, K=128, V=64, dtype="bf16", seed=940, h0=True)
    d = inp.to("cuda")
    say("case graph decode", d.shape)
    g_state = d.h0.clone()
    e_state = d.h0.clone()
    g_out = torch.empty((3, 4, 4, 64), dtype=torch.bfloat16, device="cuda")
    e_out = torch.empty_like(g_out)

    def make(st):
        launch, _ = gdn.decode_launcher(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, g_state,
                                        dt_bias=d.dt_bias, out=g_out, stream=st)
        return launch
    graph = capture(make)
    e_launch, _ = gdn.decode_launcher(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, e_state,
                                      dt_bias=d.dt_bias, out=e_out)
    for r in range(REPLAYS):
        new = make_inputs(B=3, T=4, H=2, HV=4, K=128, V=64, dtype="bf16", seed=941 + r,
                          h0=True)
        refill(d, new)
        g_state.copy_(d.h0)
        e_state.copy_(d.h0)
        e_launch()
        torch.cuda.synchronize()
        g_out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_out, e_out) and torch.equal(g_state, e_state), r


def test_kda_gate_graph_replays():
    T, H, D = 37, 3, 128
    gen = torch.Generator().manual_seed(950)
    g = torch.randn(T, H, D, generator=gen).to(torch.bfloat16).cuda()
    A = torch.randn(H, generator=gen).cuda()
    b = torch.randn(H * D, generator=gen).cuda()
    out = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    say("case graph kda_gate", (T, H, D))

    def make(st):
        launch, _ = gdn.kda_gate_launcher(g, A, b, output_dtype=torch.float32, out=out,
                                          stream=st)
        return launch
    graph = capture(make)
    for r in range(REPLAYS):
        g.copy_(torch.randn(T, H, D, generator=gen).to(torch.bfloat16))
        ref = gdn.kda_gate(g, A, b, output_dtype=torch.float32)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        assert np.isfinite(out.cpu().numpy()).all()
