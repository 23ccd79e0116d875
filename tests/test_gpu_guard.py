"""Guard bands: every buffer the library writes (o, the final state, each
gradient, the decode state and output, the KDA gate output, the workspace) is
placed inside a larger allocation whose bytes before and after it hold a fixed
pattern.  One call of each entry point on ragged packed input must leave every
band untouched (a write past a buffer's end), and must not change any input
(every input is read-only).  The outputs are NaN-filled first, so the parity
checks beside them also show that every element was written."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunkwise_amd as gdn
from gated_deltanet_chunkwise_amd.inputs import make_grads, make_inputs
from gpu_helpers import f64, run_oracle, say

pytestmark = pytest.mark.gpu

PAD = 4096          # bytes of canary on each side (a multiple of 256: alignment kept)
CANARY = 0xA5


class Guarded:
    """A contiguous tensor of `shape` inside a byte buffer with PAD canary
    bytes on both sides."""

    def __init__(self, shape, dtype, fill=None):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * esz
        self.buf = torch.full((n + 2 * PAD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + n].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)

    def intact(self):
        return bool((self.buf[:PAD] == CANARY).all() and (self.buf[-PAD:] == CANARY).all())


def snapshot(tensors):
    return [None if t is None else t.clone() for t in tensors]


def unchanged(before, after):
    return all((a is None and b is None) or torch.equal(a, b) for a, b in zip(before, after))


def guard_forward(plan, nan=True):
    s = plan.o.shape
    bands = {"o": Guarded(tuple(s), plan.o.dtype, float("nan") if nan else None),
             "workspace": Guarded((plan.ws_bytes,), torch.uint8, None)}
    bands["workspace"].t.fill_(0xFF)
    plan.o = bands["o"].t
    plan.workspace = bands["workspace"].t
    if plan.final_state is not None:
        bands["final_state"] = Guarded(tuple(plan.final_state.shape), torch.float32,
                                       float("nan"))
        plan.final_state = bands["final_state"].t
    return bands


CASES = {
    # packed, ragged: empty sequence, sub-chunk and chunk-edge lengths, GQA, h0
    "packed_bf16": dict(B=1, H=2, HV=4, K=128, V=128, dtype="bf16", seed=71, h0=True,
                        lengths=[1, 63, 64, 65, 130, 0, 200, 3]),
    "packed_fp32_k64": dict(B=1, H=2, HV=4, K=64, V=128, dtype="fp32", seed=72, h0=True,
                            lengths=[70, 0, 129, 64]),
    # output fused into the state pass (units between one and two per CU)
    "fused_bf16": dict(B=5, T=300, H=4, HV=8, K=128, V=128, dtype="bf16", seed=73, h0=True),
    # fp32 fused (K = 64, beyond one unit per CU)
    "fused_fp32_k64": dict(B=3, T=300, H=16, HV=32, K=64, V=64, dtype="fp32", seed=74, h0=True),
}


def _inputs(case):
    kw = dict(CASES[case])
    if "lengths" in kw:
        kw["T"] = sum(kw["lengths"])
    return make_inputs(**kw)


@pytest.mark.parametrize("case", sorted(CASES))
def test_forward_guard_bands(case):
    inp = _inputs(case)
    s = inp.shape
    d = inp.to("cuda")
    packed = d.cu_seqlens is not None
    say("case guard fwd", case, s)
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype, "cuda",
                          num_seqs=s["N"] if packed else None, scale=d.scale)
    bands = guard_forward(plan)
    ins = [d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0]
    before = snapshot(ins)
    o, fin = plan(*ins)
    torch.cuda.synchronize()
    for name, b in bands.items():
        assert b.intact(), "%s: a write left the buffer" % name
    assert unchanged(before, ins), "an input was modified"
    o_r, f_r = run_oracle(inp)
    tol = 1e-2 if inp.q.dtype == torch.bfloat16 else 1e-4
    for x, r in ((f64(o), o_r), (f64(fin), f_r)):
        assert np.all(np.isfinite(x))
        assert np.linalg.norm(x - r) <= tol * np.linalg.norm(r)


def test_segmented_forward_guard_bands():
    inp = _inputs("packed_bf16")
    s = inp.shape
    d = inp.to("cuda")
    say("case guard fwd segments", s)
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype, "cuda",
                          num_seqs=s["N"], scale=d.scale, seg_chunks=2)
    bands = guard_forward(plan)
    plan(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0)
    torch.cuda.synchronize()
    for name, b in bands.items():
        assert b.intact(), "%s: a write left the buffer" % name


@pytest.mark.parametrize("case", ["packed_bf16", "packed_fp32_k64"])
def test_backward_guard_bands(case):
    inp = _inputs(case)
    s = inp.shape
    d = inp.to("cuda")
    d_o, dht = make_grads(inp, 5)
    d_o, dht = d_o.cuda(), dht.cuda()
    say("case guard bwd", case, s)
    plan = gdn.GdnBackward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype, "cuda",
                           num_seqs=s["N"], scale=d.scale)
    bands = {}
    for name in ("dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "ddt_bias", "d_initial_state"):
        t = getattr(plan, name)
        bands[name] = Guarded(tuple(t.shape), t.dtype, float("nan"))
        setattr(plan, name, bands[name].t)
    bands["workspace"] = Guarded((plan.ws_bytes,), torch.uint8, None)
    bands["workspace"].t.fill_(0xFF)
    plan.workspace = bands["workspace"].t
    ins = [d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d_o, dht, d.cu_seqlens, d.h0]
    before = snapshot(ins)
    grads = plan(*ins)
    torch.cuda.synchronize()
    for name, b in bands.items():
        assert b.intact(), "%s: a write left the buffer" % name
    assert unchanged(before, ins), "an input was modified"
    for name, g in grads.items():
        assert torch.isfinite(g).all(), name + " not fully written"


def test_decode_guard_bands():
    inp = make_inputs(B=3, T=5, H=2, HV=4, K=128, V=64, dtype="bf16", seed=74, h0=True)
    d = inp.to("cuda")
    state = Guarded(tuple(d.h0.shape), torch.float32)
    state.t.copy_(d.h0)
    out = Guarded((3, 5, 4, 64), torch.bfloat16, float("nan"))
    ins = [d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias]
    before = snapshot(ins)
    gdn.decode(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, state.t, dt_bias=d.dt_bias, out=out.t)
    torch.cuda.synchronize()
    assert state.intact() and out.intact()
    assert unchanged(before, ins)
    assert torch.isfinite(out.t).all() and torch.isfinite(state.t).all()


@pytest.mark.parametrize("D", [128, 100, 7])
def test_kda_gate_guard_bands(D):
    """The vector path (D % 8 == 0) and the scalar path, with odd sizes."""
    T, H = 37, 3
    g = torch.randn(T, H, D, device="cuda").to(torch.bfloat16)
    A = torch.randn(H, device="cuda")
    b = torch.randn(H * D, device="cuda")
    out = Guarded((T, H, D), torch.float32, float("nan"))
    before = snapshot([g, A, b])
    gdn.kda_gate(g, A, b, out=out.t)
    torch.cuda.synchronize()
    assert out.intact()
    assert unchanged(before, [g, A, b])
    assert torch.isfinite(out.t).all()
