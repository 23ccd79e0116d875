"""Recurrent step (gdn_decode through the binding) against the fp64 token
oracle: the same recurrence, started from a given state, over T new tokens.
Inputs follow the forward pass's recipe (inputs.make_inputs); the state before
the tokens is h0 ~ N(0, 0.1^2), or a prefill's final state."""
import dataclasses

import numpy as np
import pytest
import torch

import gated_deltanet_chunkwise_amd as gdn
from gated_deltanet_chunkwise_amd.inputs import make_inputs
from gpu_helpers import assert_close, f64, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def run_decode(inp, state, scale=1.0):
    d = inp.to("cuda")
    st = state.clone().cuda()
    o = gdn.decode(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, st, dt_bias=d.dt_bias, scale=scale)
    torch.cuda.synchronize()
    return f64(o), f64(st)


@pytest.mark.parametrize("B,T,H,HV,K,V,dtype", [
    (4, 1, 2, 4, 128, 128, "bf16"),
    (3, 1, 1, 2, 64, 128, "fp32"),
    (2, 1, 2, 2, 128, 64, "fp32"),
    (5, 1, 4, 4, 64, 64, "bf16"),
    (2, 17, 2, 4, 128, 128, "bf16"),
    (3, 2, 1, 1, 128, 128, "fp32"),
])
def test_steps_from_a_state(B, T, H, HV, K, V, dtype):
    say("case decode", B, T, H, HV, K, V, dtype)
    inp = make_inputs(B=B, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype, seed=300 + B + T + K, h0=True)
    o, fin = run_decode(inp, inp.h0)
    o_ref, fin_ref = run_oracle(inp)
    assert_close(o, o_ref, DT[dtype], "decode o")
    assert_close(fin, fin_ref, DT[dtype], "decode state")


def test_no_bias_and_scale():
    inp = make_inputs(B=2, T=3, H=2, HV=2, K=128, V=128, dtype="fp32", seed=310, h0=True, scale=0.125)
    inp = dataclasses.replace(inp, dt_bias=None)
    o, fin = run_decode(inp, inp.h0, scale=0.125)
    o_ref, fin_ref = run_oracle(inp)
    assert_close(o, o_ref, torch.float32, "decode o (scale, no bias)")
    assert_close(fin, fin_ref, torch.float32, "decode state (scale, no bias)")


def test_prefill_then_decode_continues_the_sequence():
    # gdn_fwd over the first 200 tokens, then five single-token decode calls
    # from its final state, against the oracle over all 205 tokens
    full = make_inputs(B=2, T=205, H=2, HV=4, K=128, V=128, dtype="bf16", seed=320, h0=True)
    cut = lambda x, a, b: x[:, a:b].contiguous()  # noqa: E731
    pre = dataclasses.replace(full, q=cut(full.q, 0, 200), k=cut(full.k, 0, 200),
                              v=cut(full.v, 0, 200), g_raw=cut(full.g_raw, 0, 200),
                              beta=cut(full.beta, 0, 200))
    o_pre, fin_pre = run_gpu(pre)
    state = torch.from_numpy(fin_pre).float().cuda()
    d = full.to("cuda")
    outs = []
    for t in range(200, 205):
        o = gdn.decode(cut(d.q, t, t + 1), cut(d.k, t, t + 1), cut(d.v, t, t + 1),
                       cut(d.g_raw, t, t + 1), cut(d.beta, t, t + 1), d.A_log, state,
                       dt_bias=d.dt_bias)
        outs.append(o)
    torch.cuda.synchronize()
    o_dec = f64(torch.cat(outs, dim=1))
    o_ref, fin_ref = run_oracle(full)
    assert_close(o_pre, o_ref[:, :200], torch.bfloat16, "prefill o")
    assert_close(o_dec, o_ref[:, 200:], torch.bfloat16, "decoded o")
    assert_close(f64(state), fin_ref, torch.bfloat16, "state after decode")


def test_nothing_to_do_leaves_the_state():
    st = torch.randn(2, 2, 64, 64, device="cuda")
    keep = st.clone()
    e = torch.empty((2, 0, 1, 64), device="cuda")
    gdn.decode(e, e, torch.empty((2, 0, 2, 64), device="cuda"), torch.empty((2, 0, 2), device="cuda"),
               torch.empty((2, 0, 2), device="cuda"), torch.zeros(2, device="cuda"), st)
    torch.cuda.synchronize()
    assert torch.equal(st, keep)


def test_batch_decode_shape():
    # the benchmark's decode shape: 64 sequences, one token, H = HV = 8, K = V = 128
    say("case decode B=64 T=1 H=HV=8 K=V=128 bf16")
    inp = make_inputs(B=64, T=1, H=8, HV=8, K=128, V=128, dtype="bf16", seed=330, h0=True)
    o, fin = run_decode(inp, inp.h0)
    o_ref, fin_ref = run_oracle(inp)
    assert_close(o, o_ref, torch.bfloat16, "decode o")
    assert_close(fin, fin_ref, torch.bfloat16, "decode state")
