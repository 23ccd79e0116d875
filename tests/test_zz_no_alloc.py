"""gdn_fwd_noalloc, the forward pass whose workspace is the library's static
device scratch (for callers that cannot allocate), against gdn_fwd through the
C ABI: two calls in a row on the same GPU, the second with a smaller input
(the scratch then holds the first call's intermediates), each bit-identical to
gdn_fwd with a workspace of its own (the same kernels) and within the oracle
tolerances."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunkwise_amd as gdn
from gated_deltanet_chunkwise_amd.inputs import make_inputs, workload_inputs
from gpu_helpers import assert_close, f64, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


def _noalloc(inp):
    d = inp.to("cuda")
    s = inp.shape
    o = torch.full((s["B"], s["T"], s["HV"], s["V"]), float("nan"), dtype=d.q.dtype,
                   device="cuda")
    fin = torch.full((s["N"], s["HV"], s["K"], s["V"]), float("nan"), dtype=torch.float32,
                     device="cuda")
    gdn.fwd_noalloc(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, o, dt_bias=d.dt_bias,
                    cu_seqlens=d.cu_seqlens, initial_state=d.h0, final_state=fin,
                    scale=d.scale)
    return d, o, fin


def test_noalloc_matches_gdn_fwd_on_two_calls_in_a_row():
    first = workload_inputs("pages_bf16")       # 52.25 MiB of the 64 MiB scratch
    lengths = [1, 63, 64, 65, 130, 0, 200, 3]
    second = make_inputs(B=1, T=sum(lengths), H=2, HV=4, K=128, V=64, dtype="bf16", seed=81,
                         lengths=lengths, h0=True, scale=0.8)
    refs = [run_gpu(first), run_gpu(second)]    # gdn_fwd, each with its own workspace
    torch.cuda.synchronize()
    outs = []
    for inp in (first, second):                 # back to back on the one scratch
        say("case noalloc", inp.shape)
        keep = _noalloc(inp)
        outs.append(keep)
    torch.cuda.synchronize()
    for inp, (o_ref, f_ref), (_, o, fin) in zip((first, second), refs, outs):
        o, fin = f64(o), f64(fin)
        assert np.array_equal(o, o_ref), "o differs from gdn_fwd's"
        assert np.array_equal(fin, f_ref), "final state differs from gdn_fwd's"
        o_r, f_r = run_oracle(inp)
        assert_close(o, o_r, inp.q.dtype, "noalloc o")
        assert_close(fin, f_r, inp.q.dtype, "noalloc final")


def test_noalloc_small_fp32_after_bf16():
    """A third shape and dtype on the same scratch: fp32 at K = V = 64."""
    inp = workload_inputs("tiny_fp32")
    o_ref, f_ref = run_gpu(inp)
    _, o, fin = _noalloc(inp)
    torch.cuda.synchronize()
    assert np.array_equal(f64(o), o_ref) and np.array_equal(f64(fin), f_ref)


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    inp = workload_inputs("wide_bf16_h0")       # 836 MiB of workspace
    with pytest.raises(gdn.GdnError) as e:
        _noalloc(inp)
    assert e.value.status == 8
