"""Segment-parallel state pass (gdn_params_t.seg_chunks > 0) against the fp64
token oracle, and against the plain pass on the GPU.  The two-level algebra
itself is pinned on the CPU (pin_segment_scan)."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunkwise_amd as gdn
from gated_deltanet_chunkwise_amd.inputs import make_inputs
from gpu_helpers import assert_close, f64, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def run_seg(inp, seg_chunks, plan_out=None):
    d = inp.to("cuda")
    s = inp.shape
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype, d.q.device,
                          num_seqs=None if d.cu_seqlens is None else s["N"], scale=d.scale,
                          seg_chunks=seg_chunks)
    plan.o.fill_(float("nan"))
    plan.final_state.fill_(float("nan"))
    o, fin = plan(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0)
    torch.cuda.synchronize()
    if plan_out is not None:
        plan_out.append(plan)
    return f64(o), f64(fin)


def check(inp, L, dtype, what):
    o, fin = run_seg(inp, L)
    o_ref, fin_ref = run_oracle(inp)
    assert_close(o, o_ref, DT[dtype], what + " o")
    assert_close(fin, fin_ref, DT[dtype], what + " final")
    return o, fin


@pytest.mark.parametrize("L", [1, 2, 3, 5])
def test_tiny_fp32(L):
    say("case segments tiny fp32 L=%d" % L)
    inp = make_inputs(B=1, T=256, H=2, HV=2, K=64, V=64, dtype="fp32", seed=400,
                      A_log_range=(-5.0, -3.0))
    check(inp, L, "fp32", "seg L=%d" % L)


@pytest.mark.parametrize("L", [2, 3])
@pytest.mark.parametrize("K,V", [(128, 128), (128, 64), (64, 128)])
def test_ragged_gqa_h0_bf16(L, K, V):
    say("case segments ragged bf16 L=%d K=%d V=%d" % (L, K, V))
    inp = make_inputs(B=2, T=700, H=2, HV=4, K=K, V=V, dtype="bf16", seed=410 + K + V, h0=True,
                      A_log_range=(-5.0, -3.0))
    check(inp, L, "bf16", "seg L=%d" % L)


def test_fp32_k128_register_variant():
    # fp32 at K = 128 runs the register-buffered state pass in every mode
    say("case segments fp32 K=V=128 L=2")
    inp = make_inputs(B=1, T=520, H=1, HV=2, K=128, V=128, dtype="fp32", seed=420, h0=True,
                      A_log_range=(-5.0, -3.0))
    check(inp, 2, "fp32", "seg fp32 K=128")


@pytest.mark.parametrize("L", [1, 4])
def test_packed_with_empty_and_short_sequences(L):
    lengths = [70, 0, 1, 63, 64, 65, 200, 700, 0]
    say("case segments packed L=%d" % L, lengths)
    inp = make_inputs(B=1, T=sum(lengths), H=2, HV=4, K=128, V=128, dtype="bf16", seed=430,
                      lengths=lengths, h0=True, A_log_range=(-5.0, -3.0))
    check(inp, L, "bf16", "seg packed L=%d" % L)


def test_long_sequence_matches_oracle_and_plain_pass():
    # one 16K-token sequence per head, 16 segments of 16 chunks
    say("case segments long T=16384 L=16")
    inp = make_inputs(B=1, T=16384, H=2, HV=2, K=128, V=128, dtype="bf16", seed=440, h0=True,
                      A_log_range=(-6.0, -4.0))
    o, fin = check(inp, 16, "bf16", "seg long")
    o_plain, fin_plain = run_gpu(inp)
    assert_close(o, o_plain, torch.bfloat16, "seg vs plain o")
    assert_close(fin, fin_plain, torch.bfloat16, "seg vs plain final")


def test_stages_with_segments():
    # the state stage covers every segment launch; stage by stage = one call
    inp = make_inputs(B=2, T=300, H=2, HV=2, K=128, V=128, dtype="bf16", seed=450, h0=True)
    plans = []
    o_ref, f_ref = run_seg(inp, 2, plans)
    plan = plans[0]
    d = inp.to("cuda")
    args = (d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0)
    plan.o.fill_(float("nan"))
    plan.final_state.fill_(float("nan"))
    plan.workspace.fill_(0xFF)
    for name in gdn.STAGES:
        plan.bind(*args, stage_mask=gdn.STAGE_BITS[name])()
    torch.cuda.synchronize()
    assert np.array_equal(f64(plan.o), o_ref) and np.array_equal(f64(plan.final_state), f_ref)
    lay = plan.layout
    assert lay.num_segs == 2 * 3 and lay.seg_m > 0


def _auto_rule(units, NT, cus):
    """The documented automatic choice (include/gdn.h, GDN_SEG_AUTO)."""
    ns = 2 * cus // units
    if ns < 8:
        return 0
    L = max(-(-NT // ns), 16)
    return L if NT // L >= 8 else 0


@pytest.mark.parametrize("B,T,H,HV,packed", [(1, 16384, 2, 2, False), (2, 4100, 2, 2, False),
                                             (2, 300, 8, 8, False), (1, 5000, 2, 2, True)])
def test_automatic_segment_length(B, T, H, HV, packed):
    """GDN_SEG_AUTO picks the documented length on this device, and the call
    gives the same bits as one with that length set explicitly (or with the
    plain pass when it picks none), within the oracle's tolerance."""
    if packed:
        inp = make_inputs(B=1, T=T, H=H, HV=HV, K=128, V=128, dtype="bf16", seed=430,
                          lengths=[3000, 0, 2000], h0=True, A_log_range=(-5.0, -3.0))
    else:
        inp = make_inputs(B=B, T=T, H=H, HV=HV, K=128, V=128, dtype="bf16", seed=431 + T,
                          h0=True, A_log_range=(-5.0, -3.0))
    s = inp.shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = gdn.make_params(s["B"], s["T"], s["H"], s["HV"], 128, 128, gdn.GDN_BF16,
                        s["N"] if packed else 0, 1.0, gdn.GDN_SEG_AUTO)
    L = gdn.seg_chunks(p, packed)
    units = s["N"] * s["HV"] * 8
    expect = 0 if packed else _auto_rule(units, -(-s["T"] // 64), cus)
    say("case auto segments", s, "units", units, "cus", cus, "L", L)
    assert L == expect
    o, fin = check(inp, gdn.GDN_SEG_AUTO, "bf16", "auto L=%d" % L)
    o2, fin2 = run_seg(inp, L)
    assert np.array_equal(o, o2) and np.array_equal(fin, fin2)
