"""HIP path vs the fp64 oracle, element by element, on seeded inputs.

Every case is compared in full: rel-L2 over all elements of o and of the
final state, and max-abs.  The full-size workloads run in the launch
configuration bench.py times; their oracle is computed in batches of
sequences and key heads.
"""
import os

import numpy as np
import pytest
import torch

import gated_deltanet_chunkwise_amd as gdn
from gated_deltanet_chunkwise_amd.inputs import make_inputs, workload_inputs
from gpu_helpers import (assert_close, assert_metrics, f64, full_oracle_metrics, run_gpu,
                         run_oracle, say)

pytestmark = pytest.mark.gpu

BF, F32 = "bf16", "fp32"


def check_full(inp, tag):
    say("case", tag, inp.shape)
    o, fin = run_gpu(inp)
    o_r, fin_r = run_oracle(inp)
    dt = inp.q.dtype
    assert_close(o, o_r, dt, tag + " o")
    assert_close(fin, fin_r, dt, tag + " final")


def test_tiny_fp32_workload():
    check_full(workload_inputs("tiny_fp32"), "tiny_fp32")


@pytest.mark.parametrize("dtype", [BF, F32])
@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_ragged_gqa_h0(dtype, K, V):
    # 300 = 4 full chunks + a 44-token tail; 2 value heads per key head; h0 != 0
    inp = make_inputs(B=2, T=300, H=2, HV=4, K=K, V=V, dtype=dtype, seed=100 + K + V, h0=True,
                      scale=0.75)
    check_full(inp, "ragged_gqa_h0_%s_K%d_V%d" % (dtype, K, V))


def _edge_lengths():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "block_edge_lengths.txt")
    vals = [int(x) for line in open(path) if not line.startswith("#") for x in line.split()]
    return [t for t in vals if t <= 2048]


@pytest.mark.parametrize("dtype", [BF, F32])
@pytest.mark.parametrize("T", _edge_lengths())
def test_block_edge_lengths(dtype, T):
    # the block-edge lengths of the KDA gate precision sweep (tests/golden)
    inp = make_inputs(B=2, T=T, H=2, HV=2, K=128, V=128, dtype=dtype, seed=200 + T)
    check_full(inp, "edge_T%d_%s" % (T, dtype))


@pytest.mark.parametrize("dtype", [BF, F32])
def test_packed_edge_lengths(dtype):
    lengths = [1, 63, 64, 65, 130, 0, 200, 64, 3]
    inp = make_inputs(B=1, T=sum(lengths), H=2, HV=4, K=128, V=128, dtype=dtype, seed=300,
                      lengths=lengths, h0=True)
    check_full(inp, "packed_edges_%s" % dtype)


@pytest.mark.parametrize("dtype", [BF, F32])
def test_slow_decay_long_memory(dtype):
    # A_log in (-6, -3): chunk-level decays near 1, so the state carries across chunks
    inp = make_inputs(B=1, T=1024, H=2, HV=2, K=128, V=128, dtype=dtype, seed=400,
                      A_log_range=(-6.0, -3.0), h0=True)
    check_full(inp, "slow_decay_%s" % dtype)


def test_pages_workload_full():
    # B=2, T=2048, H=HV=8, K=V=128 bf16: small enough to compare every unit
    check_full(workload_inputs("pages_bf16"), "pages_bf16")


def test_empty_and_zero_length():
    # T = 0 with an initial state: o is empty and the final state equals h0
    inp = make_inputs(B=2, T=0, H=1, HV=2, K=64, V=64, dtype=BF, seed=5, h0=True)
    o, fin = run_gpu(inp)
    assert o.shape == (2, 0, 2, 64)
    assert np.array_equal(fin, inp.h0.numpy().astype(np.float64))


def test_deterministic():
    inp = make_inputs(B=1, T=700, H=2, HV=2, K=128, V=128, dtype=BF, seed=6, h0=True)
    a = run_gpu(inp)
    b = run_gpu(inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("packed", [False, True])
def test_stages_one_at_a_time_match_one_call(packed):
    """gdn_fwd_stages: the stages launched one by one give gdn_fwd's results
    bit for bit, and re-running one stage on a filled workspace rewrites the
    same outputs (the per-kernel timing in the benchmark relies on both)."""
    if packed:
        lengths = [70, 0, 200, 64]
        inp = make_inputs(B=1, T=sum(lengths), H=2, HV=4, K=128, V=128, dtype=BF, seed=21,
                          lengths=lengths, h0=True)
    else:
        inp = make_inputs(B=2, T=300, H=2, HV=4, K=128, V=128, dtype=BF, seed=22, h0=True)
    say("case stages", "packed" if packed else "fixed", inp.shape)
    o_ref, f_ref = run_gpu(inp)
    d = inp.to("cuda")
    s = inp.shape
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype, d.q.device,
                          num_seqs=None if d.cu_seqlens is None else s["N"], scale=d.scale)
    plan.o.fill_(float("nan"))
    plan.final_state.fill_(float("nan"))
    plan.workspace.fill_(0xFF)
    args = (d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0)
    for name in gdn.STAGES:
        plan.bind(*args, stage_mask=gdn.STAGE_BITS[name])()
    torch.cuda.synchronize()
    assert np.array_equal(f64(plan.o), o_ref) and np.array_equal(f64(plan.final_state), f_ref)
    plan.final_state.fill_(float("nan"))
    plan.bind(*args, stage_mask=gdn.STAGE_BITS["chain"])()
    plan.o.fill_(float("nan"))
    plan.bind(*args, stage_mask=gdn.STAGE_BITS["output"])()
    torch.cuda.synchronize()
    assert np.array_equal(f64(plan.o), o_ref) and np.array_equal(f64(plan.final_state), f_ref)
    # the state pass and output together (the fused kernel when the plan fuses
    # them) give the same bits as the two unfused kernels above
    say("  output fused into the state pass:", gdn.fuses_output(plan.params, plan.packed))
    plan.o.fill_(float("nan"))
    plan.final_state.fill_(float("nan"))
    plan.bind(*args, stage_mask=gdn.STAGE_BITS["chain"] | gdn.STAGE_BITS["output"])()
    torch.cuda.synchronize()
    assert np.array_equal(f64(plan.o), o_ref) and np.array_equal(f64(plan.final_state), f_ref)


@pytest.mark.parametrize("packed", [False, True])
def test_fused_output_path(packed):
    """Shapes whose state pass holds two value tiles per workgroup, where the
    output stage runs inside the state pass: parity with the oracle, and the
    same bits as the unfused kernels launched stage by stage."""
    if packed:
        lengths = [1, 300, 0, 64, 65, 129, 200]       # 7 sequences x 8 heads x 8 tiles
        inp = make_inputs(B=1, T=sum(lengths), H=4, HV=8, K=128, V=128, dtype=BF, seed=31,
                          lengths=lengths, h0=True, scale=0.5)
    else:
        inp = make_inputs(B=5, T=300, H=4, HV=8, K=128, V=128, dtype=BF, seed=32, h0=True)
    s = inp.shape
    d = inp.to("cuda")
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype, d.q.device,
                          num_seqs=None if d.cu_seqlens is None else s["N"], scale=d.scale)
    fused = gdn.fuses_output(plan.params, plan.packed)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = s["N"] * s["HV"] * (s["V"] // 16)
    say("case fused_output", "packed" if packed else "fixed", s, "units", units, "cus", cus,
        "fused", fused)
    assert fused  # bf16 without segments
    check_full(inp, "fused_output_%s" % ("packed" if packed else "fixed"))
    o_ref, f_ref = run_gpu(inp)
    plan.o.fill_(float("nan"))
    plan.final_state.fill_(float("nan"))
    args = (d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0)
    for name in gdn.STAGES:
        plan.bind(*args, stage_mask=gdn.STAGE_BITS[name])()
    torch.cuda.synchronize()
    assert np.array_equal(f64(plan.o), o_ref) and np.array_equal(f64(plan.final_state), f_ref)


@pytest.mark.parametrize("K,V,B,T,HV,h0", [(64, 64, 5, 130, 16, False), (64, 128, 5, 40, 8, True),
                                            (128, 64, 5, 200, 16, True), (128, 128, 3, 64, 16, False)])
def test_fused_output_head_sizes(K, V, B, T, HV, h0):
    """The output fused into the state pass at every supported head size, with
    ragged tails, a sequence shorter than one chunk and an exact single chunk
    (units = B * HV * V/16 between one and two times the CU count of the
    256-CU device)."""
    inp = make_inputs(B=B, T=T, H=HV // 2, HV=HV, K=K, V=V, dtype=BF, seed=40 + K + V + T,
                      h0=h0, scale=0.9)
    s = inp.shape
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], torch.bfloat16, "cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = s["N"] * s["HV"] * (s["V"] // 16)
    path = gdn.fuses_output(plan.params, False)
    say("case fused_heads", s, "units", units, "path", path)
    assert path  # bf16 without segments
    check_full(inp, "fused_heads_K%d_V%d_T%d" % (K, V, T))


@pytest.mark.parametrize("K,V,HV,packed", [(128, 128, 8, False), (64, 64, 16, False),
                                           (128, 64, 16, True)])
def test_many_units_two_tile_state_pass(K, V, HV, packed):
    """More (sequence, head, 16-column) units than two per compute unit on the
    256-CU device.  A whole call runs the state pass and the output fused, the
    fused workgroups in several rounds; the stages one at a time run the bf16
    state pass with one wave per two value tiles and the output kernel.  Both
    against the oracle."""
    if packed:
        lengths = [130, 0, 64, 1, 65, 200, 7, 128, 63, 90]   # 10 sequences
        inp = make_inputs(B=1, T=sum(lengths), H=HV // 2, HV=HV, K=K, V=V, dtype=BF, seed=50,
                          lengths=lengths, h0=True)
    else:
        inp = make_inputs(B=9, T=130, H=HV // 2, HV=HV, K=K, V=V, dtype=BF, seed=51 + K + V,
                          h0=True, A_log_range=(-4.0, 0.0))
    s = inp.shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = s["N"] * s["HV"] * (s["V"] // 16)
    say("case two_tile_state_pass", s, "units", units, "cus", cus)
    assert units > 2 * cus or cus != 256
    tag = "two_tile_K%d_V%d%s" % (K, V, "_packed" if packed else "")
    check_full(inp, tag)
    d = inp.to("cuda")
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype, d.q.device,
                          num_seqs=None if d.cu_seqlens is None else s["N"], scale=d.scale)
    assert gdn.fuses_output(plan.params, plan.packed)
    plan.o.fill_(float("nan"))
    plan.final_state.fill_(float("nan"))
    args = (d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0)
    for name in gdn.STAGES:
        plan.bind(*args, stage_mask=gdn.STAGE_BITS[name])()
    torch.cuda.synchronize()
    o_r, fin_r = run_oracle(inp)
    assert_close(f64(plan.o), o_r, inp.q.dtype, tag + " stages o")
    assert_close(f64(plan.final_state), fin_r, inp.q.dtype, tag + " stages final")


def test_split_and_resume_matches_one_call():
    # the final state is a checkpoint: run [0, s) then [s, T) from it
    inp = make_inputs(B=1, T=640, H=2, HV=2, K=128, V=128, dtype=F32, seed=7,
                      A_log_range=(-5.0, -3.0))
    o, fin = run_gpu(inp)
    s = 300
    import dataclasses
    first = dataclasses.replace(inp, q=inp.q[:, :s], k=inp.k[:, :s], v=inp.v[:, :s],
                                g_raw=inp.g_raw[:, :s], beta=inp.beta[:, :s])
    o1, f1 = run_gpu(first)
    second = dataclasses.replace(inp, q=inp.q[:, s:], k=inp.k[:, s:], v=inp.v[:, s:],
                                 g_raw=inp.g_raw[:, s:], beta=inp.beta[:, s:],
                                 h0=torch.from_numpy(f1).float())
    o2, f2 = run_gpu(second)
    assert_close(np.concatenate([o1, o2], axis=1), o, torch.float32, "resume o")
    assert_close(f2, fin, torch.float32, "resume final")


# ---------------------------------------------------------------------------
# full-size workloads, every unit

# key heads per oracle batch: bounds host memory (long GQA: 8 key heads = 16
# value heads of 65536 tokens per batch, about 3 GB of fp64 arrays)
HEADS_PER_BATCH = {"wide_bf16_h0": 16, "packed_bf16": 16, "long_gqa_bf16": 8}


@pytest.mark.parametrize("name", ["wide_bf16_h0", "packed_bf16", "long_gqa_bf16"])
def test_full_size_workload(name):
    """The full-size workloads in the launch configuration bench.py times,
    compared with the oracle over every element of o and of the final state
    (rel-L2 of each tensor as a whole, and max-abs)."""
    inp = workload_inputs(name)
    say("case", name, inp.shape)
    o, fin = run_gpu(inp)
    # every element written (outputs are NaN-filled before the call) and finite
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(fin))
    m = full_oracle_metrics(inp, o, fin, HEADS_PER_BATCH[name])
    dt = inp.q.dtype
    assert_metrics(m["o"], dt, "%s o (all elements)" % name)
    assert_metrics(m["final"], dt, "%s final (all elements)" % name)


@pytest.mark.parametrize("K,V,packed", [(128, 128, False), (64, 128, False), (64, 64, True)])
def test_many_units_fp32_state_pass(K, V, packed):
    """fp32 with more (sequence, head, 16-column) units than compute units on
    the 256-CU device: not the K-split state pass.  At K = 128 one wave per
    unit (the register variant) and the output kernel; at K = 64 a whole call
    runs the state pass and the output fused (two value tiles per workgroup),
    and the stages one at a time the two-wave LDS ring and the output kernel,
    both against the oracle and each other."""
    if packed:
        lengths = [130, 0, 64, 1, 65, 200, 7, 128, 63, 90]   # 10 sequences
        inp = make_inputs(B=1, T=sum(lengths), H=8, HV=16, K=K, V=V, dtype=F32, seed=62,
                          lengths=lengths, h0=True)
    else:
        inp = make_inputs(B=9, T=130, H=2, HV=4, K=K, V=V, dtype=F32, seed=61 + K, h0=True)
    s = inp.shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = s["N"] * s["HV"] * (s["V"] // 16)
    say("case fp32_many_units", s, "units", units, "cus", cus)
    assert units > cus or cus != 256
    tag = "fp32_many_units_K%d_V%d%s" % (K, V, "_packed" if packed else "")
    check_full(inp, tag)
    d = inp.to("cuda")
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], d.q.dtype, d.q.device,
                          num_seqs=None if d.cu_seqlens is None else s["N"], scale=d.scale)
    fused = gdn.fuses_output(plan.params, plan.packed)
    say("  output fused into the state pass:", fused)
    assert fused == (K == 64 and units > cus)
    o_ref, f_ref = run_gpu(inp)
    plan.o.fill_(float("nan"))
    plan.final_state.fill_(float("nan"))
    args = (d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0)
    for name in gdn.STAGES:
        plan.bind(*args, stage_mask=gdn.STAGE_BITS[name])()
    torch.cuda.synchronize()
    o_r, fin_r = run_oracle(inp)
    assert_close(f64(plan.o), o_r, inp.q.dtype, tag + " stages o")
    assert_close(f64(plan.final_state), fin_r, inp.q.dtype, tag + " stages final")
    # the state pass is the same either way; o's fp32 MFMA sums group the
    # reduction index differently when fused, so o agrees to fp32 rounding
    assert np.array_equal(f64(plan.final_state), f_ref)
    assert np.allclose(f64(plan.o), o_ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("K,V,packed,dtype", [(128, 128, False, BF), (64, 128, True, BF),
                                               (128, 64, True, BF), (64, 64, False, F32),
                                               (128, 128, True, F32)])
def test_shared_key_head_workgroups(K, V, packed, dtype):
    """Two value heads per key head and enough (chunk, value head) workgroups
    to fill the 256-CU device eight times over: where the output stage runs as
    a kernel of its own (these fp32 shapes; bf16 with segments, since a whole
    bf16 call fuses it into the state pass) it runs one workgroup per (chunk,
    key head) for both of its value heads (the key head's Q and K loads and
    its Q K^T shared).  Ragged tails, an empty sequence and one shorter than a
    chunk."""
    if packed:
        lengths = [4100, 1, 0, 64, 3999, 129]
        inp = make_inputs(B=1, T=sum(lengths), H=8, HV=16, K=K, V=V, dtype=dtype, seed=91 + K + V,
                          lengths=lengths, h0=True, scale=0.7)
    else:
        inp = make_inputs(B=2, T=8229, H=4, HV=8, K=K, V=V, dtype=dtype, seed=92, h0=True)
    s = inp.shape
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], inp.q.dtype, "cuda",
                          num_seqs=s["N"] if packed else None)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = plan.layout.num_slots * s["HV"]
    say("case shared_key_head", s, "workgroups", wgs, "cus", cus)
    assert wgs >= 8 * cus or cus != 256
    tag = "shared_kh_%s_K%d_V%d%s" % (dtype, K, V, "_packed" if packed else "")
    o_r, fin_r = run_oracle(inp)
    o, fin = run_gpu(inp)
    assert_close(o, o_r, inp.q.dtype, tag + " o")
    assert_close(fin, fin_r, inp.q.dtype, tag + " final")
    if gdn.fuses_output(plan.params, packed):
        # the whole call fuses the output into the state pass; with segments
        # the separate output kernel runs, a workgroup per (chunk, key head)
        o, fin = run_gpu(inp, seg_chunks=16)
        assert_close(o, o_r, inp.q.dtype, tag + " segments o")
        assert_close(fin, fin_r, inp.q.dtype, tag + " segments final")


@pytest.mark.parametrize("H,HV,T,packed,dtype", [
    (8, 32, 200, False, BF),     # four value heads per key head, key heads on every XCD, split WY
    (8, 32, 2100, False, BF),    # the same beyond one dispatch round (non-split WY)
    (8, 64, 700, True, BF),      # eight per key head, packed
    (1, 8, 300, False, BF),      # eight per key head, fewer key heads than XCDs
    (8, 32, 300, True, F32),     # fp32, four per key head, packed
])
def test_wide_gqa_groups(H, HV, T, packed, dtype):
    """GQA groups of four and eight value heads per key head: the block-to-head
    maps of WY, the fused state pass and the output (a key head's value heads
    on one XCD when H is a multiple of 8) at group sizes above two, every
    element against the oracle."""
    K, V = 64, 64
    if packed:
        lengths = [T - 170, 0, 64, 106]
        inp = make_inputs(B=1, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype, seed=71 + HV,
                          lengths=lengths, h0=True)
    else:
        inp = make_inputs(B=1, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype, seed=72 + HV + T, h0=True)
    check_full(inp, "gqa_groups_H%d_HV%d_T%d%s_%s" % (H, HV, T, "_packed" if packed else "",
                                                     dtype))


@pytest.mark.parametrize("dtype", [BF, F32])
def test_extreme_decay(dtype):
    """A_log in [4, 5]: every token's gate is about -100, so the state is all
    but reset at every token, cumulative gates reach thousands within a chunk
    and their forward-in-time differences would overflow exp: the masked
    entries must be selected away, never multiplied by zero (no inf or NaN)."""
    inp = make_inputs(B=2, T=150, H=2, HV=4, K=128, V=128, dtype=dtype, seed=75, h0=True,
                      A_log_range=(4.0, 5.0))
    check_full(inp, "extreme_decay_%s" % dtype)
