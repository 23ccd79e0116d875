"""KDA per-channel gate on the GPU (gdn_kda_gate through the binding) against
the fp64 oracle, element by element.

Inputs follow the KDA gate guide's tests ("tests", "GPU precision validation"):
g ~ N(0,1) in the test dtype, A_log ~ N(0,1) fp32, dt_bias ~ N(0,1) fp32
[H*D], over its T / H / D grid (block-edge T values 31-33, 63-65, 127-129).

Tolerance.  The kernel evaluates in fp32 and rounds once to the output dtype.
With x = g + dt_bias, the fp32 result carries a relative error below
(|x| + 8) * 2^-24:
  * |x| * 2^-24 from rounding x, because d log softplus / dx = sigmoid / softplus <= 1;
  * about 8 ulp more from exp, log1p, exp(A_log) and the product.
The test allows twice that.  Where the fp32 result is subnormal (e^x below
2^-126, for x < -87), the error is absolute instead: one subnormal step 2^-149
from exp, scaled by |exp(A_log)|, plus one from the product.  The test allows
(2 |exp(A_log)| + 2) * 2^-149.  A 16-bit output adds half an ulp of that
format.
The guide's own criterion, allclose with atol = rtol = 1e-3, compares against
a reference rounded to the output dtype.  Against an fp64 reference, a value
that lands next to a rounding boundary can round to the neighbour, so the
bound used here is "fp32 error + half an output ulp".  For fp32 outputs the
guide's allclose is asserted as well.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_chunkwise_amd as gdn
import oracle
from gpu_helpers import say

pytestmark = pytest.mark.gpu

DT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}
MANT = {"bf16": 7, "fp16": 10}
MIN_NORMAL = {"bf16": 2.0 ** -126, "fp16": 2.0 ** -14}


def make(T, H, D, dtype, bias, seed, lead=None):
    gen = torch.Generator().manual_seed(seed)
    shape = (lead or (T,)) + (H, D)
    g = torch.randn(shape, generator=gen).to(DT[dtype])
    A = torch.randn(H, generator=gen)
    b = torch.randn(H * D, generator=gen) if bias else None
    return g, A, b


def check(g, A, b, out_dtype, y):
    g64 = g.float().numpy().astype(np.float64)
    A64 = A.numpy().astype(np.float64)
    b64 = None if b is None else b.numpy().astype(np.float64)
    ref = oracle.kda_gate(g64, A64, b64)
    got = y.float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    H, D = g.shape[-2:]
    x = g64 + (0.0 if b64 is None else b64.reshape(H, D))
    scale = np.exp(A64)[:, None]
    bound = 2.0 * (np.abs(x) + 8.0) * 2.0 ** -24 * np.abs(ref) + (2.0 * scale + 2.0) * 2.0 ** -149
    if out_dtype != "fp32":
        mag = np.maximum(np.abs(ref), MIN_NORMAL[out_dtype])
        bound = bound + 0.5 * 2.0 ** (np.floor(np.log2(mag)) - MANT[out_dtype])
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    say("   max |err| %.3e, worst err/bound %.3f" % (float(err.max()) if err.size else 0.0, worst))
    assert np.all(err <= bound), worst
    if out_dtype == "fp32":
        assert np.allclose(got, ref, atol=1e-3, rtol=1e-3)


def run(g, A, b, out_dtype, out=None):
    d = lambda t: None if t is None else t.cuda()  # noqa: E731
    y = gdn.kda_gate(d(g), d(A), d(b), output_dtype=DT[out_dtype], out=out)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T", [1, 16, 31, 32, 33, 63, 64, 65, 127, 128, 129, 512, 1024, 2048, 4096])
def test_sequence_lengths(T):
    say("case kda T=%d H=8 D=128 bf16->bf16 bias" % T)
    g, A, b = make(T, 8, 128, "bf16", True, 100 + T)
    check(g, A, b, "bf16", run(g, A, b, "bf16"))


@pytest.mark.parametrize("H", [4, 8, 12, 16, 32])
@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("bias", [False, True])
def test_heads_and_channels(H, D, bias):
    say("case kda T=65 H=%d D=%d fp32->fp32 bias=%s" % (H, D, bias))
    g, A, b = make(65, H, D, "fp32", bias, 7 * H + D + bias)
    check(g, A, b, "fp32", run(g, A, b, "fp32"))


@pytest.mark.parametrize("din", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("dout", ["fp32", "bf16", "fp16"])
def test_dtype_pairs(din, dout):
    say("case kda T=129 H=12 D=96 %s->%s" % (din, dout))
    g, A, b = make(129, 12, 96, din, True, 31)
    check(g, A, b, dout, run(g, A, b, dout))


@pytest.mark.parametrize("D", [1, 5, 100])
def test_channels_not_a_multiple_of_8(D):
    # the scalar kernel
    say("case kda T=33 H=4 D=%d fp16->fp32" % D)
    g, A, b = make(33, 4, D, "fp16", True, 40 + D)
    check(g, A, b, "fp32", run(g, A, b, "fp32"))


def test_unaligned_views_take_the_scalar_path():
    say("case kda unaligned views")
    g, A, b = make(20, 4, 64, "fp32", True, 50)
    gd = torch.empty(g.numel() + 1, device="cuda")
    gd[1:] = g.reshape(-1).cuda()
    gv = gd[1:].view(g.shape)           # 4-byte aligned, not 16
    od = torch.empty(g.numel() + 1, device="cuda")
    ov = od[1:].view(g.shape)
    gdn.kda_gate(gv, A.cuda(), b.cuda(), out=ov)
    torch.cuda.synchronize()
    check(g, A, b, "fp32", ov)


def test_in_place_and_leading_dims():
    say("case kda in place, g [2,3,H,D]")
    g, A, b = make(None, 8, 128, "bf16", True, 60, lead=(2, 3))
    gd = g.cuda()
    y = gdn.kda_gate(gd, A.cuda(), b.cuda(), out=gd)
    torch.cuda.synchronize()
    assert y.data_ptr() == gd.data_ptr()
    check(g, A, b, "bf16", gd)


def test_branches_and_extremes():
    # softplus identity above 20, its log1p branch just below, deep negatives
    say("case kda extremes")
    vals = torch.tensor([-100.0, -30.0, -5.0, 0.0, 19.99, 20.0, 20.01, 50.0])
    g = vals.repeat(4 * 64 // 8).reshape(1, 4, 64).repeat(3, 1, 1)
    A = torch.tensor([0.0, -2.0, 1.5, 3.0])
    check(g, A, None, "fp32", run(g, A, None, "fp32"))


def test_empty():
    g = torch.empty((0, 4, 64), device="cuda")
    y = gdn.kda_gate(g, torch.zeros(4, device="cuda"))
    assert y.shape == g.shape


def test_benchmark_shape():
    # the guide's timing configuration: T=2048, H=16, D=128, bf16
    say("case kda T=2048 H=16 D=128 bf16->bf16 bias")
    g, A, b = make(2048, 16, 128, "bf16", True, 70)
    check(g, A, b, "bf16", run(g, A, b, "bf16"))
