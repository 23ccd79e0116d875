"""The torch-facing wrappers validate every tensor against the plan on the host
before anything reaches the library: shape, dtype, then device and contiguity.
Plans are built on the CPU (workspace sizing is a pure host call); the
library handle is replaced by one that fails on any use, so each case proves
that nothing was marshalled to a library call."""
import pytest
import torch

import gated_deltanet_chunkwise_amd as gdn

B, T, H, HV, K, V = 2, 70, 2, 4, 64, 128


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError("library call %s reached" % name)


def inputs(dtype=torch.bfloat16, packed=False, N=3):
    f32 = torch.float32
    Bx = 1 if packed else B
    Nx = N if packed else B
    d = dict(q=torch.zeros(Bx, T, H, K, dtype=dtype), k=torch.zeros(Bx, T, H, K, dtype=dtype),
             v=torch.zeros(Bx, T, HV, V, dtype=dtype), g_raw=torch.zeros(Bx, T, HV, dtype=f32),
             beta=torch.zeros(Bx, T, HV, dtype=f32), A_log=torch.zeros(HV, dtype=f32),
             dt_bias=torch.zeros(HV, dtype=f32),
             cu_seqlens=torch.tensor([0, 10, 40, T], dtype=torch.int64) if packed else None,
             initial_state=torch.zeros(Nx, HV, K, V, dtype=f32))
    return d


def fwd_plan(dtype=torch.bfloat16, packed=False):
    Bx = 1 if packed else B
    plan = gdn.GdnForward(Bx, T, H, HV, K, V, dtype, "cpu", num_seqs=3 if packed else None)
    plan.lib = _NoCalls()
    return plan


def call_fwd(plan, d):
    return plan._args(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"], d["dt_bias"],
                      d["cu_seqlens"], d["initial_state"], None)


BAD = [
    ("q", lambda d: d["q"][:, :-1], ValueError),
    ("k", lambda d: d["k"].reshape(d["k"].shape[0], T, H * 2, K // 2), ValueError),
    ("v", lambda d: d["v"][..., :64].contiguous(), ValueError),
    ("v", lambda d: d["v"].float(), TypeError),
    ("q", lambda d: d["q"].float(), TypeError),
    ("g_raw", lambda d: d["g_raw"].to(torch.bfloat16), TypeError),
    ("beta", lambda d: d["beta"][:, :, :2].contiguous(), ValueError),
    ("A_log", lambda d: torch.zeros(H), ValueError),
    ("dt_bias", lambda d: torch.zeros(HV, dtype=torch.float64), TypeError),
    ("initial_state", lambda d: torch.zeros(1, HV, K, V), ValueError),
    ("initial_state", lambda d: torch.zeros(d["initial_state"].shape, dtype=torch.bfloat16),
     TypeError),
]


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("i", range(len(BAD)))
def test_forward_mismatch_raises_before_the_library(packed, i):
    name, mutate, exc = BAD[i]
    plan = fwd_plan(packed=packed)
    d = inputs(packed=packed)
    d[name] = mutate(d)
    with pytest.raises(exc, match="^%s " % name):
        call_fwd(plan, d)


def test_packed_offsets_checked():
    plan = fwd_plan(packed=True)
    for bad, exc in ((torch.tensor([0, 10, T], dtype=torch.int64), ValueError),
                     (torch.tensor([0, 10, 40, T], dtype=torch.int32), TypeError)):
        d = inputs(packed=True)
        d["cu_seqlens"] = bad
        with pytest.raises(exc, match="cu_seqlens"):
            call_fwd(plan, d)
    d = inputs(packed=True)
    d["cu_seqlens"] = None
    with pytest.raises(ValueError, match="cu_seqlens"):
        call_fwd(plan, d)
    d = inputs(packed=False)
    d["cu_seqlens"] = torch.tensor([0, T], dtype=torch.int64)
    with pytest.raises(ValueError, match="cu_seqlens"):
        call_fwd(fwd_plan(packed=False), d)


def test_required_inputs():
    for name in ("q", "k", "v", "g_raw", "beta", "A_log"):
        d = inputs()
        d[name] = None
        with pytest.raises(ValueError, match="^%s " % name):
            call_fwd(fwd_plan(), d)


def test_fp32_plan_rejects_bf16_tensors():
    d = inputs(dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="q"):
        call_fwd(fwd_plan(dtype=torch.float32), d)


def test_matching_host_tensors_fail_on_placement_only():
    """Correct shapes and dtypes on the host: the only complaint is that they
    are not GPU tensors (still before any library call)."""
    d = inputs()
    with pytest.raises(ValueError, match="GPU tensor"):
        call_fwd(fwd_plan(), d)


def bwd_plan(dtype=torch.bfloat16):
    plan = gdn.GdnBackward(B, T, H, HV, K, V, dtype, "cpu")
    plan.lib = _NoCalls()
    return plan


def call_bwd(plan, d, d_o, dht):
    return plan._args(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"], d["dt_bias"],
                      d["cu_seqlens"], d["initial_state"], d_o, dht, None)


@pytest.mark.parametrize("i", range(len(BAD)))
def test_backward_forward_inputs_checked(i):
    name, mutate, exc = BAD[i]
    d = inputs()
    d[name] = mutate(d)
    d_o = torch.zeros(B, T, HV, V, dtype=torch.bfloat16)
    with pytest.raises(exc, match="^%s " % name):
        call_bwd(bwd_plan(), d, d_o, None)


def test_backward_gradient_seeds_checked():
    d = inputs()
    good_do = torch.zeros(B, T, HV, V, dtype=torch.bfloat16)
    for d_o, dht, exc, what in (
            (good_do.float(), None, TypeError, "d_o"),
            (good_do[:, :-1], None, ValueError, "d_o"),
            (None, None, ValueError, "d_o"),
            (good_do, torch.zeros(B, HV, K, V, dtype=torch.bfloat16), TypeError, "d_final_state"),
            (good_do, torch.zeros(B, HV, V, K), ValueError, "d_final_state")):
        with pytest.raises(exc, match="^%s " % what):
            call_bwd(bwd_plan(), d, d_o, dht)
    with pytest.raises(ValueError, match="GPU tensor"):
        call_bwd(bwd_plan(), d, good_do, torch.zeros(B, HV, K, V))


def test_library_shares_torchs_hip_runtime():
    """Loading the library before torch is imported must still leave one HIP
    runtime in the process (torch's): the binding imports torch first."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from gated_deltanet_chunkwise_amd import _binding\n"
            "assert 'torch' not in sys.modules\n"
            "_binding.load_library()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n" % root)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300, cwd=root)
    assert out.returncode == 0, out.stderr[-2000:]
    runtimes = eval(out.stdout.strip().splitlines()[-1])
    assert len(runtimes) == 1, runtimes


def test_autograd_op_checks_placement_before_any_launch():
    """gated_delta_rule has no CPU path: host tensors are refused by the same
    checks as fwd(), before anything is launched."""
    d = inputs()
    leaves = {n: t.clone().requires_grad_(True) for n, t in d.items()
              if t is not None and t.dtype != torch.int64}
    with pytest.raises(ValueError, match="GPU tensor"):
        gdn.gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g_raw"],
                             leaves["beta"], leaves["A_log"], leaves["dt_bias"],
                             initial_state=leaves["initial_state"])
