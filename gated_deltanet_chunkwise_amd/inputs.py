"""Seeded synthetic inputs for the GDN forward pass (shared by tests, bench and
smoke; holds none of the method's arithmetic: the gate, decays and recurrence
are computed only by the library and by the oracle).

Recipe (one torch CPU Generator, fixed draw order q, k, v, beta, a, A_log,
dt_bias, h0, lengths):
  q, k     ~ N(0,1) fp32, L2-normalised per (token, head) over K, then cast
             to the workload dtype (bf16 with round-to-nearest-even)
  v        ~ N(0,1), cast to the workload dtype
  beta     = sigmoid(N(0,1)) fp32                [B,T,HV]
  g_raw a  ~ N(0,1) fp32                         [B,T,HV]
  A_log    ~ U(lo, hi) fp32, default U(0, 2)     [HV]
  dt_bias  ~ N(0, 0.1^2) fp32                    [HV]
  h0       ~ N(0, 0.1^2) fp32 [N,HV,K,V] when requested
  packed lengths: N-1 integers U[lo, hi]; the last is T - sum, accepted when
             it also lies in [lo, hi] (else all are redrawn).
Backward seeds (make_grads, a second Generator seeded separately, draw order
d_o, d_final_state):
  d_o      ~ N(0,1), cast to the workload dtype   [B,T,HV,V]
  d_final_state ~ N(0, 0.1^2) fp32                [N,HV,K,V] when requested
"""
import dataclasses

import torch

WORKLOADS = {
    # small fp32 case the oracle finishes in well under a second
    "tiny_fp32": dict(B=1, T=256, H=2, HV=2, K=64, V=64, dtype="fp32"),
    # the pages' shape (B=2, T=2048, HV=8), K=V=128, bf16
    "pages_bf16": dict(B=2, T=2048, H=8, HV=8, K=128, V=128, dtype="bf16"),
    # wider batch with a non-zero initial state
    "wide_bf16_h0": dict(B=4, T=8192, H=16, HV=16, K=128, V=128, dtype="bf16", h0=True),
    # 12 packed sequences, 32768 tokens, lengths in [64, 6000]
    "packed_bf16": dict(B=1, T=32768, H=16, HV=16, K=128, V=128, dtype="bf16",
                        num_seqs=12, len_range=(64, 6000)),
    # one long sequence, 16 q/k heads each shared by 2 of 32 value heads
    "long_gqa_bf16": dict(B=1, T=65536, H=16, HV=32, K=128, V=128, dtype="bf16"),
    # one long sequence with few heads: 32 (sequence, head, 16-column) units, so
    # the plain state pass leaves most CUs idle (the segment-parallel case)
    "long_single_bf16": dict(B=1, T=65536, H=4, HV=4, K=128, V=128, dtype="bf16"),
    # the same sequence with 16 and 64 units (segment-parallel cost model)
    "long_h2_bf16": dict(B=1, T=65536, H=2, HV=2, K=128, V=128, dtype="bf16"),
    "long_h8_bf16": dict(B=1, T=65536, H=8, HV=8, K=128, V=128, dtype="bf16"),
}
# Seeds per workload (20260 + index in the order above).
SEEDS = {name: 20260 + i for i, name in enumerate(WORKLOADS)}

DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class GdnInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g_raw: torch.Tensor
    beta: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    h0: torch.Tensor = None
    cu_seqlens: torch.Tensor = None
    scale: float = 1.0

    @property
    def shape(self):
        B, T, H, K = self.q.shape
        return dict(B=B, T=T, H=H, HV=self.v.shape[2], K=K, V=self.v.shape[3],
                    N=B if self.cu_seqlens is None else self.cu_seqlens.numel() - 1)

    def to(self, device):
        kw = {f.name: getattr(self, f.name) for f in dataclasses.fields(self)}
        for n, t in kw.items():
            if isinstance(t, torch.Tensor):
                kw[n] = t.to(device).contiguous()
        return GdnInputs(**kw)


def packed_lengths(gen, T, N, lo, hi, max_tries=100000):
    """N lengths in [lo, hi] summing to T (rejection sampling on the last one)."""
    if N == 1:
        if not lo <= T <= hi:
            raise ValueError("T outside the length range")
        return [T]
    for _ in range(max_tries):
        first = torch.randint(lo, hi + 1, (N - 1,), generator=gen).tolist()
        last = T - sum(first)
        if lo <= last <= hi:
            return first + [last]
    raise RuntimeError("could not draw packed lengths")


def make_inputs(B, T, H, HV, K, V, dtype="bf16", seed=0, h0=False, num_seqs=None,
                len_range=(64, 6000), lengths=None, A_log_range=(0.0, 2.0), scale=1.0):
    """Seeded inputs on the CPU (see the module docstring for the recipe)."""
    gen = torch.Generator().manual_seed(int(seed))
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype

    def unit_rows(shape):
        x = torch.randn(shape, generator=gen, dtype=torch.float32)
        x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        return x.to(dt)

    q = unit_rows((B, T, H, K))
    k = unit_rows((B, T, H, K))
    v = torch.randn((B, T, HV, V), generator=gen, dtype=torch.float32).to(dt)
    beta = torch.sigmoid(torch.randn((B, T, HV), generator=gen, dtype=torch.float32))
    g_raw = torch.randn((B, T, HV), generator=gen, dtype=torch.float32)
    lo, hi = A_log_range
    A_log = lo + (hi - lo) * torch.rand((HV,), generator=gen, dtype=torch.float32)
    dt_bias = 0.1 * torch.randn((HV,), generator=gen, dtype=torch.float32)
    packed = num_seqs is not None or lengths is not None
    N = (len(lengths) if lengths is not None else num_seqs) if packed else B
    h0_t = (0.1 * torch.randn((N, HV, K, V), generator=gen, dtype=torch.float32)) if h0 else None
    cu = None
    if packed:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        if lengths is None:
            lengths = packed_lengths(gen, T, num_seqs, *len_range)
        if sum(lengths) != T:
            raise ValueError("lengths must sum to T")
        cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()), dtype=torch.int64)
    return GdnInputs(q=q, k=k, v=v, g_raw=g_raw, beta=beta, A_log=A_log, dt_bias=dt_bias,
                     h0=h0_t, cu_seqlens=cu, scale=scale)


def workload_inputs(name, **overrides):
    """Inputs for a named workload (WORKLOADS), seeded with SEEDS[name]."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    seed = cfg.pop("seed", SEEDS[name])
    return make_inputs(seed=seed, **cfg)


def make_grads(inp, seed, final_state_grad=True):
    """Seeded output gradients for the backward pass: (d_o, d_final_state or None)."""
    gen = torch.Generator().manual_seed(int(seed))
    s = inp.shape
    d_o = torch.randn((s["B"], s["T"], s["HV"], s["V"]), generator=gen,
                      dtype=torch.float32).to(inp.q.dtype)
    dht = None
    if final_state_grad:
        dht = 0.1 * torch.randn((s["N"], s["HV"], s["K"], s["V"]), generator=gen,
                                dtype=torch.float32)
    return d_o, dht
