"""Per-kernel parity: decode the intermediates the kernels leave in the
workspace (chunk-local cumsum, WY factors w/u, decayed keys, chunk-start
states, v_new) and compare each with the chunkwise oracle's intermediates.

The fragment orders decoded here are the ones the kernels document: a k32
fragment holds, for lane l (g = l // 16), the k offsets
4g + i (i < 4) and 16 + 4g + (i - 4) (i >= 4) of a 32-wide block; a D tile
holds rows 4g + r of column l % 16.
"""
import math

import numpy as np
import pytest
import torch

import gated_deltanet_chunkwise_amd as gdn
from gated_deltanet_chunkwise_amd.inputs import make_inputs
from gpu_helpers import f64, metrics, run_gpu, say
import oracle
from oracle import chunkwise

pytestmark = pytest.mark.gpu

LANE = np.arange(64)
G_OF_LANE = LANE // 16
LC = LANE % 16
KSLOT = np.array([[4 * g + i if i < 4 else 12 + 4 * g + i for i in range(8)] for g in range(4)])


def read(ws, off, HV, slots, used, per_slot, dtype):
    """The first `used` chunk slots of each head of a [HV][slots][per_slot]
    workspace array, as fp64 [HV][used][per_slot].  Slots past `used` (the
    packed layout's slot count is an upper bound) were never written and are
    not read."""
    esz = 2 if dtype == torch.bfloat16 else 4
    raw = ws[off:off + HV * slots * per_slot * esz].view(HV, slots, per_slot * esz)
    return raw[:, :used].contiguous().view(dtype).float().cpu().numpy().astype(np.float64)


def decode_w(buf, HV, slots, K):
    """wf [hv][slot][ct<4][kb<K/32][lane][8] -> w[hv][slot][c][kk]."""
    f = buf.reshape(HV, slots, 4, K // 32, 64, 8)
    out = np.zeros((HV, slots, 64, K))
    for ct in range(4):
        for kb in range(K // 32):
            for i in range(8):
                out[:, :, 16 * ct + LC, 32 * kb + KSLOT[G_OF_LANE, i]] = f[:, :, ct, kb, :, i]
    return out


def decode_kt(buf, HV, slots, K):
    """ktf [hv][slot][mt<K/16][cb<2][lane][8] -> kd[hv][slot][c][kk]."""
    f = buf.reshape(HV, slots, K // 16, 2, 64, 8)
    out = np.zeros((HV, slots, 64, K))
    for mt in range(K // 16):
        for cb in range(2):
            for i in range(8):
                out[:, :, 32 * cb + KSLOT[G_OF_LANE, i], 16 * mt + LC] = f[:, :, mt, cb, :, i]
    return out


def decode_u(buf, HV, slots, V):
    """uf [hv][slot][vt][cp<2][lane][2][4] (tiles ct = 2cp + q) -> u[hv][slot][c][v]."""
    f = buf.reshape(HV, slots, V // 16, 2, 64, 2, 4)
    out = np.zeros((HV, slots, 64, V))
    for vt in range(V // 16):
        for cp in range(2):
            for q in range(2):
                for r in range(4):
                    ct = 2 * cp + q
                    out[:, :, 16 * ct + 4 * G_OF_LANE + r, 16 * vt + LC] = f[:, :, vt, cp, :, q, r]
    return out


def decode_hc(buf, HV, slots, K, V):
    """hcf [hv][slot][vt][kb][lane][8] -> H[hv][slot][kk][v]."""
    f = buf.reshape(HV, slots, V // 16, K // 32, 64, 8)
    out = np.zeros((HV, slots, K, V))
    for vt in range(V // 16):
        for kb in range(K // 32):
            for i in range(8):
                out[:, :, 32 * kb + KSLOT[G_OF_LANE, i], 16 * vt + LC] = f[:, :, vt, kb, :, i]
    return out


def decode_vn(buf, HV, slots, V):
    """vnf [hv][slot][vt][cb<2][lane][8] -> v_new[hv][slot][c][v]."""
    f = buf.reshape(HV, slots, V // 16, 2, 64, 8)
    out = np.zeros((HV, slots, 64, V))
    for vt in range(V // 16):
        for cb in range(2):
            for i in range(8):
                out[:, :, 32 * cb + KSLOT[G_OF_LANE, i], 16 * vt + LC] = f[:, :, vt, cb, :, i]
    return out


def decode_pm(buf, HV, slots):
    """pf [hv][slot][it<4][jb<2][lane][8] (P^T fragments, jb <= it/2 written)
    -> P[hv][slot][i][j] (query row i, key column j)."""
    f = buf.reshape(HV, slots, 4, 2, 64, 8)
    out = np.zeros((HV, slots, 64, 64))
    for it in range(4):
        for jb in range(it // 2 + 1):
            for i in range(8):
                out[:, :, 16 * it + LC, 32 * jb + KSLOT[G_OF_LANE, i]] = f[:, :, it, jb, :, i]
    return out


def cmp(x, r, tol, what):
    m = metrics(x, r)
    say("  %-22s rel_l2=%.3e max_abs=%.3e" % (what, m["rel_l2"], m["max_abs"]))
    assert np.all(np.isfinite(x)), what
    assert m["rel_l2"] <= tol, (what, m)


@pytest.mark.parametrize("dtype,tol", [("fp32", 2e-5), ("bf16", 1.5e-2)])
@pytest.mark.parametrize("packed", [False, True])
def test_intermediates(dtype, tol, packed):
    K = V = 128
    if packed:
        lengths = [70, 0, 64, 66]
        inp = make_inputs(B=1, T=sum(lengths), H=1, HV=2, K=K, V=V, dtype=dtype, seed=9,
                          lengths=lengths, h0=True, A_log_range=(-4.0, 0.0))
    else:
        inp = make_inputs(B=2, T=200, H=1, HV=2, K=K, V=V, dtype=dtype, seed=8, h0=True,
                          A_log_range=(-4.0, 0.0))
    say("case intermediates", dtype, "packed" if packed else "fixed", inp.shape)
    plans = []
    # NaN bytes first: a used slot the kernels failed to write does not pass
    run_gpu(inp, plans, ws_fill=0xFF)
    plan = plans[0]
    lay = plan.layout
    s = inp.shape
    HV = s["HV"]
    lens = ([s["T"]] * s["B"] if inp.cu_seqlens is None
            else (inp.cu_seqlens[1:] - inp.cu_seqlens[:-1]).tolist())
    used = sum((n + 63) // 64 for n in lens)
    ws = plan.workspace
    rd = lambda off, per, dt: read(ws, off, HV, lay.num_slots, used, per, dt)  # noqa: E731
    slots = used
    et = inp.q.dtype
    fused = gdn.fuses_output(plan.params, plan.packed)
    say("  output fused into the state pass:", fused)
    pm = None
    if fused:
        # the full call left the masked, decayed Q K^T of every chunk (from WY)
        # and no chunk states; the state pass alone writes those
        pm = decode_pm(rd(lay.pm, 64 * 64, et), HV, slots)
        d = inp.to("cuda")
        plan.bind(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, d.dt_bias, d.cu_seqlens, d.h0,
                  stage_mask=gdn.STAGE_BITS["chain"])()
        torch.cuda.synchronize()
    gam = rd(lay.gamma, 64, torch.float32).reshape(HV, slots, 64)
    bet = rd(lay.beta, 64, torch.float32).reshape(HV, slots, 64)
    w = decode_w(rd(lay.w, 64 * K, et), HV, slots, K)
    kd = decode_kt(rd(lay.kt, 64 * K, et), HV, slots, K)
    u = decode_u(rd(lay.u, 64 * V, et), HV, slots, V)
    hc = decode_hc(rd(lay.hc, K * V, et), HV, slots, K, V)
    vn = decode_vn(rd(lay.vn, 64 * V, et), HV, slots, V)

    q, k, v = f64(inp.q), f64(inp.k), f64(inp.v)
    g = oracle.gate(f64(inp.g_raw), f64(inp.A_log), f64(inp.dt_bias))
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    _, _, kept = chunkwise.fwd(q, k, v, g, f64(inp.beta), cu_seqlens=cu, h0=f64(inp.h0),
                               keep=True)
    # chunk slots in sequence order
    slot = 0
    for n in range(s["N"]):
        steps = kept[(n, 0)]
        for c in range(len(steps)):
            for hv in range(HV):
                st = kept[(n, hv)][c]
                L = len(st["G"])
                tag = "n%d c%d hv%d" % (n, c, hv)
                cmp(gam[hv, slot, :L], st["G"] * math.log2(math.e), 1e-5, tag + " gamma")
                assert np.allclose(gam[hv, slot, L:], gam[hv, slot, L - 1]), tag + " gamma pad"
                assert np.all(bet[hv, slot, L:] == 0), tag + " beta pad"
                cmp(w[hv, slot, :L], st["w"], tol, tag + " w")
                cmp(u[hv, slot, :L], st["u"], tol, tag + " u")
                cmp(kd[hv, slot, :L], st["kdecay"], tol, tag + " kdecay")
                cmp(hc[hv, slot], st["H0"], tol, tag + " chunk-start state")
                cmp(vn[hv, slot, :L], st["v_new"], tol, tag + " v_new")
                if pm is not None:
                    cmp(pm[hv, slot, :L, :L], st["P"], tol, tag + " P (masked QK^T)")
                    assert not np.any(pm[hv, slot, L:]), tag + " P rows past the end"
                    assert not np.any(pm[hv, slot, :, L:]), tag + " P columns past the end"
                for name, arr in (("w", w), ("u", u), ("kd", kd), ("vn", vn)):
                    assert not np.any(arr[hv, slot, L:]), tag + " %s rows past the end" % name
            slot += 1


def test_sequence_order_longest_first():
    """The chunk map's seq_order: a permutation of the packed sequences by
    decreasing chunk count (counts of 1023 chunks and more share the first
    bucket, in any order), and seq_slot's prefix of the chunk counts."""
    lengths = [1, 300, 0, 64, 65, 129, 70000, 200, 5000, 65500, 63, 640, 0, 3]
    inp = make_inputs(B=1, T=sum(lengths), H=1, HV=1, K=64, V=64, dtype="bf16", seed=80,
                      lengths=lengths)
    s = inp.shape
    say("case seq_order", s)
    plan_out = []
    run_gpu(inp, plan_out=plan_out)
    plan = plan_out[0]
    lay = gdn.workspace_layout(plan.params, plan.packed)
    N = len(lengths)
    ws = plan.workspace
    order = ws[lay.seq_order:lay.seq_order + 4 * N].view(torch.int32).cpu().numpy()
    first = ws[lay.seq_slot:lay.seq_slot + 4 * (N + 1)].view(torch.int32).cpu().numpy()
    nch = np.array([(n + 63) // 64 for n in lengths])
    assert np.array_equal(first, np.concatenate([[0], np.cumsum(nch)]))
    assert sorted(order.tolist()) == list(range(N))
    keys = np.minimum(nch[order], 1023)
    assert np.all(np.diff(keys) <= 0), (order, nch[order])
    assert set(order[:2].tolist()) == {6, 9}          # the two sequences past the last bucket
