"""The C ABI boundary on the CPU: the library loads, exports every entry point
include/gdn.h declares, and validates arguments without touching a GPU (no
device pointer is ever dereferenced by these calls)."""
import ctypes
import os
import re

import pytest

import gated_deltanet_chunkwise_amd as gdn
from gated_deltanet_chunkwise_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EALIGN, EWS, ELAUNCH, ESCRATCH = range(9)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(_binding.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gdn.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    seen = set()
    for s in range(9):
        msg = gdn.status_string(s)
        assert msg and msg not in seen
        seen.add(msg)
    assert gdn.status_string(99) == "unknown status"


def P(**kw):
    d = dict(B=2, T=200, H=4, HV=8, K=128, V=64, dtype=gdn.GDN_BF16, num_seqs=0, scale=1.0)
    d.update(kw)
    return gdn.make_params(**d)


def ptrs(**over):
    """12 fake, aligned, never-dereferenced addresses in gdn_fwd's order."""
    names = ["q", "k", "v", "g_raw", "beta", "A_log", "dt_bias", "cu_seqlens",
             "initial_state", "o", "final_state", "workspace"]
    base = {n: 0x10000 * (i + 1) for i, n in enumerate(names)}
    base["cu_seqlens"] = None
    base.update(over)
    return [base[n] for n in names]


def test_valid_call_checks_ok():
    p = P()
    ws = gdn.workspace_size(p)
    assert gdn.check(p, ptrs(), ws) == OK
    assert gdn.check(p, ptrs(initial_state=None, final_state=None, dt_bias=None), ws) == OK


@pytest.mark.parametrize("name", ["q", "k", "v", "g_raw", "beta", "A_log", "o", "workspace"])
def test_required_pointer_null(name):
    p = P()
    assert gdn.check(p, ptrs(**{name: None}), gdn.workspace_size(p)) == ENULL


@pytest.mark.parametrize("name,addr", [("q", 0x10008), ("o", 0x10004), ("v", 0x10002),
                                       ("g_raw", 0x10002), ("beta", 0x10001),
                                       ("A_log", 0x10003), ("initial_state", 0x10002),
                                       ("final_state", 0x10001), ("workspace", 0x10080)])
def test_misaligned(name, addr):
    p = P()
    assert gdn.check(p, ptrs(**{name: addr}), gdn.workspace_size(p)) == EALIGN


def test_workspace_too_small():
    p = P()
    assert gdn.check(p, ptrs(), gdn.workspace_size(p) - 1) == EWS


@pytest.mark.parametrize("kw,status", [
    (dict(HV=6), ESHAPE),            # HV % H != 0
    (dict(H=0), ESHAPE),
    (dict(T=-1), ESHAPE),
    (dict(B=-2), ESHAPE),
    (dict(K=96), EUNSUP),
    (dict(V=256), EUNSUP),
    (dict(K=32), EUNSUP),
    (dict(dtype=7), EDTYPE),
])
def test_bad_shapes(kw, status):
    p = P(**kw)
    assert gdn.check(p, ptrs(), 1 << 40) == status
    assert gdn.workspace_size(p) == 0


def test_packed_rules():
    # cu_seqlens needs B == 1
    assert gdn.check(P(num_seqs=3), ptrs(cu_seqlens=0x90000), 1 << 40) == ESHAPE
    p = P(B=1, T=1000, num_seqs=3)
    ws = gdn.workspace_size(p, packed=True)
    assert gdn.check(p, ptrs(cu_seqlens=0x90000), ws) == OK
    assert gdn.check(p, ptrs(cu_seqlens=0x90004), ws) == EALIGN
    assert gdn.check(p, ptrs(cu_seqlens=0x90000), ws - 256) == EWS


def test_stage_mask_outside_the_stages_is_rejected():
    """gdn_fwd_stages validates like gdn_fwd, then refuses unknown stage bits
    before anything is enqueued (the fake pointers are never used)."""
    lib = gdn.load_library()
    p = P()
    ws = gdn.workspace_size(p)
    vp = [ctypes.c_void_p(a) for a in ptrs()]
    for mask in (gdn.STAGE_ALL + 1, 1 << 31):
        assert lib.gdn_fwd_stages(ctypes.byref(p), *vp, ws, mask, None) == EUNSUP
    # argument errors come first, as in gdn_fwd
    vp_null = [ctypes.c_void_p(a) if a else None for a in ptrs(q=None)]
    assert lib.gdn_fwd_stages(ctypes.byref(p), *vp_null, ws, 1, None) == ENULL
    assert gdn.STAGE_ALL == 15 and gdn.STAGE_BITS["chain"] == 4


def test_empty_token_batch_needs_no_token_pointers():
    p = P(T=0)
    null = dict(q=None, k=None, v=None, g_raw=None, beta=None, A_log=None, o=None)
    assert gdn.check(p, ptrs(**null), gdn.workspace_size(p)) == OK


def test_workspace_layout():
    for dtype, esz in ((gdn.GDN_BF16, 2), (gdn.GDN_F32, 4)):
        for packed in (False, True):
            B = 1 if packed else 3
            p = P(B=B, T=1000, dtype=dtype, num_seqs=5 if packed else 0)
            lay = gdn.workspace_layout(p, packed)
            slots = 1000 // 64 + 5 if packed else B * ((1000 + 63) // 64)
            assert lay.num_slots == slots
            HV, K, V = 8, 128, 64
            hsl = HV * slots
            offs = [lay.gamma, lay.beta, lay.w, lay.kt, lay.u, lay.hc, lay.vn, lay.pm,
                    lay.chunk_map, lay.seq_slot, lay.seq_order, lay.total]
            assert all(o % 256 == 0 for o in offs)
            assert offs == sorted(offs)
            assert lay.beta - lay.gamma >= hsl * 64 * 4
            assert lay.kt - lay.w >= hsl * 64 * K * esz
            assert lay.u - lay.kt >= hsl * 64 * K * esz
            assert lay.hc - lay.u >= hsl * 64 * V * esz
            assert lay.vn - lay.hc >= hsl * K * V * esz
            assert lay.pm - lay.vn >= hsl * 64 * V * esz
            # P^T fragments: [it 4][jb 2][lane 64] of 8 elements per chunk and head
            assert lay.chunk_map - lay.pm >= hsl * 4 * 2 * 64 * 8 * esz
            if packed:
                assert lay.seq_slot - lay.chunk_map >= slots * 16
                assert lay.seq_order - lay.seq_slot >= (5 + 1) * 4
                assert lay.total - lay.seq_order >= 5 * 4
            assert lay.total == gdn.workspace_size(p, packed)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(_binding, "_LIB", None)
    monkeypatch.setattr(_binding, "_LIB_PATH", "/nonexistent/libgdn.so")
    with pytest.raises(OSError):
        _binding.load_library()


def test_kda_gate_validation():
    """gdn_kda_gate rejects bad arguments before enqueuing anything."""
    lib = gdn.load_library()
    F32, BF16, F16 = gdn.GDN_F32, gdn.GDN_BF16, gdn.GDN_F16
    g, A, b, y = (ctypes.c_void_p(0x10000 * i) for i in (1, 2, 3, 4))

    def call(g=g, gt=BF16, A=A, b=b, y=y, yt=F32, T=8, H=4, D=64):
        return lib.gdn_kda_gate(g, gt, A, b, y, yt, T, H, D, None)
    assert call(T=-1) == ESHAPE
    assert call(H=0) == ESHAPE
    assert call(D=0) == ESHAPE
    assert call(T=1 << 62, H=4, D=64) == ESHAPE            # T*H*D beyond int64
    assert call(gt=7) == EDTYPE
    assert call(yt=-1) == EDTYPE
    assert call(g=None) == ENULL
    assert call(A=None) == ENULL
    assert call(y=None) == ENULL
    assert call(g=ctypes.c_void_p(0x10001)) == EALIGN       # bf16 needs 2 bytes
    assert call(y=ctypes.c_void_p(0x10002)) == EALIGN       # fp32 needs 4
    assert call(b=ctypes.c_void_p(0x30002)) == EALIGN
    # nothing to do: no pointer is needed and nothing is enqueued
    assert call(g=None, A=None, b=None, y=None, T=0) == OK
    assert F16 == 2


def test_decode_validation():
    """gdn_decode: gdn_fwd's size rules, fixed-length sequences only, a state is
    required, and nothing is enqueued when there are no tokens."""
    lib = gdn.load_library()
    vp = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(9)]   # q k v g beta A dt state o

    def call(p, ptrs=vp):
        return lib.gdn_decode(ctypes.byref(p), *ptrs, None)
    assert call(P(num_seqs=2, B=1)) == ESHAPE
    assert call(P(K=96)) == EUNSUP
    assert call(P(dtype=gdn.GDN_F16)) == EDTYPE
    assert call(P(HV=6)) == ESHAPE
    assert call(P(), vp[:7] + [None] + vp[8:]) == ENULL               # state
    assert call(P(), [None] + vp[1:]) == ENULL                         # q
    assert call(P(), vp[:3] + [ctypes.c_void_p(0x40002)] + vp[4:]) == EALIGN
    # no tokens: only the state is needed, and nothing is launched
    none = [None] * 7 + [vp[7], None]
    assert call(P(T=0), none) == OK
    assert call(P(B=0), none) == OK


def test_segment_layout():
    """seg_chunks > 0 adds the segment tables and buffers."""
    p0 = P(B=2, T=700, H=2, HV=4, K=128, V=64)
    p2 = P(B=2, T=700, H=2, HV=4, K=128, V=64, seg_chunks=3)
    l0, l2 = gdn.workspace_layout(p0), gdn.workspace_layout(p2)
    assert l0.num_segs == 0 and l0.seg_m == 0
    assert l2.num_segs == 2 * 4                      # 11 chunks per sequence -> 4 segments
    per = l2.num_segs * 4 * 128
    assert l2.seg_e - l2.seq_seg >= (2 + 1) * 4
    assert l2.seg_m - l2.seg_e >= per * 64 * 4
    assert l2.seg_h - l2.seg_m >= per * 128 * 4
    assert l2.total - l2.seg_h >= per * 64 * 4
    assert gdn.workspace_size(p2) == l2.total > gdn.workspace_size(p0)
    # packed: an upper bound of slots / L + N segments
    lp = gdn.workspace_layout(P(B=1, T=1000, num_seqs=3, seg_chunks=2), packed=True)
    assert lp.num_segs == (1000 // 64 + 3) // 2 + 3
    # negative values other than GDN_SEG_AUTO (-1) are errors
    assert gdn.check(P(seg_chunks=-3), ptrs(), 1 << 40) == ESHAPE


def _bwd_call(lib, p, ws_bytes, **over):
    """gdn_bwd with fake, aligned device addresses (never dereferenced: every
    case below fails validation, or has no work)."""
    names = ("q", "k", "v", "g_raw", "beta", "A_log", "dt_bias", "cu_seqlens", "h0", "d_o",
             "dht", "dq", "dk", "dv", "dg_raw", "dbeta", "dA_log", "ddt_bias", "dh0", "ws")
    addr = {n: 0x100000 * (i + 1) for i, n in enumerate(names)}
    addr.update(cu_seqlens=0, h0=0, dht=0)
    addr.update(over)
    vp = [ctypes.c_void_p(addr[n]) if addr[n] else None for n in names[:-1]]
    ws = ctypes.c_void_p(addr["ws"]) if addr["ws"] else None
    return lib.gdn_bwd(ctypes.byref(p), *vp, ws, ws_bytes, None)


def test_bwd_validation():
    lib = gdn.load_library()
    p = P()
    ws = lib.gdn_bwd_workspace_size(ctypes.byref(p), 0)
    assert ws > gdn.workspace_size(p)  # the forward layout plus the backward's buffers
    for name in ("q", "k", "v", "g_raw", "beta", "A_log", "d_o", "dq", "dk", "dv", "dg_raw",
                 "dbeta", "dA_log", "ws"):
        assert _bwd_call(lib, p, ws, **{name: 0}) == ENULL, name
    for name, addr in (("q", 0x100008), ("d_o", 0x100004), ("dq", 0x100002),
                       ("dv", 0x100008), ("dg_raw", 0x100002), ("dh0", 0x100001),
                       ("ddt_bias", 0x100003), ("ws", 0x100080)):
        assert _bwd_call(lib, p, ws, **{name: addr}) == EALIGN, name
    assert _bwd_call(lib, p, ws - 256) == EWS
    bad = P(K=96)
    assert lib.gdn_bwd_workspace_size(ctypes.byref(bad), 0) == 0
    assert _bwd_call(lib, bad, ws) == EUNSUP
    assert _bwd_call(lib, P(HV=3, H=2), ws) == ESHAPE
    # the WY backward's 32-bit row offsets: 64 HV V beyond int32 is rejected
    # by the backward only (the forward takes it)
    wide = P(B=1, T=64, H=1, HV=262144, K=128, V=128)
    assert gdn.workspace_size(wide) > 0
    assert lib.gdn_bwd_workspace_size(ctypes.byref(wide), 0) == 0
    assert _bwd_call(lib, wide, ws) == EUNSUP
    assert _bwd_call(lib, P(num_seqs=2), ws, cu_seqlens=0x90000) == ESHAPE  # packed needs B == 1
    # no tokens: token pointers may be NULL (dA_log is still required)
    e = P(T=0)
    null = dict(q=0, k=0, v=0, g_raw=0, beta=0, d_o=0, dq=0, dk=0, dv=0, dg_raw=0, dbeta=0)
    assert _bwd_call(lib, e, lib.gdn_bwd_workspace_size(ctypes.byref(e), 0),
                     **dict(null, dA_log=0)) == ENULL


def test_bwd_workspace_grows_with_the_problem():
    lib = gdn.load_library()
    sizes = [lib.gdn_bwd_workspace_size(ctypes.byref(P(T=t)), 0) for t in (64, 128, 1000)]
    assert sizes[0] < sizes[1] < sizes[2]
    pk = P(B=1, T=1000, num_seqs=5)
    assert lib.gdn_bwd_workspace_size(ctypes.byref(pk), 1) > gdn.workspace_size(pk, packed=True)


def test_packed_call_without_sequences():
    """A packed call with no sequence but tokens is rejected before anything is
    enqueued, forward and backward (every per-chunk launch would otherwise read
    a chunk map nothing wrote); no sequence and no token is a valid no-op."""
    lib = gdn.load_library()
    bad = P(B=1, T=64, num_seqs=0)
    assert gdn.workspace_size(bad, packed=True) == 0
    assert gdn.check(bad, ptrs(cu_seqlens=0x90000), 1 << 40) == ESHAPE
    assert lib.gdn_bwd_workspace_size(ctypes.byref(bad), 1) == 0
    assert _bwd_call(lib, bad, 1 << 40, cu_seqlens=0x90000) == ESHAPE
    empty = P(B=1, T=0, num_seqs=0)
    ws = gdn.workspace_size(empty, packed=True)
    null = dict(q=None, k=None, v=None, g_raw=None, beta=None, A_log=None, o=None)
    assert gdn.check(empty, ptrs(cu_seqlens=0x90000, **null), ws) == OK
    # the same sizes without cu_seqlens are a fixed-length call (N = B = 1)
    assert gdn.check(bad, ptrs(), 1 << 40) == OK


def test_noalloc_rejects_problems_beyond_the_scratch():
    """gdn_fwd_noalloc checks its arguments, and that the problem's workspace
    fits GDN_SCRATCH_BYTES, before it looks up the scratch address or enqueues
    anything (so these calls never touch a GPU)."""
    lib = gdn.load_library()
    vp = lambda **kw: [ctypes.c_void_p(a) if a else None for a in ptrs(**kw)[:11]]  # noqa: E731
    # B=4, T=8192, H=HV=16, K=V=128 bf16: 836 MiB of workspace
    big = P(B=4, T=8192, H=16, HV=16, K=128, V=128)
    assert gdn.workspace_size(big) > gdn.GDN_SCRATCH_BYTES
    assert lib.gdn_fwd_noalloc(ctypes.byref(big), *vp(), None) == ESCRATCH
    # argument errors are reported like gdn_fwd's
    small = P(B=2, T=2048, H=8, HV=8, K=128, V=128)
    assert gdn.workspace_size(small) <= gdn.GDN_SCRATCH_BYTES
    assert lib.gdn_fwd_noalloc(ctypes.byref(small), *vp(q=None), None) == ENULL
    assert lib.gdn_fwd_noalloc(ctypes.byref(small), *vp(o=0x10004), None) == EALIGN
    assert lib.gdn_fwd_noalloc(ctypes.byref(P(K=96)), *vp(), None) == EUNSUP
    assert lib.gdn_fwd_noalloc(None, *vp(), None) == ENULL
    assert "scratch" in gdn.status_string(ESCRATCH)


def test_automatic_segments_layout():
    """seg_chunks = GDN_SEG_AUTO: the workspace holds the shortest segments the
    choice may take (16 chunks) for fixed-length input; packed input keeps the
    plain pass (no segment buffers).  Other negative values are rejected."""
    auto = P(B=1, T=65536, H=2, HV=2, K=128, V=128, seg_chunks=gdn.GDN_SEG_AUTO)
    assert gdn.workspace_size(auto) == gdn.workspace_size(
        P(B=1, T=65536, H=2, HV=2, K=128, V=128, seg_chunks=16))
    assert gdn.workspace_layout(auto).num_segs == 65536 // 64 // 16
    packed = P(B=1, T=65536, H=2, HV=2, K=128, V=128, num_seqs=3, seg_chunks=gdn.GDN_SEG_AUTO)
    assert gdn.workspace_size(packed, packed=True) == gdn.workspace_size(
        P(B=1, T=65536, H=2, HV=2, K=128, V=128, num_seqs=3), packed=True)
    assert gdn.workspace_size(P(seg_chunks=-2)) == 0
    assert gdn.check(P(seg_chunks=-2), ptrs(), 1 << 40) == ESHAPE
    # an explicit length is reported as given (no device query needed)
    assert gdn.seg_chunks(P(seg_chunks=5)) == 5 and gdn.seg_chunks(P()) == 0
