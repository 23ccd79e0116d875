"""fp64 CPU oracle for the Gated DeltaNet forward pass.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  It is independent of
the HIP library (no shared code, headers or helpers, and it imports nothing
from gated_deltanet_chunkwise_amd).

* ``fwd``        -- token-by-token recurrence (C, fp64, pthreads), the oracle.
* ``ref_fwd``    -- the same through ``gdn_ref_fwd``, the C twin of the
                    library's gdn_fwd (same argument order, fp64 host arrays).
* ``gate``       -- the gate activation alone (C, fp64).
* ``recurrence`` -- the recurrence from a given log-decay g (C, fp64).
* ``bwd``        -- reverse-mode derivative of ``fwd`` (C, fp64, pthreads) for
                    L = sum <do, o> + <dht, final state>.
* ``chunkwise``  -- numpy fp64 chunkwise (WY) reformulation with per-chunk
                    intermediates, and its backward (``chunkwise.bwd``); a
                    second, independent derivation used to pin the token
                    oracle and to expose intermediates.

Functions marked "parity unpinned" in their module docstring: none.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)


def _declare(lib):
    lib.gdn_oracle_gate.restype = None
    lib.gdn_oracle_gate.argtypes = [_dp, _dp, _dp, ctypes.c_int64, ctypes.c_int, _dp]
    lib.gdn_oracle_kda_gate.restype = None
    lib.gdn_oracle_kda_gate.argtypes = [_dp, _dp, _dp, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int, _dp]
    common = [ctypes.c_int] * 6 + [_i64p, ctypes.c_int, _dp, _dp, _dp]
    tail = [ctypes.c_double, _i32p, ctypes.c_int, _dp, _dp, ctypes.c_int]
    lib.gdn_oracle_recurrence.restype = ctypes.c_int
    lib.gdn_oracle_recurrence.argtypes = common + [_dp, _dp, _dp] + tail
    lib.gdn_oracle_fwd.restype = ctypes.c_int
    lib.gdn_oracle_fwd.argtypes = common + [_dp, _dp, _dp, _dp, _dp] + tail
    lib.gdn_ref_fwd.restype = ctypes.c_int
    lib.gdn_ref_fwd.argtypes = ([ctypes.c_int] * 7 + [ctypes.c_double] + [_dp] * 7 + [_i64p]
                                + [_dp] * 3 + [ctypes.c_int])
    lib.gdn_oracle_bwd.restype = ctypes.c_int
    lib.gdn_oracle_bwd.argtypes = (common + [_dp, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp,
                                             _i32p, ctypes.c_int] + [_dp] * 8 + [ctypes.c_int])
    return lib


def load(path=None):
    """Load (building if needed) the oracle library; `path` selects another build."""
    global _LIB
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _LIB is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _LIB = _declare(ctypes.CDLL(_build.LIB))
    return _LIB


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, t=_dp):
    return None if a is None else a.ctypes.data_as(t)


def default_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def gate(g_raw, A_log, dt_bias=None, lib=None):
    """g[t,hv] = -exp(A_log[hv]) * softplus(g_raw[t,hv] + dt_bias[hv]) in fp64."""
    lib = lib or load()
    g_raw = _f64(g_raw)
    A_log = _f64(A_log)
    dt_bias = _f64(dt_bias)
    HV = A_log.shape[0]
    flat = g_raw.reshape(-1, HV)
    out = np.empty_like(flat)
    lib.gdn_oracle_gate(_ptr(flat), _ptr(A_log), _ptr(dt_bias), flat.shape[0], HV, _ptr(out))
    return out.reshape(g_raw.shape)


def kda_gate(g, A_log, dt_bias=None, lib=None):
    """KDA per-channel gate in fp64: g [..., H, D] -> yg of the same shape,
    yg = -exp(A_log[h]) * softplus(g + dt_bias.reshape(H, D))."""
    lib = lib or load()
    g = _f64(g)
    A_log = _f64(A_log)
    H, D = g.shape[-2:]
    if A_log.shape != (H,):
        raise ValueError("A_log must be [H]")
    if dt_bias is not None:
        dt_bias = _f64(dt_bias).reshape(-1)
        if dt_bias.shape != (H * D,):
            raise ValueError("dt_bias must hold H*D values")
    flat = g.reshape(-1, H, D)
    out = np.empty_like(flat)
    lib.gdn_oracle_kda_gate(_ptr(flat), _ptr(A_log), _ptr(dt_bias), flat.shape[0], H, D,
                            _ptr(out))
    return out.reshape(g.shape)


def _shapes(q, v, cu_seqlens):
    q = np.asarray(q)
    if cu_seqlens is None:
        B, T, H, K = q.shape
        N = B
    else:
        B, T, H, K = q.shape
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        N = len(cu_seqlens) - 1
    HV, V = np.asarray(v).shape[2], np.asarray(v).shape[3]
    return B, T, H, HV, K, V, N


def _run(fn_name, q, k, v, gate_args, beta, cu_seqlens, h0, scale, units,
         nthreads, lib):
    lib = lib or load()
    B, T, H, HV, K, V, N = _shapes(q, v, cu_seqlens)
    q, k, v, beta, h0 = (_f64(x) for x in (q, k, v, beta, h0))
    gate_args = [_f64(a) for a in gate_args]
    cu = None if cu_seqlens is None else np.ascontiguousarray(np.asarray(cu_seqlens, np.int64))
    un = None if units is None else np.ascontiguousarray(np.asarray(units, np.int32))
    o = np.zeros((B, T, HV, V), np.float64)
    fin = np.zeros((N, HV, K, V), np.float64)
    if fn_name == "gdn_oracle_fwd":
        g_raw, A_log, dt_bias = gate_args
        rc = lib.gdn_oracle_fwd(
            B, T, H, HV, K, V, _ptr(cu, _i64p), N, _ptr(q), _ptr(k), _ptr(v),
            _ptr(g_raw), _ptr(beta), _ptr(A_log), _ptr(dt_bias), _ptr(h0),
            float(scale), _ptr(un, _i32p), 0 if un is None else len(un),
            _ptr(o), _ptr(fin), int(nthreads or default_threads()))
    else:
        (g,) = gate_args
        rc = lib.gdn_oracle_recurrence(
            B, T, H, HV, K, V, _ptr(cu, _i64p), N, _ptr(q), _ptr(k), _ptr(v),
            _ptr(g), _ptr(beta), _ptr(h0),
            float(scale), _ptr(un, _i32p), 0 if un is None else len(un),
            _ptr(o), _ptr(fin), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle returned error code %d" % rc)
    return o, fin


def fwd(q, k, v, g_raw, beta, A_log, dt_bias=None, cu_seqlens=None, h0=None,
        scale=1.0, units=None, nthreads=None, lib=None):
    """Oracle forward pass (gate + token recurrence), all in fp64.

    q, k: [B,T,H,K]; v: [B,T,HV,V]; g_raw, beta: [B,T,HV]; A_log, dt_bias: [HV];
    cu_seqlens: None or N+1 int64 offsets (then B == 1); h0: None or [N,HV,K,V].
    units: optional list of n*HV+hv ids to compute (others stay zero).
    Returns (o [B,T,HV,V], final_state [N,HV,K,V]) as float64 arrays.
    """
    return _run("gdn_oracle_fwd", q, k, v, [g_raw, A_log, dt_bias], beta,
                cu_seqlens, h0, scale, units, nthreads, lib)


def ref_fwd(q, k, v, g_raw, beta, A_log, dt_bias=None, cu_seqlens=None, initial_state=None,
            scale=1.0, nthreads=None, lib=None):
    """gdn_ref_fwd: the oracle forward pass called with gdn_fwd's argument
    order (q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state ->
    o, final_state).  Same arrays and results as ``fwd``."""
    lib = lib or load()
    B, T, H, HV, K, V, N = _shapes(q, v, cu_seqlens)
    q, k, v, g_raw, beta, A_log, dt_bias, h0 = (
        _f64(x) for x in (q, k, v, g_raw, beta, A_log, dt_bias, initial_state))
    cu = None if cu_seqlens is None else np.ascontiguousarray(np.asarray(cu_seqlens, np.int64))
    o = np.zeros((B, T, HV, V), np.float64)
    fin = np.zeros((N, HV, K, V), np.float64)
    rc = lib.gdn_ref_fwd(B, T, H, HV, K, V, N if cu is not None else 0, float(scale),
                         _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta), _ptr(A_log),
                         _ptr(dt_bias), _ptr(cu, _i64p), _ptr(h0), _ptr(o), _ptr(fin),
                         int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle returned error code %d" % rc)
    return o, fin


def recurrence(q, k, v, g, beta, cu_seqlens=None, h0=None, scale=1.0,
               units=None, nthreads=None, lib=None):
    """Token recurrence from a given log-decay g [B,T,HV] (fp64)."""
    return _run("gdn_oracle_recurrence", q, k, v, [g], beta, cu_seqlens, h0,
                scale, units, nthreads, lib)


def bwd(q, k, v, g_raw, beta, A_log, dt_bias, do, dht=None, cu_seqlens=None, h0=None,
        scale=1.0, units=None, nthreads=None, lib=None):
    """Oracle backward pass in fp64: gradients of L = sum <do, o> + <dht, final
    state> for the forward pass ``fwd`` with the same arguments.

    do: [B,T,HV,V]; dht: None (zero) or [N,HV,K,V].  units: optional list of
    n*HV+hv ids; only they contribute (dv, dg_raw, dbeta, dh0 of others stay 0).
    Returns a dict of float64 arrays: dq, dk [B,T,H,K]; dv [B,T,HV,V];
    dg_raw, dbeta [B,T,HV]; dA_log, ddt_bias [HV] (ddt_bias None without a
    bias); dh0 [N,HV,K,V].
    """
    lib = lib or load()
    B, T, H, HV, K, V, N = _shapes(q, v, cu_seqlens)
    q, k, v, beta, h0, g_raw, A_log, dt_bias, do, dht = (
        _f64(x) for x in (q, k, v, beta, h0, g_raw, A_log, dt_bias, do, dht))
    cu = None if cu_seqlens is None else np.ascontiguousarray(np.asarray(cu_seqlens, np.int64))
    un = None if units is None else np.ascontiguousarray(np.asarray(units, np.int32))
    out = dict(dq=np.zeros((B, T, H, K)), dk=np.zeros((B, T, H, K)),
               dv=np.zeros((B, T, HV, V)), dg_raw=np.zeros((B, T, HV)),
               dbeta=np.zeros((B, T, HV)), dA_log=np.zeros(HV),
               ddt_bias=None if dt_bias is None else np.zeros(HV),
               dh0=np.zeros((N, HV, K, V)))
    rc = lib.gdn_oracle_bwd(
        B, T, H, HV, K, V, _ptr(cu, _i64p), N, _ptr(q), _ptr(k), _ptr(v),
        _ptr(g_raw), _ptr(beta), _ptr(A_log), _ptr(dt_bias), _ptr(h0), float(scale),
        _ptr(do), _ptr(dht), _ptr(un, _i32p), 0 if un is None else len(un),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg_raw"]),
        _ptr(out["dbeta"]), _ptr(out["dA_log"]), _ptr(out["ddt_bias"]), _ptr(out["dh0"]),
        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle returned error code %d" % rc)
    return out
