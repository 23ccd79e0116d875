"""ctypes binding of libgdn.so: same entry points as include/gdn.h.

Argument marshalling only.  No fallback: if the library is missing or the
device is not a GPU, calls raise.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "libgdn.so")
_LIB = None

GDN_F32 = 0
GDN_BF16 = 1
GDN_F16 = 2  # KDA gate only

SYMBOLS = ("gdn_fwd_workspace_size", "gdn_fwd_workspace_layout", "gdn_fwd_check",
           "gdn_fwd", "gdn_fwd_timed", "gdn_fwd_stages", "gdn_decode", "gdn_kda_gate",
           "gdn_bwd_workspace_size", "gdn_bwd", "gdn_bwd_timed", "gdn_status_string",
           "gdn_fwd_fuses_output", "gdn_fwd_noalloc", "gdn_fwd_seg_chunks")
GDN_SEG_AUTO = -1  # include/gdn.h: seg_chunks chosen per call
GDN_SCRATCH_BYTES = 64 << 20  # include/gdn.h: the static workspace of gdn_fwd_noalloc
NUM_STAGES = 4
STAGES = ("chunk_map", "wy", "chain", "output")
# gdn_fwd_stages bits, one per entry of STAGES
STAGE_BITS = {name: 1 << i for i, name in enumerate(STAGES)}
STAGE_ALL = (1 << len(STAGES)) - 1
BWD_NUM_STAGES = 6
BWD_STAGES = ("recompute", "prep", "bwd_chain", "dqk", "bwd_wy", "sums")


class Params(ctypes.Structure):
    """gdn_params_t."""
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("seg_chunks", ctypes.c_int32)]


class WorkspaceLayout(ctypes.Structure):
    """gdn_workspace_layout_t."""
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("gamma", "beta", "w", "kt", "u", "hc", "vn", "pm", "chunk_map", "seq_slot",
                 "seq_order",
                 "seg_slot", "seq_seg", "seg_e", "seg_m", "seg_h", "total")] + [
                    ("num_slots", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                    ("num_segs", ctypes.c_int32)]


class GdnError(RuntimeError):
    def __init__(self, status, where="gdn_fwd"):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def lib_path():
    return _LIB_PATH


def load_library(path=None):
    """Load libgdn.so (raises OSError if it has not been built).

    torch is imported first: torch ships its own HIP runtime, and libgdn.so
    loaded before it would bind to the system's copy instead, leaving two
    runtimes in the process, so that torch's device pointers and streams
    are not valid in the library (every launch then fails)."""
    global _LIB
    _torch()
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            raise OSError("libgdn.so not found at %s; build it with "
                          "`python -m gated_deltanet_chunkwise_amd.build`" % _LIB_PATH)
        _LIB = _declare(ctypes.CDLL(_LIB_PATH))
    return _LIB


def _declare(lib):
    vp, fp = ctypes.c_void_p, ctypes.c_void_p
    P = ctypes.POINTER(Params)
    lib.gdn_fwd_workspace_size.restype = ctypes.c_size_t
    lib.gdn_fwd_workspace_size.argtypes = [P, ctypes.c_int]
    lib.gdn_fwd_workspace_layout.restype = ctypes.c_int
    lib.gdn_fwd_workspace_layout.argtypes = [P, ctypes.c_int, ctypes.POINTER(WorkspaceLayout)]
    lib.gdn_fwd_check.restype = ctypes.c_int
    lib.gdn_fwd_check.argtypes = [P] + [vp] * 12 + [ctypes.c_size_t]
    lib.gdn_fwd.restype = ctypes.c_int
    lib.gdn_fwd.argtypes = [P] + [vp] * 12 + [ctypes.c_size_t, fp]
    lib.gdn_fwd_timed.restype = ctypes.c_int
    lib.gdn_fwd_timed.argtypes = [P] + [vp] * 12 + [ctypes.c_size_t, fp, ctypes.c_void_p]
    lib.gdn_decode.restype = ctypes.c_int
    lib.gdn_decode.argtypes = [P] + [vp] * 9 + [fp]
    lib.gdn_kda_gate.restype = ctypes.c_int
    lib.gdn_kda_gate.argtypes = [vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, ctypes.c_int64,
                                 ctypes.c_int32, ctypes.c_int32, fp]
    lib.gdn_fwd_stages.restype = ctypes.c_int
    lib.gdn_fwd_stages.argtypes = [P] + [vp] * 12 + [ctypes.c_size_t, ctypes.c_uint, fp]
    lib.gdn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.gdn_bwd_workspace_size.argtypes = [P, ctypes.c_int]
    lib.gdn_bwd.restype = ctypes.c_int
    lib.gdn_bwd.argtypes = [P] + [vp] * 20 + [ctypes.c_size_t, fp]
    lib.gdn_bwd_timed.restype = ctypes.c_int
    lib.gdn_bwd_timed.argtypes = [P] + [vp] * 20 + [ctypes.c_size_t, fp, ctypes.c_void_p]
    lib.gdn_fwd_fuses_output.restype = ctypes.c_int
    lib.gdn_fwd_fuses_output.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_int32)]
    lib.gdn_fwd_seg_chunks.restype = ctypes.c_int
    lib.gdn_fwd_seg_chunks.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_int32)]
    lib.gdn_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_fwd_noalloc.argtypes = [P] + [vp] * 11 + [fp]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    return lib


def status_string(status):
    return load_library().gdn_status_string(int(status)).decode()


def make_params(B, T, H, HV, K, V, dtype, num_seqs=0, scale=1.0, seg_chunks=0):
    return Params(int(B), int(T), int(H), int(HV), int(K), int(V), int(num_seqs), int(dtype),
                  float(scale), int(seg_chunks))


def workspace_size(params, packed=False):
    return int(load_library().gdn_fwd_workspace_size(ctypes.byref(params), int(bool(packed))))


def workspace_layout(params, packed=False):
    lay = WorkspaceLayout()
    st = load_library().gdn_fwd_workspace_layout(ctypes.byref(params), int(bool(packed)),
                                                 ctypes.byref(lay))
    if st:
        raise GdnError(st, "gdn_fwd_workspace_layout")
    return lay


def fuses_output(params, packed=False):
    """gdn_fwd_fuses_output: True when gdn_fwd runs the output stage inside the
    state pass for these parameters on the current device."""
    f = ctypes.c_int32(0)
    st = load_library().gdn_fwd_fuses_output(ctypes.byref(params), int(bool(packed)),
                                             ctypes.byref(f))
    if st:
        raise GdnError(st, "gdn_fwd_fuses_output")
    return bool(f.value)


def seg_chunks(params, packed=False):
    """gdn_fwd_seg_chunks: the segment length gdn_fwd uses for these parameters
    on the current device (0 = the plain state pass)."""
    L = ctypes.c_int32(0)
    st = load_library().gdn_fwd_seg_chunks(ctypes.byref(params), int(bool(packed)),
                                           ctypes.byref(L))
    if st:
        raise GdnError(st, "gdn_fwd_seg_chunks")
    return int(L.value)


def check(params, ptrs, workspace_bytes):
    """gdn_fwd_check with raw integer pointers (12 of them, gdn_fwd's order)."""
    return int(load_library().gdn_fwd_check(ctypes.byref(params), *ptrs, int(workspace_bytes)))


# ---------------------------------------------------------------------------
# torch-facing wrapper

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensor(name, t, shape, dtype, required=True):
    """Raise ValueError / TypeError unless `t` has exactly `shape` and `dtype`
    (None is accepted when not required)."""
    if t is None:
        if required:
            raise ValueError("%s is required" % name)
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _check_placement(named, device):
    """Every given tensor contiguous and on `device` (checked after the shapes)."""
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda or t.device != device:
            raise ValueError("%s must be a GPU tensor on %s, got %s" % (name, device, t.device))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def _check_forward_inputs(plan, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens,
                          initial_state):
    """The forward inputs against a plan's sizes and dtype (include/gdn.h layouts)."""
    torch = _torch()
    B, T, H, HV, K, V = plan.dims
    f32 = torch.float32
    if (cu_seqlens is not None) != plan.packed:
        raise ValueError("cu_seqlens given/omitted inconsistently with the plan")
    _check_tensor("q", q, (B, T, H, K), plan.dtype)
    _check_tensor("k", k, (B, T, H, K), plan.dtype)
    _check_tensor("v", v, (B, T, HV, V), plan.dtype)
    _check_tensor("g_raw", g_raw, (B, T, HV), f32)
    _check_tensor("beta", beta, (B, T, HV), f32)
    _check_tensor("A_log", A_log, (HV,), f32)
    _check_tensor("dt_bias", dt_bias, (HV,), f32, required=False)
    _check_tensor("cu_seqlens", cu_seqlens, (plan.N + 1,), torch.int64, required=plan.packed)
    _check_tensor("initial_state", initial_state, (plan.N, HV, K, V), f32, required=False)
    return [("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta", beta), ("A_log", A_log),
            ("dt_bias", dt_bias), ("cu_seqlens", cu_seqlens), ("initial_state", initial_state)]


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.bfloat16:
        return GDN_BF16
    if dt == torch.float32:
        return GDN_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % dt)


class GdnForward:
    """A planned forward pass: outputs and workspace allocated once, so that
    calling it launches the kernels and allocates nothing.

    Shapes follow include/gdn.h: q, k [B,T,H,K]; v [B,T,HV,V]; g_raw, beta
    [B,T,HV] fp32; A_log, dt_bias [HV] fp32; cu_seqlens [N+1] int64 (B == 1);
    initial_state [N,HV,K,V] fp32.
    """

    def __init__(self, B, T, H, HV, K, V, dtype, device, num_seqs=None, scale=1.0,
                 final_state=True, seg_chunks=0):
        torch = _torch()
        self.packed = num_seqs is not None
        self.N = num_seqs if self.packed else B
        self.dims = (B, T, H, HV, K, V)
        self.dtype = dtype
        self.params = make_params(B, T, H, HV, K, V, _dtype_code(dtype),
                                  num_seqs if self.packed else 0, scale, seg_chunks)
        self.lib = load_library()
        self.layout = workspace_layout(self.params, self.packed)  # raises on bad sizes
        self.ws_bytes = int(self.layout.total)
        # 256-byte aligned (torch's caching allocator aligns blocks to at least 512)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.o = torch.empty((B, T, HV, V), dtype=dtype, device=device)
        self.final_state = (torch.empty((self.N, HV, K, V), dtype=torch.float32, device=device)
                            if final_state else None)

    def _args(self, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, stream):
        """Checked ctypes argument tuple of gdn_fwd (host-side checks only): every
        tensor's shape and dtype against the plan, then device and contiguity,
        then gdn_fwd_check; raises before anything is launched."""
        torch = _torch()
        named = _check_forward_inputs(self, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens,
                                      initial_state)
        _check_placement(named, self.o.device)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        args = (ctypes.byref(self.params), _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta),
                _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(initial_state), _ptr(self.o),
                _ptr(self.final_state), _ptr(self.workspace), self.ws_bytes,
                ctypes.c_void_p(stream.cuda_stream))
        st = self.lib.gdn_fwd_check(*args[:-1])
        if st:
            raise GdnError(st, "gdn_fwd_check")
        return args

    def __call__(self, q, k, v, g_raw, beta, A_log, dt_bias=None, cu_seqlens=None,
                 initial_state=None, stream=None, events=None):
        """Launch on `stream` (default: torch's current stream).  `events`: optional
        ctypes array of NUM_STAGES + 1 hipEvent_t recorded around the stages."""
        args = self._args(q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, stream)
        if events is None:
            st = self.lib.gdn_fwd(*args)
        else:
            st = self.lib.gdn_fwd_timed(*args, ctypes.cast(events, ctypes.c_void_p))
        if st:
            raise GdnError(st)
        return self.o, self.final_state

    def bind(self, q, k, v, g_raw, beta, A_log, dt_bias=None, cu_seqlens=None,
             initial_state=None, stream=None, stage_mask=None):
        """Marshal and check the arguments once (nothing is launched); returns a
        zero-argument callable that launches the pass (for hot loops: no
        per-call Python checks).  `stage_mask` (STAGE_BITS values) restricts it
        to those stages, through gdn_fwd_stages: meaningful once a full call
        has filled the workspace, and with cu_seqlens a mask without the
        chunk-map stage requires it (its index tables become addresses)."""
        args = self._args(q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, stream)
        keep = (q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state)
        if stage_mask is None:
            fn = self.lib.gdn_fwd
        else:
            st_fn = self.lib.gdn_fwd_stages
            mask = ctypes.c_uint(stage_mask)
            args, stream_arg = args[:-1], args[-1]
            fn = lambda *a: st_fn(*a, mask, stream_arg)  # noqa: E731

        def launch():
            keep  # the tensors stay alive as long as the callable
            st = fn(*args)
            if st:
                raise GdnError(st)
        return launch


def _any_dtype_code(dt):
    torch = _torch()
    codes = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16, torch.float16: GDN_F16}
    if dt not in codes:
        raise TypeError("dtype must be float32, bfloat16 or float16, got %s" % dt)
    return codes[dt]


def decode_launcher(q, k, v, g_raw, beta, A_log, state, dt_bias=None, scale=1.0, out=None,
                    stream=None):
    """Check and marshal gdn_decode's arguments once; returns (launch, o), where
    launch() enqueues the recurrent step over q's T tokens, updating `state` in
    place.  q, k [B,T,H,K] and v [B,T,HV,V] in bf16 or fp32; g_raw, beta
    [B,T,HV], A_log [HV], dt_bias [HV] or None, state [B,HV,K,V], all fp32."""
    torch = _torch()
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes or dtypes disagree")
    if g_raw.shape != (B, T, HV) or beta.shape != (B, T, HV) or state.shape != (B, HV, K, V):
        raise ValueError("g_raw, beta must be [B,T,HV] and state [B,HV,K,V]")
    if A_log.shape != (HV,) or (dt_bias is not None and dt_bias.shape != (HV,)):
        raise ValueError("A_log and dt_bias must be [HV]")
    if out is not None and (out.shape != (B, T, HV, V) or out.dtype != q.dtype):
        raise ValueError("out must be [B,T,HV,V] in q's dtype")
    for name, t in (("g_raw", g_raw), ("beta", beta), ("A_log", A_log), ("dt_bias", dt_bias),
                    ("state", state)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("%s must be float32" % name)
    if out is None:
        out = torch.empty((B, T, HV, V), dtype=q.dtype, device=q.device)
    for name, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta", beta),
                    ("A_log", A_log), ("dt_bias", dt_bias), ("state", state), ("out", out)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous GPU tensor" % name)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    params = make_params(B, T, H, HV, K, V, _dtype_code(q.dtype), 0, scale)
    fn = load_library().gdn_decode
    args = (ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta), _ptr(A_log),
            _ptr(dt_bias), _ptr(state), _ptr(out), ctypes.c_void_p(stream.cuda_stream))
    keep = (params, q, k, v, g_raw, beta, A_log, dt_bias, state, out)

    def launch():
        keep  # the tensors stay alive as long as the callable
        st = fn(*args)
        if st:
            raise GdnError(st, "gdn_decode")
    return launch, out


def decode(q, k, v, g_raw, beta, A_log, state, dt_bias=None, scale=1.0, out=None, stream=None):
    """Recurrent GDN step(s) through gdn_decode: returns o [B,T,HV,V] and leaves the
    state after the T tokens in `state` (updated in place)."""
    launch, out = decode_launcher(q, k, v, g_raw, beta, A_log, state, dt_bias, scale, out, stream)
    launch()
    return out


def kda_gate(g, A_log, dt_bias=None, output_dtype=None, out=None, stream=None):
    """KDA per-channel gate through gdn_kda_gate: g [..., H, D] (fp32 / bf16 / fp16),
    A_log [H] fp32, dt_bias [H*D] (or [H, D]) fp32 or None.  Returns yg, shaped
    like g, in output_dtype (default: g's dtype), or written into `out`.
    `out` may be g itself (in place) when the dtypes match."""
    launch, out = kda_gate_launcher(g, A_log, dt_bias, output_dtype, out, stream)
    launch()
    return out


def kda_gate_launcher(g, A_log, dt_bias=None, output_dtype=None, out=None, stream=None):
    """Check and marshal kda_gate's arguments once; returns (launch, out), where
    launch() enqueues gdn_kda_gate with them (for timing loops and graph capture)."""
    torch = _torch()
    if g.dim() < 2:
        raise ValueError("g must be [..., H, D]")
    H, D = g.shape[-2:]
    T = g.numel() // (H * D) if H * D else 0
    if A_log.shape != (H,) or A_log.dtype != torch.float32:
        raise ValueError("A_log must be float32 [H]")
    if dt_bias is not None and (dt_bias.numel() != H * D or dt_bias.dtype != torch.float32):
        raise ValueError("dt_bias must be float32 with H*D elements")
    if out is None:
        out = torch.empty(g.shape, dtype=output_dtype or g.dtype, device=g.device)
    elif out.shape != g.shape:
        raise ValueError("out must have g's shape")
    for name, t in (("g", g), ("A_log", A_log), ("dt_bias", dt_bias), ("out", out)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous GPU tensor" % name)
    if stream is None:
        stream = torch.cuda.current_stream(g.device)
    fn = load_library().gdn_kda_gate
    args = (_ptr(g), _any_dtype_code(g.dtype), _ptr(A_log), _ptr(dt_bias), _ptr(out),
            _any_dtype_code(out.dtype), T, H, D, ctypes.c_void_p(stream.cuda_stream))
    keep = (g, A_log, dt_bias, out)

    def launch():
        keep  # the tensors stay alive as long as the callable
        st = fn(*args)
        if st:
            raise GdnError(st, "gdn_kda_gate")
    return launch, out


class _Dims:
    """The sizes _check_forward_inputs reads from a plan."""

    def __init__(self, B, T, H, HV, K, V, dtype, N, packed):
        self.dims, self.dtype, self.N, self.packed = (B, T, H, HV, K, V), dtype, N, packed


def fwd_noalloc(q, k, v, g_raw, beta, A_log, o, dt_bias=None, cu_seqlens=None,
                initial_state=None, final_state=None, scale=1.0, stream=None):
    """gdn_fwd_noalloc: the forward pass into caller-owned o [B,T,HV,V] (q's
    dtype) and final_state [N,HV,K,V] fp32 (or None), with the library's static
    device scratch as workspace: nothing is allocated.  Raises GdnError with
    GDN_ERR_SCRATCH when the problem needs more than GDN_SCRATCH_BYTES.  Calls
    that overlap on one GPU race on its scratch (see include/gdn.h)."""
    torch = _torch()
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    packed = cu_seqlens is not None
    N = cu_seqlens.numel() - 1 if packed else B
    dims = _Dims(B, T, H, HV, K, V, q.dtype, N, packed)
    named = _check_forward_inputs(dims, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens,
                                  initial_state)
    _check_tensor("o", o, (B, T, HV, V), q.dtype)
    _check_tensor("final_state", final_state, (N, HV, K, V), torch.float32, required=False)
    _check_placement(named + [("o", o), ("final_state", final_state)], q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    params = make_params(B, T, H, HV, K, V, _dtype_code(q.dtype), N if packed else 0, scale)
    st = load_library().gdn_fwd_noalloc(
        ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta), _ptr(A_log),
        _ptr(dt_bias), _ptr(cu_seqlens), _ptr(initial_state), _ptr(o), _ptr(final_state),
        ctypes.c_void_p(stream.cuda_stream))
    if st:
        raise GdnError(st, "gdn_fwd_noalloc")
    return o, final_state


def fwd(q, k, v, g_raw, beta, A_log, dt_bias=None, cu_seqlens=None, initial_state=None,
        scale=1.0, output_final_state=True):
    """One forward pass; allocates o, final_state and the workspace with torch.

    Returns (o [B,T,HV,V] in q's dtype, final_state [N,HV,K,V] fp32 or None).
    """
    torch = _torch()
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T):
        raise ValueError("shape mismatch between q, k and v")
    if g_raw.shape != (B, T, HV) or beta.shape != (B, T, HV):
        raise ValueError("g_raw and beta must be [B,T,HV]")
    if g_raw.dtype != torch.float32 or beta.dtype != torch.float32 or A_log.dtype != torch.float32:
        raise TypeError("g_raw, beta, A_log (and dt_bias) must be float32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int64:
        raise TypeError("cu_seqlens must be int64")
    num_seqs = None if cu_seqlens is None else cu_seqlens.numel() - 1
    plan = GdnForward(B, T, H, HV, K, V, q.dtype, q.device, num_seqs=num_seqs, scale=scale,
                      final_state=output_final_state)
    return plan(q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state)


class GdnBackward:
    """A planned backward pass (gdn_bwd): gradient outputs and workspace
    allocated once, so that calling it launches the kernels and allocates
    nothing.  Inputs as for GdnForward, plus d_o [B,T,HV,V] (q's dtype) and
    d_final_state [N,HV,K,V] fp32 or None.  Outputs (attributes, overwritten
    by each call): dq, dk [B,T,H,K] and dv [B,T,HV,V] in q's dtype; dg_raw,
    dbeta [B,T,HV], dA_log [HV], ddt_bias [HV] and d_initial_state
    [N,HV,K,V] in fp32.
    """

    def __init__(self, B, T, H, HV, K, V, dtype, device, num_seqs=None, scale=1.0):
        torch = _torch()
        self.packed = num_seqs is not None
        self.N = num_seqs if self.packed else B
        self.dims = (B, T, H, HV, K, V)
        self.dtype = dtype
        self.params = make_params(B, T, H, HV, K, V, _dtype_code(dtype),
                                  num_seqs if self.packed else 0, scale)
        self.lib = load_library()
        workspace_layout(self.params, self.packed)  # raises on bad sizes
        self.ws_bytes = int(self.lib.gdn_bwd_workspace_size(ctypes.byref(self.params),
                                                            int(self.packed)))
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        f32 = torch.float32
        self.dq = torch.empty((B, T, H, K), dtype=dtype, device=device)
        self.dk = torch.empty((B, T, H, K), dtype=dtype, device=device)
        self.dv = torch.empty((B, T, HV, V), dtype=dtype, device=device)
        self.dg_raw = torch.empty((B, T, HV), dtype=f32, device=device)
        self.dbeta = torch.empty((B, T, HV), dtype=f32, device=device)
        self.dA_log = torch.empty((HV,), dtype=f32, device=device)
        self.ddt_bias = torch.empty((HV,), dtype=f32, device=device)
        self.d_initial_state = torch.empty((self.N, HV, K, V), dtype=f32, device=device)

    def grads(self):
        return dict(dq=self.dq, dk=self.dk, dv=self.dv, dg_raw=self.dg_raw, dbeta=self.dbeta,
                    dA_log=self.dA_log, ddt_bias=self.ddt_bias, dh0=self.d_initial_state)

    def _args(self, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, d_o,
              d_final_state, stream):
        torch = _torch()
        B, T, H, HV, K, V = self.dims
        named = _check_forward_inputs(self, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens,
                                      initial_state)
        _check_tensor("d_o", d_o, (B, T, HV, V), self.dtype)
        _check_tensor("d_final_state", d_final_state, (self.N, HV, K, V), torch.float32,
                      required=False)
        _check_placement(named + [("d_o", d_o), ("d_final_state", d_final_state)],
                         self.dq.device)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        return (ctypes.byref(self.params), _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta),
                _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(initial_state), _ptr(d_o),
                _ptr(d_final_state), _ptr(self.dq), _ptr(self.dk), _ptr(self.dv),
                _ptr(self.dg_raw), _ptr(self.dbeta), _ptr(self.dA_log), _ptr(self.ddt_bias),
                _ptr(self.d_initial_state), _ptr(self.workspace), self.ws_bytes,
                ctypes.c_void_p(stream.cuda_stream))

    def __call__(self, q, k, v, g_raw, beta, A_log, dt_bias, d_o, d_final_state=None,
                 cu_seqlens=None, initial_state=None, stream=None, events=None):
        """Launch on `stream` (default: torch's current stream); returns grads().
        `events`: optional ctypes array of BWD_NUM_STAGES + 1 hipEvent_t."""
        args = self._args(q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, d_o,
                          d_final_state, stream)
        if events is None:
            st = self.lib.gdn_bwd(*args)
        else:
            st = self.lib.gdn_bwd_timed(*args, ctypes.cast(events, ctypes.c_void_p))
        if st:
            raise GdnError(st, "gdn_bwd")
        return self.grads()

    def bind(self, q, k, v, g_raw, beta, A_log, dt_bias, d_o, d_final_state=None,
             cu_seqlens=None, initial_state=None, stream=None):
        """Marshal the arguments once; returns a zero-argument launcher."""
        args = self._args(q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, d_o,
                          d_final_state, stream)
        keep = (q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, d_o,
                d_final_state)
        fn = self.lib.gdn_bwd

        def launch():
            keep  # the tensors stay alive as long as the callable
            st = fn(*args)
            if st:
                raise GdnError(st, "gdn_bwd")
        return launch


_GATED_DELTA_RULE = None


def _gated_delta_rule_fn():
    """The torch.autograd.Function behind gated_delta_rule (defined on first use,
    since torch is imported lazily)."""
    global _GATED_DELTA_RULE
    if _GATED_DELTA_RULE is None:
        torch = _torch()

        class GatedDeltaRule(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state,
                        scale):
                o, fin = fwd(q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state,
                             scale=scale)
                ctx.save_for_backward(q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens,
                                      initial_state)
                ctx.scale = scale
                return o, fin

            @staticmethod
            def backward(ctx, d_o, d_fin):
                q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, h0 = ctx.saved_tensors
                B, T = q.shape[0], q.shape[1]
                HV, V = v.shape[2], v.shape[3]
                # torch may hand over expanded or strided gradients; the library
                # takes dense row-major buffers
                if d_o is None:
                    d_o = torch.zeros((B, T, HV, V), dtype=q.dtype, device=q.device)
                d_o = d_o.to(q.dtype).contiguous()
                if d_fin is not None:
                    d_fin = d_fin.to(torch.float32).contiguous()
                gr = bwd(q, k, v, g_raw, beta, A_log, dt_bias, d_o, d_fin,
                         cu_seqlens=cu_seqlens, initial_state=h0, scale=ctx.scale)
                return (gr["dq"], gr["dk"], gr["dv"], gr["dg_raw"], gr["dbeta"], gr["dA_log"],
                        gr["ddt_bias"] if dt_bias is not None else None, None,
                        gr["dh0"] if h0 is not None else None, None)

        _GATED_DELTA_RULE = GatedDeltaRule
    return _GATED_DELTA_RULE


def gated_delta_rule(q, k, v, g_raw, beta, A_log, dt_bias=None, cu_seqlens=None,
                     initial_state=None, scale=1.0):
    """fwd() as a differentiable torch op: returns (o, final_state) like fwd();
    their gradients run gdn_bwd (which recomputes the forward's intermediates)
    and reach q, k, v, g_raw, beta, A_log, dt_bias and initial_state.  Inputs
    as for fwd(): contiguous GPU tensors of the documented shapes and dtypes."""
    return _gated_delta_rule_fn().apply(q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens,
                                        initial_state, scale)


def bwd(q, k, v, g_raw, beta, A_log, dt_bias, d_o, d_final_state=None, cu_seqlens=None,
        initial_state=None, scale=1.0):
    """One backward pass (allocates outputs and workspace with torch); returns
    the dict of GdnBackward.grads()."""
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    num_seqs = None if cu_seqlens is None else cu_seqlens.numel() - 1
    plan = GdnBackward(B, T, H, HV, K, V, q.dtype, q.device, num_seqs=num_seqs, scale=scale)
    return plan(q, k, v, g_raw, beta, A_log, dt_bias, d_o, d_final_state, cu_seqlens,
                initial_state)
