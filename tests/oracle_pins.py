"""Pins of the fp64 oracle to facts other than itself.

Each pin takes an oracle library handle (oracle.load() or a build with a
planted mistake) and raises AssertionError when the oracle disagrees with:
  * closed forms and identities of the gate (softplus(0) = ln 2,
    softplus(x) - softplus(-x) = x, the identity branch above 20 from the KDA
    gate guide, "core computation logic");
  * the literal matrix form of the gated delta rule, brute force at T <= 16,
    and its unrolled transition product;
  * identities of the recurrence (no write + no decay keeps the state; full
    decay resets it; orthonormal keys with beta = 1 store and retrieve values
    exactly; a re-written key returns its newest value; g = 0 is the
    Widrow-Hoff / LMS delta rule; K = V = 1 is a scalar linear recurrence with
    a product-sum closed form);
  * the independent chunkwise (WY) reformulation at several chunk sizes with
    ragged tails;
  * invariants: packed = separate sequences, state passing, grouped heads =
    repeated heads, causality, joint linearity in (v, h0), scale;
  * for the backward: central finite differences of the forward oracle's
    L = sum <do, o> + <dht, final state> in every input, the closed form of
    the gradients when all keys are zero (the state then only decays), and
    the independent chunkwise derivation of the gradient at several chunk
    sizes.
"""
import math

import numpy as np

import oracle
from oracle import chunkwise

TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * ref, "%s: max abs err %.3e (ref %.3e)" % (what, err, ref)


def _rand(rng, B, T, H, HV, K, V, g_lo=-1.5, g_hi=-0.01, unit=True):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, HV, V))
    g = rng.uniform(g_lo, g_hi, (B, T, HV))
    beta = rng.uniform(0.05, 0.95, (B, T, HV))
    return q, k, v, g, beta


# ---------------------------------------------------------------------------
# gate

def pin_gate(lib):
    A = np.array([0.0, math.log(3.0), -1.0, 2.0])
    z = np.zeros(4)
    # softplus(0) = ln 2, so g = -exp(A_log) ln 2
    g0 = oracle.gate(np.zeros((1, 4)), A, z, lib=lib)
    _close(g0[0], -np.exp(A) * math.log(2.0), 1e-15, "gate at 0")
    # exp(A_log) is a pure scale: A_log = ln 3 triples g(A_log = 0)
    x = np.linspace(-8, 8, 33)
    raw = np.stack([x, x, x, x], axis=1)
    g = oracle.gate(raw, A, z, lib=lib)
    _close(g[:, 1], 3.0 * g[:, 0], 1e-14, "A_log scale")
    # softplus(x) - softplus(-x) = x for every x (odd part of softplus)
    xs = np.array([0.3, 1.0, 5.0, 10.0, 15.0, 19.9])
    gp = oracle.gate(xs[:, None], A[:1], z[:1], lib=lib)[:, 0]
    gm = oracle.gate(-xs[:, None], A[:1], z[:1], lib=lib)[:, 0]
    _close(-(gp - gm), xs, 1e-13, "softplus odd part")
    # above 20 the guide's softplus is the identity, exactly
    big = np.array([[20.5], [33.0], [1e6]])
    _close(oracle.gate(big, A[:1], z[:1], lib=lib)[:, 0], -big[:, 0], 0.0, "identity branch")
    # just below: log(1+e^x) = x + log(1+e^-x)
    gb = oracle.gate(np.array([[19.5]]), A[:1], z[:1], lib=lib)[0, 0]
    assert abs(-gb - (19.5 + math.log1p(math.exp(-19.5)))) <= 1e-14 * 19.5
    assert -gb != 19.5, "softplus below 20 must not be the identity"
    # very negative: softplus(x) ~ e^x (relative)
    gn = oracle.gate(np.array([[-30.0]]), A[:1], z[:1], lib=lib)[0, 0]
    assert abs(-gn / math.exp(-30.0) - 1.0) < 1e-12
    # dt_bias shifts the argument
    db = np.array([0.25, -0.5, 1.0, 0.0])
    _close(oracle.gate(raw, A, db, lib=lib), oracle.gate(raw + db, A, z, lib=lib), 1e-15,
           "dt_bias shift")
    # a = +inf gives g = -inf (full decay); A_log = -inf gives g = 0 (no decay)
    assert oracle.gate(np.array([[np.inf]]), A[:1], z[:1], lib=lib)[0, 0] == -np.inf
    assert oracle.gate(np.array([[1.0]]), np.array([-np.inf]), z[:1], lib=lib)[0, 0] == 0.0


def pin_kda_gate(lib):
    """KDA per-channel gate: yg[t,h,d] = -exp(A_log[h]) softplus(g[t,h,d] + dt_bias[h,d])."""
    rng = np.random.default_rng(17)
    T, H, D = 7, 3, 5
    g = rng.standard_normal((T, H, D)) * 4.0
    A = rng.standard_normal(H)
    b = rng.standard_normal(H * D)
    y = oracle.kda_gate(g, A, b, lib=lib)
    # a library routine: softplus(x) = logaddexp(0, x) = log(e^0 + e^x) (below 20)
    ref = -np.exp(A)[None, :, None] * np.logaddexp(0.0, g + b.reshape(H, D)[None])
    _close(y, ref, 1e-14, "kda gate vs logaddexp")
    # indexing by hand on a tiny case: bias per (head, channel), scale per head
    for t in range(T):
        for h in range(H):
            for d in range(D):
                x = g[t, h, d] + b[h * D + d]
                want = -math.exp(A[h]) * math.log1p(math.exp(x))
                assert abs(y[t, h, d] - want) <= 1e-14 * abs(want), (t, h, d)
    # no bias = zero bias
    _close(oracle.kda_gate(g, A, None, lib=lib), oracle.kda_gate(g, A, np.zeros(H * D), lib=lib),
           0.0, "no bias")
    # shifting g by c[h,d] and the bias by -c leaves yg unchanged
    c = rng.standard_normal((H, D))
    _close(oracle.kda_gate(g + c[None], A, b - c.reshape(-1), lib=lib), y, 1e-14,
           "bias shift")
    # exp(A_log[h]) scales head h only
    A2 = A.copy()
    A2[1] += math.log(5.0)
    y2 = oracle.kda_gate(g, A2, b, lib=lib)
    _close(y2[:, 1], 5.0 * y[:, 1], 1e-14, "head scale")
    _close(np.delete(y2, 1, axis=1), np.delete(y, 1, axis=1), 0.0, "other heads")
    # identity branch above 20, exactly; D = 1 is the per-head gate of the GDN path
    big = np.full((2, H, 1), 25.0)
    _close(oracle.kda_gate(big, A, None, lib=lib)[..., 0], np.tile(-np.exp(A) * 25.0, (2, 1)), 0.0,
           "identity branch")
    g1 = rng.standard_normal((T, H, 1))
    b1 = rng.standard_normal(H)
    _close(oracle.kda_gate(g1, A, b1, lib=lib)[..., 0], oracle.gate(g1[..., 0], A, b1, lib=lib),
           0.0, "D = 1 is the per-head gate")
    # leading dimensions flatten into T
    g4 = rng.standard_normal((2, 3, H, D))
    _close(oracle.kda_gate(g4, A, b, lib=lib).reshape(-1, H, D),
           oracle.kda_gate(g4.reshape(-1, H, D), A, b, lib=lib), 0.0, "flattening")


# ---------------------------------------------------------------------------
# brute force: the literal matrix form S_t = e^g S (I - b k k^T) + b v k^T

def brute_force(q, k, v, g, beta, h0=None, scale=1.0):
    """Literal V x K matrix recurrence for one (sequence, head) stream."""
    T, K = k.shape
    V = v.shape[1]
    S = np.zeros((V, K)) if h0 is None else np.array(h0, np.float64).T.copy()
    o = np.zeros((T, V))
    for t in range(T):
        P = np.eye(K) - beta[t] * np.outer(k[t], k[t])
        S = math.exp(g[t]) * S @ P + beta[t] * np.outer(v[t], k[t])
        o[t] = scale * S @ q[t]
    return o, S.T


def pin_brute_force(lib):
    rng = np.random.default_rng(11)
    for (B, T, H, HV, K, V, use_h0, scale) in [(1, 16, 1, 1, 5, 3, False, 1.0),
                                                 (2, 9, 2, 4, 4, 6, True, 0.7),
                                                 (1, 13, 1, 2, 8, 8, True, 1.0)]:
        q, k, v, g, beta = _rand(rng, B, T, H, HV, K, V, unit=False)
        h0 = 0.3 * rng.standard_normal((B, HV, K, V)) if use_h0 else None
        o, fin = oracle.recurrence(q, k, v, g, beta, h0=h0, scale=scale, lib=lib)
        G = HV // H
        for b in range(B):
            for hv in range(HV):
                ob, Hb = brute_force(q[b, :, hv // G], k[b, :, hv // G], v[b, :, hv], g[b, :, hv],
                                     beta[b, :, hv], None if h0 is None else h0[b, hv], scale)
                _close(o[b, :, hv], ob, 1e-13, "brute o")
                _close(fin[b, hv], Hb, 1e-13, "brute state")


def pin_transition_product(lib):
    """S_T = S_0 A_1...A_T + sum_j b_j v_j k_j^T A_{j+1}...A_T, A_t = e^g (I - b k k^T)."""
    rng = np.random.default_rng(12)
    T, K, V = 12, 6, 4
    q, k, v, g, beta = _rand(rng, 1, T, 1, 1, K, V, unit=False)
    h0 = rng.standard_normal((1, 1, K, V))
    _, fin = oracle.recurrence(q, k, v, g, beta, h0=h0, lib=lib)
    A = [math.exp(g[0, t, 0]) * (np.eye(K) - beta[0, t, 0] * np.outer(k[0, t, 0], k[0, t, 0]))
         for t in range(T)]

    def prod(lo):
        M = np.eye(K)
        for t in range(lo, T):
            M = M @ A[t]
        return M

    S = h0[0, 0].T @ prod(0)
    for j in range(T):
        S = S + beta[0, j, 0] * np.outer(v[0, j, 0], k[0, j, 0]) @ prod(j + 1)
    _close(fin[0, 0], S.T, 1e-12, "transition product")


# ---------------------------------------------------------------------------
# identities of the recurrence

def pin_identities(lib):
    rng = np.random.default_rng(13)
    B, T, H, HV, K, V = 2, 10, 1, 2, 6, 5
    q, k, v, _, _ = _rand(rng, B, T, H, HV, K, V)
    h0 = rng.standard_normal((B, HV, K, V))
    zeros = np.zeros((B, T, HV))
    # beta = 0, g = 0: the state never changes, o_t = H0^T q_t
    o, fin = oracle.recurrence(q, k, v, zeros, zeros, h0=h0, lib=lib)
    _close(fin, h0, 0.0, "beta=0,g=0 state")
    for b in range(B):
        for hv in range(HV):
            _close(o[b, :, hv], q[b, :, 0] @ h0[b, hv], 1e-14, "beta=0,g=0 output")
    # g = -inf (a = +inf through the gate): H_t = b_t k_t v_t^T, o_t = b_t (k_t.q_t) v_t
    beta = rng.uniform(0.1, 0.9, (B, T, HV))
    A0, db = np.zeros(HV), np.zeros(HV)
    o, fin = oracle.fwd(q, k, v, np.full((B, T, HV), np.inf), beta, A0, db, h0=h0, lib=lib)
    for b in range(B):
        for hv in range(HV):
            kq = np.sum(k[b, :, 0] * q[b, :, 0], axis=-1)
            _close(o[b, :, hv], (beta[b, :, hv] * kq)[:, None] * v[b, :, hv], 1e-14, "reset o")
            _close(fin[b, hv], beta[b, -1, hv] * np.outer(k[b, -1, 0], v[b, -1, hv]), 1e-14,
                   "reset state")
    # g = 0, beta = 1, orthonormal keys: each stored value is retrieved exactly
    K2, V2, m = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((K2, K2)))
    keys = Qm[:, :m].T                       # m orthonormal rows
    vals = rng.standard_normal((m, V2))
    kk = keys[None, :, None, :]
    o, fin = oracle.recurrence(kk, kk, vals[None, :, None, :], np.zeros((1, m, 1)),
                               np.ones((1, m, 1)), lib=lib)
    _close(fin[0, 0].T @ keys.T, vals.T, 1e-14, "orthonormal retrieval")
    # o_t = S_t k_t with q = k: the value just written
    _close(o[0, :, 0], vals, 1e-14, "orthonormal readout")
    # re-writing the same unit key with beta = 1 returns the newest value
    u = keys[0]
    kk = np.stack([u, keys[1], u])[None, :, None, :]
    vv = rng.standard_normal((1, 3, 1, V2))
    _, fin = oracle.recurrence(kk, kk, vv, np.zeros((1, 3, 1)), np.ones((1, 3, 1)), lib=lib)
    _close(fin[0, 0].T @ u, vv[0, 2, 0], 1e-14, "rewrite")
    _close(fin[0, 0].T @ keys[1], vv[0, 1, 0], 1e-14, "rewrite keeps other key")
    # g = 0: Widrow-Hoff / LMS, S <- S + b (v - S k) k^T
    qq, k3, v3, _, b3 = _rand(rng, 1, 7, 1, 1, 4, 3, unit=False)
    S = np.zeros((3, 4))
    for t in range(7):
        S = S + b3[0, t, 0] * np.outer(v3[0, t, 0] - S @ k3[0, t, 0], k3[0, t, 0])
    _, fin = oracle.recurrence(qq, k3, v3, np.zeros((1, 7, 1)), b3, lib=lib)
    _close(fin[0, 0], S.T, 1e-14, "LMS")
    # K = V = 1: h_t = c_t h_{t-1} + d_t, c_t = e^g (1 - b k^2), d_t = b k v;
    # h_T = (prod c) h_0 + sum_j d_j prod_{i>j} c_i
    T1 = 9
    k1 = rng.uniform(-1.5, 1.5, (1, T1, 1, 1))
    v1 = rng.standard_normal((1, T1, 1, 1))
    g1 = rng.uniform(-1, 0, (1, T1, 1))
    b1 = rng.uniform(0, 1, (1, T1, 1))
    h01 = np.array([[[[0.7]]]])
    _, fin = oracle.recurrence(k1, k1, v1, g1, b1, h0=h01, lib=lib)
    c = np.exp(g1[0, :, 0]) * (1 - b1[0, :, 0] * k1[0, :, 0, 0] ** 2)
    d = b1[0, :, 0] * k1[0, :, 0, 0] * v1[0, :, 0, 0]
    closed = np.prod(c) * 0.7 + sum(d[j] * np.prod(c[j + 1:]) for j in range(T1))
    _close(fin[0, 0, 0, 0], closed, 1e-14, "scalar closed form")


# ---------------------------------------------------------------------------
# chunkwise reformulation and invariants

def pin_chunkwise(lib):
    rng = np.random.default_rng(14)
    # ragged tails, several chunk sizes, grouped heads, h0, scale
    B, T, H, HV, K, V = 2, 203, 2, 4, 8, 6
    q, k, v, g, beta = _rand(rng, B, T, H, HV, K, V)
    h0 = 0.5 * rng.standard_normal((B, HV, K, V))
    o_ref, f_ref = oracle.recurrence(q, k, v, g, beta, h0=h0, scale=0.8, lib=lib)
    for C in (16, 32, 64):
        o_c, f_c = chunkwise.fwd(q, k, v, g, beta, h0=h0, chunk=C, scale=0.8)
        _close(o_c, o_ref, 1e-12, "chunkwise o C=%d" % C)
        _close(f_c, f_ref, 1e-12, "chunkwise state C=%d" % C)
    # packed sequences with lengths around chunk edges
    lens = [1, 63, 64, 65, 10, 0, 128]
    cu = np.concatenate([[0], np.cumsum(lens)])
    Tt = int(cu[-1])
    q, k, v, g, beta = _rand(rng, 1, Tt, 1, 2, 8, 8, g_lo=-0.3)
    h0 = rng.standard_normal((len(lens), 2, 8, 8))
    o_ref, f_ref = oracle.recurrence(q, k, v, g, beta, cu_seqlens=cu, h0=h0, lib=lib)
    o_c, f_c = chunkwise.fwd(q, k, v, g, beta, cu_seqlens=cu, h0=h0, chunk=64)
    _close(o_c, o_ref, 1e-12, "chunkwise packed o")
    _close(f_c, f_ref, 1e-12, "chunkwise packed state")


def pin_invariants(lib):
    rng = np.random.default_rng(15)
    lens = [5, 17, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    Tt = int(cu[-1])
    H, HV, K, V = 2, 4, 6, 5
    q, k, v, g, beta = _rand(rng, 1, Tt, H, HV, K, V)
    h0 = rng.standard_normal((3, HV, K, V))
    o, fin = oracle.recurrence(q, k, v, g, beta, cu_seqlens=cu, h0=h0, lib=lib)
    # packed = separate runs
    for n, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        on, fn = oracle.recurrence(q[:, s:e], k[:, s:e], v[:, s:e], g[:, s:e], beta[:, s:e],
                                   h0=h0[n:n + 1], lib=lib)
        _close(o[:, s:e], on, 0.0, "packed vs separate o")
        _close(fin[n:n + 1], fn, 0.0, "packed vs separate state")
    # state passing: split the second sequence at 7
    s, e = int(cu[1]), int(cu[2])
    sl1, sl2 = slice(s, s + 7), slice(s + 7, e)
    o1, f1 = oracle.recurrence(q[:, sl1], k[:, sl1], v[:, sl1], g[:, sl1], beta[:, sl1],
                               h0=h0[1:2], lib=lib)
    o2, f2 = oracle.recurrence(q[:, sl2], k[:, sl2], v[:, sl2], g[:, sl2], beta[:, sl2], h0=f1,
                               lib=lib)
    _close(np.concatenate([o1, o2], axis=1), o[:, s:e], 1e-14, "state passing o")
    _close(f2, fin[1:2], 1e-14, "state passing state")
    # grouped heads = explicitly repeated q/k heads
    G = HV // H
    qr, kr = np.repeat(q, G, axis=2), np.repeat(k, G, axis=2)
    o_r, f_r = oracle.recurrence(qr, kr, v, g, beta, cu_seqlens=cu, h0=h0, lib=lib)
    _close(o_r, o, 0.0, "GQA o")
    _close(f_r, fin, 0.0, "GQA state")
    # causality: changing token t' changes no o_t with t < t'
    tp = 20
    v2, k2, q2 = v.copy(), k.copy(), q.copy()
    v2[:, tp] += 1.0
    k2[:, tp] = rng.standard_normal(k2[:, tp].shape)
    q2[:, tp] += 0.5
    o2, _ = oracle.recurrence(q2, k2, v2, g, beta, cu_seqlens=cu, h0=h0, lib=lib)
    _close(o2[:, :tp], o[:, :tp], 0.0, "causality")
    assert np.max(np.abs(o2[:, tp] - o[:, tp])) > 1e-3
    # joint linearity in (v, h0) for fixed q, k, g, beta
    vb = rng.standard_normal(v.shape)
    hb = rng.standard_normal(h0.shape)
    a1, a2 = 0.6, -1.7
    oa, fa = oracle.recurrence(q, k, a1 * v + a2 * vb, g, beta, cu_seqlens=cu,
                               h0=a1 * h0 + a2 * hb, lib=lib)
    ob, fb = oracle.recurrence(q, k, vb, g, beta, cu_seqlens=cu, h0=hb, lib=lib)
    _close(oa, a1 * o + a2 * ob, 1e-13, "linearity o")
    _close(fa, a1 * fin + a2 * fb, 1e-13, "linearity state")
    # scale multiplies o only
    os_, fs_ = oracle.recurrence(q, k, v, g, beta, cu_seqlens=cu, h0=h0, scale=0.25, lib=lib)
    _close(os_, 0.25 * o, 1e-15, "scale o")
    _close(fs_, fin, 0.0, "scale state")


def pin_full_forward(lib):
    """fwd = gate followed by the recurrence, with dt_bias and without."""
    rng = np.random.default_rng(16)
    B, T, H, HV, K, V = 1, 40, 1, 2, 4, 4
    q, k, v, _, beta = _rand(rng, B, T, H, HV, K, V)
    a = rng.standard_normal((B, T, HV))
    A_log = rng.uniform(0, 2, HV)
    db = 0.1 * rng.standard_normal(HV)
    o1, f1 = oracle.fwd(q, k, v, a, beta, A_log, db, lib=lib)
    g = oracle.gate(a, A_log, db, lib=lib)
    o2, f2 = oracle.recurrence(q, k, v, g, beta, lib=lib)
    _close(o1, o2, 0.0, "fwd = gate + recurrence")
    _close(f1, f2, 0.0, "fwd state")
    o3, _ = oracle.fwd(q, k, v, a + db, beta, A_log, None, lib=lib)
    _close(o3, o1, 1e-15, "dt_bias None")


def pin_segment_scan(lib):
    """The two-level form equals the flat chunkwise form (and so the token
    oracle), for several segment lengths, packed ragged sequences and h0; and a
    chunk's linear map M_c is the chunk step run with V = 0."""
    rng = np.random.default_rng(19)
    B, T, H, HV, K, V = 1, 300, 1, 2, 8, 5
    lengths = [130, 0, 65, 105]
    cu = np.cumsum([0] + lengths)
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, HV, V))
    g = -rng.uniform(0.0, 0.3, (B, T, HV))
    beta = rng.uniform(0.2, 1.0, (B, T, HV))
    h0 = rng.standard_normal((len(lengths), HV, K, V))
    o_ref, f_ref = chunkwise.fwd(q, k, v, g, beta, cu_seqlens=cu, h0=h0, chunk=16, scale=0.5)
    for L in (1, 2, 3, 100):
        o_s, f_s = chunkwise.segment_scan(q, k, v, g, beta, cu_seqlens=cu, h0=h0, chunk=16,
                                          seg_chunks=L, scale=0.5)
        _close(o_s, o_ref, 1e-11, "segment scan o (L=%d)" % L)
        _close(f_s, f_ref, 1e-11, "segment scan final (L=%d)" % L)
    # the linear part: chunk_step with zero values from X equals M_c X
    Kc, gc, bc = k[0, :16, 0], g[0, :16, 1], beta[0, :16, 1]
    X = rng.standard_normal((K, 3))
    _, HX, _ = chunkwise.chunk_step(np.zeros_like(Kc), Kc, np.zeros((16, 3)), gc, bc, X)
    _close(chunkwise.chunk_transition(Kc, gc, bc) @ X, HX, 1e-13, "chunk transition")
    # and M_c is the product of the per-token maps e^g (I - b k k^T) (transposed form)
    M = np.eye(K)
    for t in range(16):
        M = (math.exp(gc[t]) * (np.eye(K) - bc[t] * np.outer(Kc[t], Kc[t]))) @ M
    _close(chunkwise.chunk_transition(Kc, gc, bc), M, 1e-13, "transition = token product")


# ---------------------------------------------------------------------------
# backward

def _bwd_case(rng, B, T, H, HV, K, V, N):
    """Small random inputs for the backward pins (keys not normalised, so the
    rank-one updates are not special; one raw gate above the softplus identity
    threshold of 20)."""
    q = 0.7 * rng.standard_normal((B, T, H, K))
    k = 0.6 * rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, HV, V))
    g_raw = rng.standard_normal((B, T, HV))
    g_raw[0, min(2, T - 1), 0] = 25.0
    beta = rng.uniform(0.1, 0.9, (B, T, HV))
    A_log = rng.uniform(-1.0, 0.5, HV)
    dt_bias = 0.3 * rng.standard_normal(HV)
    h0 = rng.standard_normal((N, HV, K, V))
    do = rng.standard_normal((B, T, HV, V))
    dht = rng.standard_normal((N, HV, K, V))
    return dict(q=q, k=k, v=v, g_raw=g_raw, beta=beta, A_log=A_log, dt_bias=dt_bias, h0=h0), do, dht


def pin_bwd_finite_differences(lib):
    """Every gradient of the backward oracle equals the central finite
    difference (step 1e-6, fp64) of L = sum <do, o> + <dht, final state>
    computed by the forward oracle; fixed-length and packed sequences (one of
    them empty), grouped value heads, h0, dt_bias and scale."""
    rng = np.random.default_rng(31)
    cases = [dict(B=2, T=5, H=1, HV=2, K=3, V=2, cu=None),
             dict(B=1, T=7, H=2, HV=4, K=2, V=3, cu=np.array([0, 3, 3, 7]))]
    eps = 1e-6
    for c in cases:
        N = c["B"] if c["cu"] is None else len(c["cu"]) - 1
        x, do, dht = _bwd_case(rng, c["B"], c["T"], c["H"], c["HV"], c["K"], c["V"], N)
        scale = 0.7

        def loss(xx):
            o, fin = oracle.fwd(xx["q"], xx["k"], xx["v"], xx["g_raw"], xx["beta"], xx["A_log"],
                                xx["dt_bias"], cu_seqlens=c["cu"], h0=xx["h0"], scale=scale,
                                lib=lib)
            return float(np.sum(do * o) + np.sum(dht * fin))

        gr = oracle.bwd(x["q"], x["k"], x["v"], x["g_raw"], x["beta"], x["A_log"], x["dt_bias"],
                        do, dht, cu_seqlens=c["cu"], h0=x["h0"], scale=scale, lib=lib)
        names = dict(q="dq", k="dk", v="dv", g_raw="dg_raw", beta="dbeta", A_log="dA_log",
                     dt_bias="ddt_bias", h0="dh0")
        for name, gname in names.items():
            fd = np.zeros_like(x[name])
            for idx in np.ndindex(x[name].shape):
                xp = {kk: vv.copy() for kk, vv in x.items()}
                xm = {kk: vv.copy() for kk, vv in x.items()}
                xp[name][idx] += eps
                xm[name][idx] -= eps
                fd[idx] = (loss(xp) - loss(xm)) / (2 * eps)
            _close(gr[gname], fd, 2e-7, "finite differences %s (%s)" % (gname, c))


def pin_bwd_no_keys(lib):
    """With every key zero the state only decays, H_t = P_t h0 with
    P_t = prod_{s<=t} exp(g_s), and the gradients have closed forms:
    dH_t = sum_{s>=t} scale (P_s/P_t) q_s do_s^T + (P_T/P_t) dht, dh0 = dH_0,
    dq_t = scale P_t h0 do_t, dk_t = beta_t dH_t v_t, dv = dbeta = 0,
    dg_t = sum_{s>=t} scale P_s q_s^T h0 do_s + P_T <h0, dht>."""
    rng = np.random.default_rng(32)
    B, T, H, HV, K, V = 1, 6, 1, 1, 3, 2
    x, do, dht = _bwd_case(rng, B, T, H, HV, K, V, 1)
    x["k"][:] = 0.0
    x["g_raw"][0, 2, 0] = 0.4
    scale = 1.3
    gr = oracle.bwd(x["q"], x["k"], x["v"], x["g_raw"], x["beta"], x["A_log"], x["dt_bias"],
                    do, dht, h0=x["h0"], scale=scale, lib=lib)
    xg = x["g_raw"][0, :, 0] + x["dt_bias"][0]
    sp = np.log1p(np.exp(xg))
    g = -math.exp(x["A_log"][0]) * sp
    P = np.exp(np.cumsum(g))
    h0, q, v, dO, beta = x["h0"][0, 0], x["q"][0, :, 0], x["v"][0, :, 0], do[0, :, 0], x["beta"][0, :, 0]
    dH = [None] * T
    for t in range(T):
        acc = (P[-1] / P[t]) * dht[0, 0]
        for s in range(t, T):
            acc = acc + scale * (P[s] / P[t]) * np.outer(q[s], dO[s])
        dH[t] = acc
    dh0 = scale * sum(P[s] * np.outer(q[s], dO[s]) for s in range(T)) + P[-1] * dht[0, 0]
    _close(gr["dh0"][0, 0], dh0, 1e-12, "no keys: dh0")
    _close(gr["dq"][0, :, 0], np.stack([scale * P[t] * h0 @ dO[t] for t in range(T)]), 1e-12,
           "no keys: dq")
    _close(gr["dk"][0, :, 0], np.stack([beta[t] * dH[t] @ v[t] for t in range(T)]), 1e-12,
           "no keys: dk")
    _close(gr["dv"], np.zeros_like(gr["dv"]), 0.0, "no keys: dv")
    _close(gr["dbeta"], np.zeros_like(gr["dbeta"]), 0.0, "no keys: dbeta")
    dg = np.array([sum(scale * P[s] * (q[s] @ h0 @ dO[s]) for s in range(t, T))
                   + P[-1] * np.sum(h0 * dht[0, 0]) for t in range(T)])
    slope = 1.0 / (1.0 + np.exp(-xg))
    _close(gr["dg_raw"][0, :, 0], dg * (-math.exp(x["A_log"][0])) * slope, 1e-12, "no keys: dg_raw")
    _close(gr["dA_log"], [np.sum(dg * g)], 1e-12, "no keys: dA_log")
    _close(gr["ddt_bias"], [np.sum(dg * (-math.exp(x["A_log"][0])) * slope)], 1e-12,
           "no keys: ddt_bias")


def pin_bwd_chunkwise(lib):
    """The chunkwise backward (a chunk-by-chunk derivation of the WY form's
    gradient, oracle/chunkwise.py) equals the token oracle's reverse sweep, at
    chunk sizes 8, 16 and 64 over packed ragged sequences (one empty), grouped
    heads, h0 and dht.  dg_raw is compared through the gate's own derivative."""
    rng = np.random.default_rng(33)
    lengths = [37, 0, 70]
    cu = np.cumsum([0] + lengths)
    B, T, H, HV, K, V = 1, int(cu[-1]), 1, 2, 5, 4
    x, do, dht = _bwd_case(rng, B, T, H, HV, K, V, len(lengths))
    scale = 0.9
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["g_raw"], x["beta"], x["A_log"], x["dt_bias"],
                     do, dht, cu_seqlens=cu, h0=x["h0"], scale=scale, lib=lib)
    g = oracle.gate(x["g_raw"], x["A_log"], x["dt_bias"], lib=lib)
    xr = x["g_raw"] + x["dt_bias"]
    slope = np.where(xr > 20, 1.0, 1.0 / (1.0 + np.exp(-np.minimum(xr, 20))))
    for C in (8, 16, 64):
        cw = chunkwise.bwd(x["q"], x["k"], x["v"], g, x["beta"], do, dht, cu_seqlens=cu,
                           h0=x["h0"], chunk=C, scale=scale)
        for name in ("dq", "dk", "dv", "dbeta", "dh0"):
            _close(cw[name], ref[name], 1e-10, "chunkwise bwd %s (C=%d)" % (name, C))
        _close(cw["dg"] * (-np.exp(x["A_log"])) * slope, ref["dg_raw"], 1e-10,
               "chunkwise bwd dg (C=%d)" % C)


ALL_PINS = [pin_gate, pin_kda_gate, pin_brute_force, pin_transition_product, pin_identities,
            pin_chunkwise, pin_invariants, pin_full_forward, pin_segment_scan,
            pin_bwd_finite_differences, pin_bwd_no_keys, pin_bwd_chunkwise]
