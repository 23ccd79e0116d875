"""The fp64 oracle against closed forms, brute force, identities, the chunkwise
reformulation and invariants (see tests/oracle_pins.py)."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.load())


def test_threads_and_units_do_not_change_results():
    rng = np.random.default_rng(3)
    q, k, v, g, beta = oracle_pins._rand(rng, 3, 50, 2, 4, 8, 8)
    o1, f1 = oracle.recurrence(q, k, v, g, beta, nthreads=1)
    o8, f8 = oracle.recurrence(q, k, v, g, beta, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(f1, f8)
    units = [1, 6, 11]
    ou, fu = oracle.recurrence(q, k, v, g, beta, units=units)
    for u in units:
        n, hv = divmod(u, 4)
        assert np.array_equal(ou[n, :, hv], o1[n, :, hv])
        assert np.array_equal(fu[n, hv], f1[n, hv])
    # units not requested stay zero
    assert not ou[0, :, 0].any()


def test_invalid_arguments_rejected():
    rng = np.random.default_rng(4)
    q, k, v, g, beta = oracle_pins._rand(rng, 1, 10, 2, 3, 4, 4)  # HV % H != 0
    with pytest.raises(ValueError):
        oracle.recurrence(q, k, v, g, beta)
    q, k, v, g, beta = oracle_pins._rand(rng, 1, 10, 1, 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.recurrence(q, k, v, g, beta, cu_seqlens=[0, 4, 3, 10])  # decreasing
    with pytest.raises(ValueError):
        oracle.recurrence(q, k, v, g, beta, cu_seqlens=[0, 4, 9])  # does not end at T
    with pytest.raises(ValueError):
        oracle.recurrence(q, k, v, g, beta, units=[5])


def test_bwd_threads_and_units_do_not_change_results():
    rng = np.random.default_rng(5)
    x, do, dht = oracle_pins._bwd_case(rng, 2, 20, 1, 3, 4, 5, 2)
    args = (x["q"], x["k"], x["v"], x["g_raw"], x["beta"], x["A_log"], x["dt_bias"], do, dht)
    r1 = oracle.bwd(*args, h0=x["h0"], nthreads=1)
    r8 = oracle.bwd(*args, h0=x["h0"], nthreads=8)
    for name in r1:
        assert np.array_equal(r1[name], r8[name]), name
    # one key head read by all three value heads: the units of sequence 1 give
    # that sequence's rows in full and nothing for sequence 0
    ru = oracle.bwd(*args, h0=x["h0"], units=[3, 4, 5])
    for name in ("dq", "dk", "dv", "dg_raw", "dbeta"):
        assert np.array_equal(ru[name][1], r1[name][1]), name
        assert not ru[name][0].any(), name
    assert np.array_equal(ru["dh0"][1], r1["dh0"][1]) and not ru["dh0"][0].any()


def test_ref_fwd_twin_matches_fwd():
    """gdn_ref_fwd (gdn_fwd's argument order) gives fwd's results bit for bit,
    fixed-length and packed, with and without a bias and an initial state."""
    rng = np.random.default_rng(6)
    q, k, v, _, beta = oracle_pins._rand(rng, 2, 40, 2, 4, 8, 6)
    g_raw = rng.normal(size=(2, 40, 4))
    A_log = rng.uniform(0, 2, 4)
    dt_bias = rng.normal(0, 0.1, 4)
    h0 = rng.normal(size=(2, 4, 8, 6))
    for b, h in ((dt_bias, h0), (None, None)):
        o1, f1 = oracle.fwd(q, k, v, g_raw, beta, A_log, b, h0=h, scale=0.5)
        o2, f2 = oracle.ref_fwd(q, k, v, g_raw, beta, A_log, b, initial_state=h, scale=0.5)
        assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
    cu = np.array([0, 30, 30, 80])
    one = lambda t: t.reshape(1, 80, *t.shape[2:])  # noqa: E731
    h3 = rng.normal(size=(3, 4, 8, 6))
    o1, f1 = oracle.fwd(one(q), one(k), one(v), one(g_raw), one(beta), A_log, dt_bias,
                        cu_seqlens=cu, h0=h3)
    o2, f2 = oracle.ref_fwd(one(q), one(k), one(v), one(g_raw), one(beta), A_log, dt_bias,
                            cu_seqlens=cu, initial_state=h3)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
