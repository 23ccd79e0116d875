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
