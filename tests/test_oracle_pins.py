"""The oracle against its pins (CPU only): every pin in tests/_pins.py must hold."""
import pytest

import _pins


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=[p.__name__ for p in _pins.ALL_PINS])
def test_pin(oracle_mod, pin):
    pin(oracle_mod.default())


def test_thread_count_does_not_change_result(oracle_mod):
    import numpy as np
    import pk_inputs
    A = pk_inputs.normal_bf16((37, 256), 1.0, 41)
    B = pk_inputs.normal_bf16((256, 19), 1.0, 42)
    o = oracle_mod.default()
    assert np.array_equal(o.gemm(A, B, nthreads=1), o.gemm(A, B, nthreads=5))


def test_row_sampling_matches_full(oracle_mod):
    import numpy as np
    import pk_inputs
    A = pk_inputs.normal_bf16((50, 64), 1.0, 51)
    B = pk_inputs.normal_bf16((64, 30), 1.0, 52)
    o = oracle_mod.default()
    rows = [0, 7, 49, 13]
    assert np.array_equal(o.gemm_rows(A, B, rows), o.gemm(A, B)[rows])
