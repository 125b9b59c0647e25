"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle
from oracle_pins import (FAST_CHECKS, check_activation_closed_forms, check_finite_differences)


@pytest.mark.parametrize("name,check", FAST_CHECKS, ids=[n for n, _ in FAST_CHECKS])
def test_oracle_pin(oracle_lib, name, check):
    check(oracle)


def test_activation_closed_forms(oracle_lib):
    check_activation_closed_forms(oracle_lib)


@pytest.mark.parametrize("act,window,gate,self_attn", [
    ("gelu", (-1, -1), False, False),
    ("silu", (-1, -1), True, False),
    ("softmax", (1, 0), True, True),
    ("softmax", (-1, -1), False, True),
    ("gelu", (0, 1), True, True),
])
def test_oracle_finite_differences(oracle_lib, act, window, gate, self_attn):
    check_finite_differences(oracle, act, 0.9, window, gate, self_attn=self_attn)


def test_oracle_rejects_bad_arguments(oracle_lib):
    import numpy as np
    q = np.zeros((2, 1, 4))
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, [0, 2, 1], [0, 1, 2], act="gelu", scale=1.0)  # decreasing offsets
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, [1, 2], [0, 2], act="gelu", scale=1.0)  # offsets[0] != 0


def test_oracle_threads_agree(oracle_lib):
    """The result does not depend on the thread count (items are independent)."""
    import numpy as np
    from oracle_pins import rand_problem
    pb = rand_problem(11, [30, 1, 17, 0, 9], None, h=3, d=16, gate=True)
    a = oracle.bwd(pb["q"], pb["k"], pb["v"], pb["do"], pb["qo"], pb["ko"], act="softmax",
                   scale=0.25, g=pb["g"], window=(4, 0), want_dg=True, nthreads=1)
    b = oracle.bwd(pb["q"], pb["k"], pb["v"], pb["do"], pb["qo"], pb["ko"], act="softmax",
                   scale=0.25, g=pb["g"], window=(4, 0), want_dg=True, nthreads=5)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
