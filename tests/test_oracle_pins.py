"""The fp64 oracle against library routines, closed forms and invariants (see oracle_pins.py)."""
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.load())


def test_default_scales():
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(5))
    q = rng.standard_normal((1, 4, 96)).astype(np.float32)
    k = rng.standard_normal((1, 6, 2, 96)).astype(np.float32)
    v = rng.standard_normal((1, 6, 2, 96)).astype(np.float32)
    lens = np.array([6], np.int32)
    assert np.array_equal(oracle.gqa_decode(q, k, v, lens), oracle.gqa_decode(q, k, v, lens, 1.0 / np.sqrt(96.0)))
    # MLA default is 1/sqrt(nope + rope) = 1/12 at the MiniMind MLA widths (96 + 48)
    args = pins._mla_inputs(rng, 1, 8, 96, 48, 96, 128, 5)
    L = np.array([5], np.int32)
    assert np.array_equal(oracle.mla_decode_absorbed(*args, L), oracle.mla_decode_absorbed(*args, L, 1.0 / 12.0))


def test_group_count_rejected():
    import numpy as np
    with pytest.raises(ValueError):
        oracle.gqa_decode(np.zeros((1, 6, 4)), np.zeros((1, 2, 4, 4)), np.zeros((1, 2, 4, 4)), [2])
