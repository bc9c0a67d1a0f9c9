"""The parity helpers themselves (CPU): code distance and relative error."""
import numpy as np

from _parity import code_steps, rel_err


def test_code_steps_counts_signed_zero():
    a = np.array([0x00, 0x80, 0x01, 0x81, 0x7E, 0x7F, 0x10], np.uint8)
    b = np.array([0x80, 0x00, 0x01, 0x01, 0x7D, 0xFF, 0x12], np.uint8)
    assert code_steps(a, b).tolist() == [1, 1, 0, 2, 1, 254, 2]


def test_code_steps_symmetric_and_zero_on_equal():
    rng = np.random.default_rng(0)
    a = rng.integers(0, 256, 5000).astype(np.uint8)
    b = rng.integers(0, 256, 5000).astype(np.uint8)
    assert np.array_equal(code_steps(a, b), code_steps(b, a))
    assert not code_steps(a, a).any()


def test_rel_err_nan_and_zero():
    got = rel_err(np.array([np.nan, 0.0, 1.0, 2.0]), np.array([np.nan, 0.0, 0.0, 1.0]))
    assert got.tolist() == [0.0, 0.0, np.inf, 1.0]
