"""CPU checks of the test helpers the GPU parity tests rely on: the tolerance
check rejects anything not shown to be within its bound (NaN and infinities
included), and the threaded and matmul routes to the oracle's results agree
with the oracle's own entry points."""
import numpy as np
import pytest

import oracle
from dequant_quantized_gemv_amd import synth
from tests.gpu_helpers import assert_within, gemm_reference, oracle_rows


def test_assert_within_rejects_nan_and_inf():
    ref = np.ones(3)
    s = np.ones(3)
    for bad in (np.nan, np.inf, -np.inf):
        y = np.array([1.0, bad, 1.0])
        with pytest.raises(AssertionError):
            assert_within(y, ref, s, 1e-4, "planted")
    assert_within(np.array([1.0, 1.00005, 0.99995]), ref, s, 1e-4, "inside")
    with pytest.raises(AssertionError):
        assert_within(np.array([1.0, 1.0002, 1.0]), ref, s, 1e-4, "outside")


def test_assert_within_zero_scale_needs_exact_zero():
    ref = np.zeros(2)
    s = np.zeros(2)
    assert_within(np.array([0.0, -0.0]), ref, s, 1e-4, "zeros")
    with pytest.raises(AssertionError):
        assert_within(np.array([0.0, 1e-30]), ref, s, 1e-4, "tiny")


@pytest.mark.parametrize("fmt", ["q4_0", "q4_1", "q8_0", "q5_0", "q5_1"])
def test_oracle_rows_equals_oracle_dot(fmt):
    m, k, n = 173, 256, 3
    w = synth.quant_matrix(fmt, m, k, seed=31, tensor_id=1, d_range=(1e-3, 2e-2))
    x = np.ascontiguousarray(synth.activations(k, n, seed=31, tensor_id=2))
    y, s = oracle.dot(fmt, w, m, k, x, n)
    y2, s2 = oracle_rows(oracle.dot, fmt, w, m, k, x, n)
    assert np.array_equal(y, y2) and np.array_equal(s, s2)
    q, qs = oracle.dot_x8(fmt, w, m, k, x, n)
    q2, qs2 = oracle_rows(oracle.dot_x8, fmt, w, m, k, x, n)
    assert np.array_equal(q, q2) and np.array_equal(qs, qs2)


@pytest.mark.parametrize("fmt", ["q4_0", "q4_1", "q8_0", "q5_0", "q5_1"])
def test_gemm_reference_matches_oracle_dot_f16(fmt):
    m, k, n = 41, 320, 5
    w = synth.quant_matrix(fmt, m, k, seed=33, tensor_id=1, d_range=(1e-3, 2e-2))
    xh = synth.activations(k, n, seed=33, tensor_id=2, dtype=np.float16)
    y, s = oracle.dot(fmt, w, m, k, xh.view(np.uint16), n, x_is_f16=True)
    y2, s2 = gemm_reference(oracle, fmt, w, m, k, xh)
    np.testing.assert_allclose(y2, y, rtol=0, atol=1e-12 * s.max())
    np.testing.assert_allclose(s2, s, rtol=1e-13)
