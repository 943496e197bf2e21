"""Pins of the oracle's SRHT rotation (the pages' alternative to SRFT, [QF] Methodology 1 and
Key results "SRFT vs SRHT"), reading R13: SRHT(x) = d^-1/2 H diag(s) x with the
Sylvester-ordered Walsh-Hadamard matrix."""
import numpy as np
import pytest
import scipy.linalg

from oracle import kvq_oracle as O


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_matches_scipy(d):
    # library routine: scipy builds the same Sylvester-ordered matrix by recursion
    assert np.array_equal(O.hadamard_matrix(d), scipy.linalg.hadamard(d).astype(np.float64))


@pytest.mark.parametrize("d", [128, 256])
def test_srht_orthogonal_and_exact_inverse(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((7, d))
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    y = O.srht(x, s)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    np.testing.assert_allclose(O.inverse_srht(y, s), x, atol=1e-12)
    # dot products survive the rotation (what the decode in the rotated domain relies on)
    np.testing.assert_allclose(O.srht(x[:3], s) @ O.srht(x[3:6], s).T, x[:3] @ x[3:6].T, atol=1e-11)


@pytest.mark.parametrize("d", [128, 256])
def test_srht_closed_forms(d):
    ones = np.ones(d)
    # H 1 = d e_0, so the all-ones vector maps to sqrt(d) e_0
    e0 = np.zeros(d)
    e0[0] = np.sqrt(d)
    np.testing.assert_allclose(O.srht(ones, ones), e0, atol=1e-12)
    # a delta at position j maps to column j of H / sqrt(d): signs (-1)^popcount(i & j)
    j = 37
    x = np.zeros(d)
    x[j] = 1.0
    expect = np.array([(-1.0) ** bin(i & j).count("1") for i in range(d)]) / np.sqrt(d)
    np.testing.assert_allclose(O.srht(x, ones), expect, atol=1e-15)
    # the sign vector acts before H: s = -1 everywhere negates the output
    np.testing.assert_allclose(O.srht(x, -ones), -expect, atol=1e-15)


def test_transform_dispatch_and_write_path():
    rng = np.random.default_rng(5)
    d = 128
    x16 = rng.standard_normal((3, 40, d)).astype(np.float16)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    np.testing.assert_array_equal(O.rotate(x16, s, "srht"), O.srht(x16, s))
    np.testing.assert_array_equal(O.rotate(x16, s, "srft"), O.srft(x16, s))
    with pytest.raises(ValueError):
        O.rotate(x16, s, "dct")
    lam = O.calibrate_lambda(x16, s, 16, transform="srht")[:, None, :]
    codes, scales = O.quantize(x16, s, lam, 4, transform="srht")
    assert np.abs(codes).max() <= 7
    # dequantize inverts the rotation of the same transform: the error is the quantizer's
    xh = O.dequantize(codes, scales, s, lam, transform="srht")
    err = np.abs(O.srht(xh, s) - O.srht(x16.astype(np.float64), s))
    step = np.repeat(scales.astype(np.float64), 16, axis=-1) * lam
    assert (err <= 0.5 * step + 1e-9).all()
