"""Pins for the oracle's SRFT (no GPU).

The SRFT is pack(F diag(s) x) with F the unitary DFT ("When Quantization Is Free",
technical summary, Methodology 1).  Each check below ties the oracle to something other
than its own formula: a library FFT, textbook DFT pairs, orthogonality and its inverse.
"""
import numpy as np
import pytest

from oracle import kvq_oracle as O

DIMS = [8, 16, 128, 256]


def _matrix(d):
    """Columns = SRFT of the basis vectors with s = 1."""
    return O.srft(np.eye(d), np.ones(d)).T


@pytest.mark.parametrize("d", DIMS)
def test_orthogonal(d):
    Q = _matrix(d)
    assert np.abs(Q @ Q.T - np.eye(d)).max() < 1e-13
    assert np.abs(Q.T @ Q - np.eye(d)).max() < 1e-13


@pytest.mark.parametrize("d", DIMS)
def test_dft_matches_library_fft(d):
    rng = np.random.default_rng(d)
    z = rng.standard_normal(d) + 1j * rng.standard_normal(d)
    assert np.abs(O.unitary_dft(z) - np.fft.fft(z, norm="ortho")).max() < 1e-12
    assert np.abs(O.inverse_unitary_dft(z) - np.fft.ifft(z, norm="ortho")).max() < 1e-12


@pytest.mark.parametrize("d", DIMS)
def test_layout_against_rfft(d):
    """Slots 0/1 hold bins 0 and d/2; slots 2k/2k+1 hold sqrt2 * (Re, Im) of bin k."""
    rng = np.random.default_rng(100 + d)
    x = rng.standard_normal(d)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    y = O.srft(x, s)
    R = np.fft.rfft(s * x, norm="ortho")
    m = d // 2
    assert abs(y[0] - R[0].real) < 1e-12
    assert abs(y[1] - R[m].real) < 1e-12
    for k in range(1, m):
        assert abs(y[2 * k] - np.sqrt(2) * R[k].real) < 1e-12
        assert abs(y[2 * k + 1] - np.sqrt(2) * R[k].imag) < 1e-12


@pytest.mark.parametrize("d", DIMS)
def test_textbook_pairs(d):
    n = np.arange(d)
    one = np.ones(d)
    m = d // 2
    # delta at 0 -> flat spectrum
    delta = np.zeros(d)
    delta[0] = 1.0
    expect = np.full(d, np.sqrt(2.0) / np.sqrt(d))
    expect[0] = expect[1] = 1.0 / np.sqrt(d)
    expect[3::2] = 0.0
    assert np.abs(O.srft(delta, one) - expect).max() < 1e-13
    # constant -> DC only
    e = np.zeros(d)
    e[0] = np.sqrt(d)
    assert np.abs(O.srft(one, one) - e).max() < 1e-12
    # alternating -> Nyquist only
    e = np.zeros(d)
    e[1] = np.sqrt(d)
    assert np.abs(O.srft((-1.0) ** n, one) - e).max() < 1e-12
    # cosine / sine at bin k0 -> one slot each, with the e^{-i...} sign convention
    for k0 in (1, 3, m - 1):
        e = np.zeros(d)
        e[2 * k0] = np.sqrt(d / 2)
        assert np.abs(O.srft(np.cos(2 * np.pi * k0 * n / d), one) - e).max() < 1e-12
        e = np.zeros(d)
        e[2 * k0 + 1] = -np.sqrt(d / 2)
        assert np.abs(O.srft(np.sin(2 * np.pi * k0 * n / d), one) - e).max() < 1e-12


@pytest.mark.parametrize("d", DIMS)
def test_parseval_inverse_and_inner_product(d):
    rng = np.random.default_rng(7 * d)
    x = rng.standard_normal((5, d))
    q = rng.standard_normal((5, d))
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    y = O.srft(x, s)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=0, atol=1e-12)
    assert np.abs(O.inverse_srft(y, s) - x).max() < 1e-12
    assert np.abs((O.srft(q, s) * y).sum(-1) - (q * x).sum(-1)).max() < 1e-11
    # inverse against the library's inverse real FFT
    m = d // 2
    R = np.zeros((5, m + 1), dtype=complex)
    R[:, 0] = y[:, 0]
    R[:, m] = y[:, 1]
    R[:, 1:m] = (y[:, 2:d:2] + 1j * y[:, 3:d:2]) / np.sqrt(2)
    assert np.abs(s * np.fft.irfft(R, n=d, norm="ortho") - O.inverse_srft(y, s)).max() < 1e-12


def test_sign_is_applied_before_the_dft():
    d = 128
    rng = np.random.default_rng(3)
    x = rng.standard_normal(d)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    assert np.abs(O.srft(x, s) - O.srft(s * x, np.ones(d))).max() < 1e-13
    # a sign vector must matter (catches a dropped s)
    assert np.abs(O.srft(x, s) - O.srft(x, np.ones(d))).max() > 1e-3


def test_calibrate_lambda_is_rotated_absmax():
    d, n = 128, 40
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, n, d)).astype(np.float16)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    lam = O.calibrate_lambda(x, s, 16)
    assert lam.shape == (2, d)
    # against the library FFT of each calibration token
    R = np.fft.rfft(s * x[:, :16].astype(np.float64), norm="ortho")
    m = d // 2
    ref = np.empty((2, 16, d))
    ref[..., 0] = R[..., 0].real
    ref[..., 1] = R[..., m].real
    ref[..., 2::2] = np.sqrt(2) * R[..., 1:m].real
    ref[..., 3::2] = np.sqrt(2) * R[..., 1:m].imag
    assert np.abs(lam - np.abs(ref).max(axis=1)).max() < 1e-12
    # tokens after n_cal do not count; an all-zero channel gets lambda = 1
    z = np.zeros((1, 4, d), dtype=np.float16)
    assert np.all(O.calibrate_lambda(z, s, 4) == 1.0)
