"""Pins for the oracle's quantizer, packing and dequantizer (no GPU).

Write path: per-channel lambda rescale, per-group absmax, rounding to signed int4/int8,
two int4 per byte ("When Quantization Is Free", technical summary, Methodology 2 and 3).
"""
import numpy as np
import pytest

from oracle import kvq_oracle as O

G = O.GROUP


def _data(seed, n, d, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    if outliers:
        x[:, rng.choice(d, 3, replace=False)] *= 20.0
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    lam = np.exp(rng.uniform(-1, 1, d))
    return x.astype(np.float16), s, lam


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("d", [128, 256])
def test_code_range_and_full_scale(bits, d):
    x, s, lam = _data(bits * d, 200, d)
    codes, scales = O.quantize(x, s, lam, bits)
    qmax = O.QMAX[bits]
    assert codes.dtype == np.int8 and scales.dtype == np.float16
    assert codes.shape == x.shape and scales.shape == (200, d // G)
    assert codes.min() >= -qmax and codes.max() <= qmax
    g = np.abs(codes.reshape(200, d // G, G)).max(-1)
    # every group with a (normal) nonzero scale reaches +-qmax: a/scale is qmax*(1 +- 2^-11)
    assert np.all(g[scales > 0] == qmax)


@pytest.mark.parametrize("bits", [4, 8])
def test_rounding_error_bound(bits):
    d = 128
    x, s, lam = _data(5 + bits, 300, d)
    u = O.rotated_scaled(x, s, lam)
    codes, scales = O.quantize(x, s, lam, bits)
    sc = np.repeat(scales.astype(np.float64), G, axis=-1)
    err = np.abs(u - codes * sc)
    # half a step, plus the float32 rounding of u taken before the decision
    assert np.all(err <= sc / 2 * (1 + 1e-5) + np.abs(u) * 2 ** -23)


def test_odd_symmetry_and_power_of_two_equivariance():
    d = 128
    x, s, lam = _data(21, 300, d)
    c, sc = O.quantize(x, s, lam, 4)
    c2, sc2 = O.quantize(-x, s, lam, 4)
    assert np.array_equal(c2, -c) and np.array_equal(sc2, sc)
    c3, sc3 = O.quantize((x.astype(np.float32) / 4).astype(np.float16), s, lam, 4)
    assert np.array_equal(c3, c)
    assert np.array_equal(sc3.astype(np.float32) * 4, sc.astype(np.float32))
    c4, sc4 = O.quantize(x, s, lam * 2.0, 8)
    c5, sc5 = O.quantize(x, s, lam, 8)
    assert np.array_equal(c4, c5) and np.array_equal(sc4.astype(np.float32) * 2, sc5.astype(np.float32))


def test_zero_vector_and_zero_group():
    d = 128
    s = np.ones(d)
    c, sc = O.quantize(np.zeros((2, d), np.float16), s, np.ones(d), 4)
    assert not c.any() and not sc.astype(np.float32).any()
    # a vector whose rotation is exactly one DFT bin leaves the other groups at scale 0
    n = np.arange(d)
    x = (np.cos(2 * np.pi * 5 * n / d)).astype(np.float16)
    c, sc = O.quantize(x, s, np.ones(d), 4)
    assert (sc.astype(np.float32) > 0).sum() >= 1
    assert np.all(c.reshape(-1, G)[sc.reshape(-1).astype(np.float32) == 0] == 0)


def test_scale_saturates_at_fp16_max():
    d = 128
    s = np.ones(d)
    x = np.full((1, d), 60000.0, dtype=np.float16)   # DC = 60000 * sqrt(128) / lambda
    c, sc = O.quantize(x, s, np.full(d, 1e-2), 4)
    assert sc.astype(np.float32)[0, 0] == 65504.0
    assert c[0, 0] == 7


def test_subnormal_scale_clamps_codes():
    d = 128
    s = np.ones(d)
    tiny = np.zeros((1, d), np.float16)
    tiny[0, 0] = np.float16(6e-8)                     # smallest fp16 subnormal
    c, sc = O.quantize(tiny, s, np.ones(d), 4)
    assert np.abs(c).max() <= 7
    assert np.all((sc.astype(np.float32) == 0) | (np.abs(c.reshape(-1, G)).max(-1) > 0))


def test_constructed_example_is_recovered_exactly():
    """Choose codes and scales, build x from them, and quantize it back.

    Integers sit 0.5 away from every rounding tie and the fp16 rounding of x moves u by far
    less, so the codes must come back exactly.
    """
    d = 128
    rng = np.random.default_rng(1234)
    n = 64
    for bits in (4, 8):
        qmax = O.QMAX[bits]
        codes = rng.integers(-qmax, qmax + 1, size=(n, d)).astype(np.int8)
        codes.reshape(n, d // G, G)[:, :, 0] = qmax * np.where(rng.random((n, d // G)) < 0.5, -1, 1)
        scales = (rng.uniform(0.5, 2.0, size=(n, d // G))).astype(np.float16)
        s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
        lam = np.exp(rng.uniform(-0.5, 0.5, d))
        y = lam * codes * np.repeat(scales.astype(np.float64), G, axis=-1)
        x = O.inverse_srft(y, s)
        x16 = x.astype(np.float16)
        # the fp16 rounding of x moves every rotated channel by well under half a code step
        step = lam * np.repeat(scales.astype(np.float64), G, axis=-1)
        moved = np.abs(O.srft(x16.astype(np.float64) - x, s)) / step
        assert moved.max() < 0.4
        c2, _ = O.quantize(x16, s, lam, bits)
        assert np.array_equal(c2, codes)
        # without the fp16 input rounding, codes and scales come back bit-exact
        c3, sc3 = O.quantize_decision(O.srft(x, s) / lam, bits)
        assert np.array_equal(c3, codes)
        assert np.array_equal(sc3.view(np.int16), scales.view(np.int16))


def test_pack_bytes_by_hand():
    codes = np.array([[1, -1, -7, 7, 0, -8 + 1, 3, -2]], dtype=np.int8)
    # two's-complement nibbles, low nibble = even channel
    expect = np.array([[0xF1, 0x79, 0x90, 0xE3]], dtype=np.uint8)
    assert np.array_equal(O.pack_codes(codes, 4), expect)
    assert np.array_equal(O.unpack_codes(expect, 4), codes)
    c8 = np.array([[-1, 127, -127, 0]], dtype=np.int8)
    assert np.array_equal(O.pack_codes(c8, 8), np.array([[0xFF, 0x7F, 0x81, 0x00]], np.uint8))
    assert np.array_equal(O.unpack_codes(O.pack_codes(c8, 8), 8), c8)
    rng = np.random.default_rng(0)
    c = rng.integers(-7, 8, size=(10, 128)).astype(np.int8)
    assert np.array_equal(O.unpack_codes(O.pack_codes(c, 4), 4), c)


@pytest.mark.parametrize("bits", [4, 8])
def test_dequantize_error_bound(bits):
    """x_hat - x is the inverse rotation of the rounding error, so its norm is bounded by it."""
    d = 128
    x, s, lam = _data(77 + bits, 100, d)
    c, sc = O.quantize(x, s, lam, bits)
    xh = O.dequantize(c, sc, s, lam)
    step = lam * np.repeat(sc.astype(np.float64), G, axis=-1)
    bound = np.linalg.norm(step / 2, axis=-1) * (1 + 1e-4)
    err = np.linalg.norm(xh - x.astype(np.float64), axis=-1)
    assert np.all(err <= bound)


def test_method_beats_plain_per_token_scaling_on_outlier_keys():
    """Directional claim of Methodology 3: on d=128 keys with outlier coordinates a single
    per-token absmax scale fails; the rotated, lambda-scaled, group-of-16 quantizer does
    far better (reconstruction-error comparison on synthetic Student-t keys)."""
    d = 128
    rng = np.random.default_rng(5)
    x = rng.standard_t(3, size=(512, d))
    x[:, rng.choice(d, 4, replace=False)] *= 20
    x16 = x.astype(np.float16)
    x64 = x16.astype(np.float64)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    lam = O.calibrate_lambda(x16, s, 256)
    c, sc = O.quantize(x16, s, lam, 4)
    err_ours = np.linalg.norm(O.dequantize(c, sc, s, lam) - x64)
    # baseline: one absmax scale per token, no rotation, no lambda
    a = np.abs(x64).max(-1, keepdims=True) / 7
    err_tok = np.linalg.norm(np.clip(np.rint(x64 / a), -7, 7) * a - x64)
    assert err_ours < 0.6 * err_tok


def test_exact_ties_round_half_to_even():
    """The pages fix no rounding mode; the reading is round-half-to-even (gfx950 v_rndne_f32).
    With scale exactly 1, u/scale hits exact .5 ties."""
    u = np.array([[7.0, 2.5, -2.5, 3.5, -3.5, 0.5, -0.5, 1.5, -1.5, 4.5, -4.5, 5.5, -5.5, 6.5, -6.5, 0.0]])
    codes, scales = O.quantize_decision(u, 4)
    assert scales[0, 0] == np.float16(1.0)
    assert codes[0].tolist() == [7, 2, -2, 4, -4, 0, 0, 2, -2, 4, -4, 6, -6, 6, -6, 0]


# ---- one scale per vector (group = d): the per-token comparison mode ----

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("d", [128, 256])
def test_per_token_equals_grouped_when_every_group_has_the_same_absmax(bits, d):
    """If every group of 16 holds the same absmax, the vector's one scale equals every group's
    scale, so the codes of the two modes are identical (catches a wrong axis or reshape)."""
    rng = np.random.default_rng(11 + d + bits)
    u = rng.uniform(-1, 1, size=(40, d))
    amax = rng.uniform(0.5, 3.0, size=(40, 1))
    u = u / np.abs(u).max(-1, keepdims=True) * 0.999 * amax
    g = u.reshape(40, d // G, G)
    idx = rng.integers(0, G, size=(40, d // G))
    sign = np.where(rng.random((40, d // G)) < 0.5, -1.0, 1.0)
    np.put_along_axis(g, idx[..., None], (sign * amax)[..., None], axis=-1)
    u = g.reshape(40, d)
    c_tok, s_tok = O.quantize_decision(u, bits, group=d)
    c_grp, s_grp = O.quantize_decision(u, bits)
    assert s_tok.shape == (40, 1) and s_grp.shape == (40, d // G)
    assert np.array_equal(np.repeat(s_tok, d // G, axis=-1), s_grp)
    assert np.array_equal(c_tok, c_grp)


@pytest.mark.parametrize("bits", [4, 8])
def test_per_token_scale_is_the_vector_absmax(bits):
    """group = d: scale = fp16(max|u| / qmax); the largest element maps to +-qmax; every code is
    within half a step of u / scale; dequantize inverts up to that error."""
    d = 128
    x, s, lam = _data(21, 64, d)
    qmax = O.QMAX[bits]
    u = O.rotated_scaled(x, s, lam)
    c, sc = O.quantize_decision(u, bits, group=d)
    u32 = u.astype(np.float32)
    want = (np.abs(u32).max(-1) / np.float32(qmax)).astype(np.float16)
    assert np.array_equal(sc[:, 0], want)
    top = np.abs(u32).argmax(-1)
    assert np.all(np.abs(c[np.arange(64), top]) == qmax)
    step = sc.astype(np.float64)
    assert np.all(np.abs(u - c * step) <= 0.5 * step * (1 + 1e-6) + 1e-12)
    xh = O.dequantize(c, sc, s, lam, group=d)
    bound = np.linalg.norm(lam * 0.5 * step, axis=-1) * (1 + 1e-9)
    assert np.all(np.linalg.norm(xh - x.astype(np.float64), axis=-1) <= bound + 1e-9)


def test_grouped_scales_beat_one_scale_per_vector_after_rotation():
    """With the rotation and lambda in place, 16-channel groups still lower the reconstruction
    error against one scale per vector on outlier keys (Methodology 3's per-group claim), and
    one scale per vector without rotation is the worst of the three."""
    d = 128
    rng = np.random.default_rng(9)
    x = rng.standard_t(3, size=(512, d))
    x[:, rng.choice(d, 4, replace=False)] *= 20
    x16 = x.astype(np.float16)
    x64 = x16.astype(np.float64)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    lam = O.calibrate_lambda(x16, s, 256)
    err = {}
    for name, grp in (("group16", G), ("per_token", d)):
        c, sc = O.quantize(x16, s, lam, 4, group=grp)
        err[name] = np.linalg.norm(O.dequantize(c, sc, s, lam, group=grp) - x64)
    a = np.abs(x64).max(-1, keepdims=True) / 7
    err["per_token_unrotated"] = np.linalg.norm(np.clip(np.rint(x64 / a), -7, 7) * a - x64)
    assert err["group16"] < err["per_token"] < err["per_token_unrotated"]
