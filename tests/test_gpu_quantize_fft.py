"""GPU parity of kvq_quantize_fft, the write path with the rotation as an in-register FFT (one
lane per vector), against the oracle under the write path's bar (packing bit-exact, codes within
the rounding-tie rule, scales bit-equal or one fp16 ulp apart), on both transforms, both widths,
both head dims, per-group and per-vector scales, with and without lambda, shared and per-row
signs, ragged token counts across its 256-token tiles and written at an offset.  Its planes are
also compared with kvq_quantize's: the two forms agree byte for byte except on near-ties."""
import numpy as np
import pytest

from kv_cache_quantization_srft_amd import kvq, synth
from oracle import kvq_oracle as O

from gpu_parity import CODE_MISMATCH_RATE, check_quantize, gpu_quantize, say

pytestmark = pytest.mark.gpu


def _data(rng, B, H, n, d):
    std = np.exp(rng.uniform(np.log(0.5), np.log(4.0), size=(B, H, 1, d)))
    out = np.where(rng.random((B, H, 1, d)) < 0.03, 20.0, 1.0)
    return synth.to_fp16(rng.standard_t(4, size=(B, H, n, d)) * std * out)


# d, bits, transform, B, H, n, lambda, per-row signs, group, pos, extra capacity
CASES = [
    (128, 4, "srft", 2, 3, 700, True, False, 16, 0, 0),
    (128, 8, "srft", 3, 2, 257, False, True, 16, 9, 31),
    (128, 4, "srft", 1, 5, 255, True, True, 128, 3, 0),
    (128, 4, "srht", 2, 2, 513, True, False, 16, 0, 7),
    (128, 8, "srht", 1, 3, 300, False, False, 128, 0, 0),
    (256, 4, "srft", 2, 2, 511, True, True, 16, 1, 0),
    (256, 8, "srft", 1, 3, 260, True, False, 256, 0, 12),
    (256, 4, "srht", 2, 1, 333, False, True, 16, 40, 0),
    (256, 8, "srht", 1, 2, 129, True, False, 16, 0, 0),
    (128, 4, "srft", 1, 1, 1, True, False, 16, 5, 2),
]


@pytest.mark.parametrize("d,bits,transform,B,H,n,lam,per_row_sign,group,pos,extra", CASES)
def test_quantize_fft_parity(d, bits, transform, B, H, n, lam, per_row_sign, group, pos, extra):
    rng = np.random.default_rng(d * 7 + bits + B * H * n + group + pos)
    cap = pos + n + extra
    x = _data(rng, B, H, n, d)
    s = np.stack([synth.random_signs(300 + b, d) for b in range(B)]) if per_row_sign else synth.random_signs(8, d)
    lam_v = synth.random_lambda(rng, (B, H, d), 0.5, 8.0) if lam else None
    kw = dict(capacity=cap, pos=pos, sign_bs=d if per_row_sign else 0, lambda_bs=H * d if lam else 0,
              transform=transform, group=group)
    cb, sc, _ = gpu_quantize(x, s, lam_v, bits, entry=kvq.kvq_quantize_fft, **kw)
    lam_b = 1.0 if lam_v is None else lam_v[:, :, None, :].astype(np.float64)
    srow = s[:, None, None, :] if per_row_sign else s
    u = O.rotated_scaled(x, srow, lam_b, transform)
    label = f"fft d{d} b{bits} {transform} g{group}"
    n_diff, n_ulp = check_quantize(cb[:, :, pos:pos + n], sc[:, :, pos:pos + n], u, bits, label, group=group)
    say("quantize_fft: tie flips", n_diff, "scale ulps", n_ulp, label)
    keep = np.ones(cap, bool)
    keep[pos:pos + n] = False
    assert np.all(cb[:, :, keep] == 0xAB)
    assert np.all(np.isnan(sc[:, :, keep].astype(np.float32)))
    # the MFMA form of the same write path: identical bytes up to near-tie flips
    cm, sm, _ = gpu_quantize(x, s, lam_v, bits, **kw)
    n_sc = int((sm.view(np.int16) != sc.view(np.int16)).sum())
    gm, gf = O.unpack_codes(cm, bits), O.unpack_codes(cb, bits)
    n_code = int((gm != gf).sum())
    assert n_sc <= max(1, CODE_MISMATCH_RATE * sc.size) and n_code <= max(2, 2 * CODE_MISMATCH_RATE * gf.size), \
        (n_sc, n_code)
    if n_code:
        assert np.abs(gm.astype(int) - gf.astype(int)).max() == 1


def test_quantize_fft_edge_values():
    """Zero vectors (zero scales and codes), fp16-maximum inputs (saturated scales), subnormal and
    tiny inputs, and a tiny lambda."""
    d = 128
    s = synth.random_signs(11, d)
    rng = np.random.default_rng(11)
    x = np.zeros((1, 1, 6, d), np.float16)
    x[0, 0, 1] = 65504.0
    x[0, 0, 2, 3] = np.float16(6e-8)
    x[0, 0, 3] = synth.to_fp16(rng.standard_normal(d) * 1e-4)
    x[0, 0, 4] = -65504.0
    x[0, 0, 5, ::2] = 1.0
    for bits in (4, 8):
        for lam in (None, np.full(d, 1e-3, np.float32)):
            cb, sc, _ = gpu_quantize(x, s, lam, bits, entry=kvq.kvq_quantize_fft)
            u = O.rotated_scaled(x, s, 1.0 if lam is None else lam.astype(np.float64))
            check_quantize(cb, sc, u, bits, f"fft edge b{bits} lam={lam is not None}")
            assert np.all(cb[0, 0, 0] == 0) and np.all(sc[0, 0, 0].astype(np.float32) == 0)


def test_quantize_fft_constructed_example_bit_exact():
    """Inputs built from chosen codes and scales: the FFT form must return those exact bytes."""
    d = 256
    rng = np.random.default_rng(4321)
    n = 300
    for bits in (4, 8):
        qmax = O.QMAX[bits]
        codes = rng.integers(-qmax, qmax + 1, size=(n, d)).astype(np.int8)
        codes.reshape(n, d // 16, 16)[:, :, 0] = qmax * np.where(rng.random((n, d // 16)) < 0.5, -1, 1)
        scales = rng.uniform(0.5, 2.0, size=(n, d // 16)).astype(np.float16)
        s = synth.random_signs(78, d)
        lam = np.exp(rng.uniform(-0.5, 0.5, d)).astype(np.float32)
        y = lam.astype(np.float64) * codes * np.repeat(scales.astype(np.float64), 16, axis=-1)
        x16 = O.inverse_srft(y, s).astype(np.float16)[None, None]
        cb, sc, _ = gpu_quantize(x16, s, lam, bits, entry=kvq.kvq_quantize_fft)
        assert np.array_equal(cb[0, 0], O.pack_codes(codes, bits))
