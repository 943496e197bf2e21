"""GPU parity of the write path (kvq_quantize), dequantize and lambda calibration against the
CPU oracle, through the C ABI.  Inputs are seeded synthetic K/V with each workload's shapes and
value statistics."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_srft_amd import kvq, synth
from oracle import kvq_oracle as O

from gpu_parity import check_quantize, dev, gpu_quantize, planes, say, DEQUANT_RTOL

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def _lam_oracle(x16, s, n_cal):
    """Oracle-calibrated lambda, rounded to float32 as it is passed to the kernel."""
    return O.calibrate_lambda(x16, s, n_cal).astype(np.float32)


def _run(x16, s, lam, bits, label, **kw):
    say("quantize", label, x16.shape, bits)
    cb, sc, lay = gpu_quantize(x16, s, lam, bits, **kw)
    pos = kw.get("pos", 0)
    n = x16.shape[2]
    lam_b = np.ones(x16.shape[-1]) if lam is None else np.asarray(lam, np.float64)
    if lam_b.ndim == 2:
        lam_b = lam_b[None, :, None, :]
    elif lam_b.ndim == 3:
        lam_b = lam_b[:, :, None, :]
    u = O.rotated_scaled(x16, s if np.ndim(s) == 1 else s[:, None, None, :], lam_b)
    return check_quantize(cb[:, :, pos:pos + n], sc[:, :, pos:pos + n], u, bits, label), cb, sc


def test_tiny_workload():
    w = W[1]
    s = synth.signs(w)
    for t in (synth.K_TENSOR, synth.V_TENSOR):
        x = synth.kv(w, 0, t)
        _run(x, s, None, 4, f"tiny t{t}")


def test_qwen_like_layer_with_calibrated_lambda():
    w = W[2]
    s = synth.signs(w)
    for layer in (0, 27):
        for t in (synth.K_TENSOR, synth.V_TENSOR):
            x = synth.kv(w, layer, t)
            lam = _lam_oracle(x, s, w.n_cal)[0]
            _run(x, s, lam, 4, f"qwen L{layer} t{t}")


def test_gemma_like_k8v4_d256():
    w = W[3]
    s = synth.signs(w)
    x = synth.kv(w, 3, synth.K_TENSOR, seq_len=700)
    _run(x, s, None, 8, "gemma K int8")
    x = synth.kv(w, 3, synth.V_TENSOR, seq_len=700)
    _run(x, s, None, 4, "gemma V int4")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("d", [128, 256])
def test_loguniform_std_and_student_t(bits, d):
    rng = np.random.default_rng(d + bits)
    std = np.exp(rng.uniform(np.log(0.5), np.log(8.0), size=(1, 3, 1, d)))
    x = synth.to_fp16(std * rng.standard_normal((1, 3, 513, d)))
    s = synth.random_signs(5, d)
    lam = _lam_oracle(x, s, 512)[0]
    _run(x, s, lam, bits, f"loguniform d{d} b{bits}")
    x = synth.to_fp16(rng.standard_t(4, size=(2, 2, 300, d)) * np.where(rng.random((2, 2, 1, d)) < 0.03, 20, 1))
    _run(x, s, None, bits, f"t4 d{d} b{bits}")


def test_append_ragged_positions_and_untouched_slots():
    rng = np.random.default_rng(3)
    d = 128
    s = synth.random_signs(3, d)
    lam = np.exp(rng.uniform(-1, 1, (2, d))).astype(np.float32)
    for pos, n in ((0, 1), (17, 1), (100, 37), (5, 300)):
        x = synth.to_fp16(rng.standard_normal((3, 2, n, d)))
        (_, _), cb, sc = _run(x, s, lam, 4, f"append pos{pos} n{n}", capacity=pos + n + 9, pos=pos)
        # bytes outside [pos, pos+n) keep their fill value
        assert np.all(cb[:, :, :pos] == 0xAB) and np.all(cb[:, :, pos + n:] == 0xAB)
        assert np.all(np.isnan(sc[:, :, :pos].astype(np.float32)))
        assert np.all(np.isnan(sc[:, :, pos + n:].astype(np.float32)))


def test_per_row_sign_and_lambda_strides():
    rng = np.random.default_rng(8)
    B, H, n, d = 3, 2, 70, 256
    x = synth.to_fp16(rng.standard_normal((B, H, n, d)) * 3)
    s = np.stack([synth.random_signs(i, d) for i in range(B)])
    lam = np.exp(rng.uniform(-1, 1, (B, H, d))).astype(np.float32)
    say("quantize strides")
    cb, sc, _ = gpu_quantize(x, s.reshape(-1), lam, 4, sign_bs=d, lambda_bs=H * d)
    u = O.rotated_scaled(x, s[:, None, None, :], lam[:, :, None, :].astype(np.float64))
    check_quantize(cb, sc, u, 4, "strides")


def test_edge_values():
    d = 128
    s = synth.random_signs(11, d)
    rng = np.random.default_rng(11)
    x = np.zeros((1, 1, 6, d), np.float16)
    x[0, 0, 1] = 65504.0                                  # saturating scale
    x[0, 0, 2, 3] = np.float16(6e-8)                     # subnormal input -> subnormal/zero scales
    x[0, 0, 3] = synth.to_fp16(rng.standard_normal(d) * 1e-4)
    x[0, 0, 4] = -65504.0
    x[0, 0, 5, ::2] = 1.0
    for bits in (4, 8):
        (_, _), cb, sc = _run(x, s, None, bits, f"edge b{bits}")
        assert np.all(cb[0, 0, 0] == 0) and np.all(sc[0, 0, 0].astype(np.float32) == 0)
    lam = np.full(d, 1e-3, np.float32)
    _run(x, s, lam, 4, "edge tiny lambda")


def test_constructed_example_bit_exact():
    """Inputs built from chosen codes and scales: the GPU must return those exact bytes."""
    d = 128
    rng = np.random.default_rng(1234)
    n = 256
    for bits in (4, 8):
        qmax = O.QMAX[bits]
        codes = rng.integers(-qmax, qmax + 1, size=(n, d)).astype(np.int8)
        codes.reshape(n, d // 16, 16)[:, :, 0] = qmax * np.where(rng.random((n, d // 16)) < 0.5, -1, 1)
        scales = rng.uniform(0.5, 2.0, size=(n, d // 16)).astype(np.float16)
        s = synth.random_signs(77, d)
        lam = np.exp(rng.uniform(-0.5, 0.5, d)).astype(np.float32)
        y = lam.astype(np.float64) * codes * np.repeat(scales.astype(np.float64), 16, axis=-1)
        x16 = O.inverse_srft(y, s).astype(np.float16)[None, None]
        say("constructed", bits)
        cb, sc, _ = gpu_quantize(x16, s, lam, bits)
        assert np.array_equal(cb[0, 0], O.pack_codes(codes, bits))


def test_deterministic():
    w = W[2]
    s = synth.signs(w)
    x = synth.kv(w, 5, synth.K_TENSOR)
    lam = _lam_oracle(x, s, 512)[0]
    a = gpu_quantize(x, s, lam, 4)
    b = gpu_quantize(x, s, lam, 4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.int16), b[1].view(np.int16))


@pytest.mark.parametrize("d,bits", [(128, 4), (128, 8), (256, 4), (256, 8)])
def test_dequantize_on_oracle_planes(d, bits):
    rng = np.random.default_rng(d * bits)
    B, H, n = 2, 3, 333
    x = synth.to_fp16(rng.standard_t(4, size=(B, H, n, d)))
    s = synth.random_signs(d, d)
    lam = np.exp(rng.uniform(-1, 1, (H, d))).astype(np.float32)
    oc, osc = O.quantize(x, s, lam[None, :, None, :], bits)
    lay = kvq.make_layout(B, H, H, d, n + 4)
    cpl = np.zeros((B, H, n + 4, d * bits // 8), np.uint8)
    spl = np.zeros((B, H, n + 4, d // 16), np.float16)
    cpl[:, :, 4:] = O.pack_codes(oc, bits)
    spl[:, :, 4:] = osc
    out = torch.full((B * H * n * d,), float("nan"), dtype=torch.float32, device="cuda")
    say("dequantize", d, bits)
    kvq.kvq_dequantize(lay, bits, dev(cpl), dev(spl.view(np.int16)), 4, n, dev(s), 0, dev(lam), 0, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(B, H, n, d).astype(np.float64)
    ref = O.dequantize(oc, osc, s, lam[None, :, None, :])
    err = np.abs(got - ref).max(-1)
    scale = np.abs(ref).max(-1)
    assert np.all(err <= DEQUANT_RTOL * scale + 1e-30), err.max()


@pytest.mark.parametrize("d", [128, 256])
def test_calibrate_lambda(d):
    rng = np.random.default_rng(d)
    B, H, n = 2, 2, 700
    x = synth.to_fp16(rng.standard_t(3, size=(B, H, n, d)) * np.where(rng.random((B, H, 1, d)) < 0.03, 20, 1))
    x[1, 1, :, :] = 0                                      # an all-zero row -> lambda = 1
    s = synth.random_signs(d + 1, d)
    lay = kvq.make_layout(B, H, H, d, n)
    lam = torch.full((B * H * d,), float("nan"), dtype=torch.float32, device="cuda")
    say("calibrate", d)
    kvq.kvq_calibrate_lambda(lay, dev(x), n, 512, dev(s), 0, lam)
    torch.cuda.synchronize()
    got = lam.cpu().numpy().reshape(B, H, d)
    ref = O.calibrate_lambda(x, s, 512)
    norm = np.linalg.norm(x[:, :, :512].astype(np.float64), axis=-1).max(-1)[..., None]
    assert np.all(np.abs(got - ref) <= 1e-5 * ref + 1e-6 * norm)
    assert np.all(got[1, 1] == 1.0)
