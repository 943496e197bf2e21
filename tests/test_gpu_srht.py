"""GPU parity of the SRHT variant (layout.transform = KVQ_TRANSFORM_SRHT: d^-1/2 H diag(s) x,
the pages' alternative rotation) against the CPU oracle, through the C ABI: write path,
dequantize, calibration and fused decode, at d = 128 and d = 256, with the same tolerances as
the SRFT path."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_srft_amd import kvq, synth
from oracle import kvq_oracle as O

from gpu_parity import ATTN_ATOL, DEQUANT_RTOL, check_quantize, dev, gpu_decode, gpu_quantize, say

pytestmark = pytest.mark.gpu
T = "srht"


@pytest.mark.parametrize("d,bits,lam", [(128, 4, True), (128, 8, False), (256, 8, False), (256, 4, True)])
def test_write_path(d, bits, lam):
    rng = np.random.default_rng(100 + d + bits)
    B, H, n = 2, 3, 257
    x = synth.to_fp16(rng.standard_t(3, size=(B, H, n, d)) * np.where(rng.random((B, H, 1, d)) < 0.03, 20, 1))
    s = synth.random_signs(7 * d, d)
    la = O.calibrate_lambda(x, s, 128, transform=T)[0].astype(np.float32) if lam else None
    say("srht quantize", d, bits, lam)
    cb, sc, _ = gpu_quantize(x, s, la, bits, transform=T)
    u = O.rotated_scaled(x, s, 1.0 if la is None else la[None, :, None, :], transform=T)
    check_quantize(cb, sc, u, bits, label=f"srht d{d} b{bits}")


@pytest.mark.parametrize("d,bits", [(128, 4), (256, 8)])
def test_dequantize(d, bits):
    rng = np.random.default_rng(200 + d)
    B, H, n = 2, 2, 300
    x = synth.to_fp16(rng.standard_normal((B, H, n, d)))
    s = synth.random_signs(d + 3, d)
    lam = np.exp(rng.uniform(-1, 1, (H, d))).astype(np.float32)
    oc, osc = O.quantize(x, s, lam[None, :, None, :], bits, transform=T)
    lay = kvq.make_layout(B, H, H, d, n, transform=T)
    out = torch.full((B * H * n * d,), float("nan"), dtype=torch.float32, device="cuda")
    say("srht dequantize", d, bits)
    kvq.kvq_dequantize(lay, bits, dev(O.pack_codes(oc, bits)), dev(osc.view(np.int16)), 0, n, dev(s), 0, dev(lam), 0,
                       out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(B, H, n, d).astype(np.float64)
    ref = O.dequantize(oc, osc, s, lam[None, :, None, :], transform=T)
    assert np.all(np.abs(got - ref).max(-1) <= DEQUANT_RTOL * np.abs(ref).max(-1) + 1e-30)


@pytest.mark.parametrize("d", [128, 256])
def test_calibrate(d):
    rng = np.random.default_rng(300 + d)
    B, H, n = 1, 2, 600
    x = synth.to_fp16(rng.standard_t(3, size=(B, H, n, d)))
    s = synth.random_signs(d + 5, d)
    lay = kvq.make_layout(B, H, H, d, n, transform=T)
    lam = torch.full((B * H * d,), float("nan"), dtype=torch.float32, device="cuda")
    say("srht calibrate", d)
    kvq.kvq_calibrate_lambda(lay, dev(x), n, 512, dev(s), 0, lam)
    torch.cuda.synchronize()
    got = lam.cpu().numpy().reshape(B, H, d)
    ref = O.calibrate_lambda(x, s, 512, transform=T)
    norm = np.linalg.norm(x[:, :, :512].astype(np.float64), axis=-1).max(-1)[..., None]
    assert np.all(np.abs(got - ref) <= 1e-5 * ref + 1e-6 * norm)


@pytest.mark.parametrize("d,G,kb,S", [(128, 6, 4, 1500), (128, 1, 4, 200), (256, 4, 8, 900)])
def test_decode(d, G, kb, S):
    rng = np.random.default_rng(400 + d + G)
    B, Hkv = 2, 2
    k = synth.to_fp16(rng.standard_t(3, size=(B, Hkv, S, d)) * np.where(rng.random((B, Hkv, 1, d)) < 0.03, 20, 1))
    v = synth.to_fp16(rng.standard_normal((B, Hkv, S, d)))
    q = synth.to_fp16(rng.standard_normal((B, Hkv * G, d)))
    sk = synth.random_signs(11 * d, d)
    sv = synth.random_signs(13 * d, d)
    lk = O.calibrate_lambda(k, sk, 256, transform=T).astype(np.float32)
    lv = O.calibrate_lambda(v, sv, 256, transform=T).astype(np.float32)
    kc, ks = O.quantize(k, sk, lk[:, :, None, :], kb, transform=T)
    vc, vs = O.quantize(v, sv, lv[:, :, None, :], 4, transform=T)
    say("srht decode", d, G, kb, S)
    got = gpu_decode(q, kc, ks, vc, vs, kb, sk, sv, lk, lv, S, seq_lens=[S, S // 3], lambda_bs=Hkv * d, transform=T)
    ref = O.decode_attention_quantized(q, kc, ks, vc, vs, sk, sv, lk[:, :, None, :], lv[:, :, None, :], [S, S // 3],
                                       transform=T)
    assert np.abs(got - ref).max() <= ATTN_ATOL
