"""Pins for the oracle's decode attention (no GPU).

Attention is softmax(q K^T / sqrt(d)) V; tiled online softmax only reorders the sums
(hotdry blog, "Flash Attention 与 Metal 内核融合").
"""
import math

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O


def _rand(seed, B, Hq, Hkv, S, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    return q, k, v


def test_single_token_returns_its_value():
    q, k, v = _rand(1, 2, 4, 2, 7, 16)
    o = O.decode_attention(q, k, v, 1)
    for h in range(4):
        assert np.allclose(o[:, h], v[:, h // 2, 0], atol=1e-15)


def test_equal_keys_or_zero_query_average_the_values():
    q, k, v = _rand(2, 1, 2, 1, 9, 16)
    k[:] = k[:, :, :1]
    o = O.decode_attention(q, k, v, 9)
    assert np.allclose(o[0, 0], v[0, 0].mean(0), atol=1e-14)
    q0, k, v = _rand(3, 1, 2, 1, 9, 16)
    o = O.decode_attention(np.zeros_like(q0), k, v, 9)
    assert np.allclose(o[0, 1], v[0, 0].mean(0), atol=1e-14)


def test_against_library_sdpa_with_gqa_and_ragged_lengths():
    B, Hq, Hkv, S, d = 3, 6, 2, 33, 32
    q, k, v = _rand(4, B, Hq, Hkv, S, d)
    lens = np.array([33, 1, 20])
    o = O.decode_attention(q, k, v, lens)
    G = Hq // Hkv
    for b in range(B):
        L = int(lens[b])
        kk = torch.from_numpy(np.repeat(k[b, :, :L], G, axis=0))[None]
        vv = torch.from_numpy(np.repeat(v[b, :, :L], G, axis=0))[None]
        qq = torch.from_numpy(q[b])[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[0, :, 0].numpy()
        assert np.abs(o[b] - ref).max() < 1e-12


def test_brute_force_loops_on_tiny_quantized_cache():
    """Scalar Python loops over tokens (math.exp) agree with the vectorised oracle."""
    d, S = 128, 12
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 1, 1, S, d)).astype(np.float16)
    q = rng.standard_normal((1, 1, d)).astype(np.float16)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    lam = np.ones(d)
    kc, ks = O.quantize(x[0], s, lam, 4)
    vc, vs = O.quantize(x[1], s, lam, 4)
    o = O.decode_attention_quantized(q, kc, ks, vc, vs, s, s, lam, lam, S)
    kh = O.dequantize(kc, ks, s, lam)[0, 0]
    vh = O.dequantize(vc, vs, s, lam)[0, 0]
    qq = q[0, 0].astype(float)
    logits = [sum(qq[c] * kh[t, c] for c in range(d)) / math.sqrt(d) for t in range(S)]
    mx = max(logits)
    w = [math.exp(a - mx) for a in logits]
    tot = sum(w)
    ref = [sum(w[t] * vh[t, c] for t in range(S)) / tot for c in range(d)]
    assert np.abs(o[0, 0] - np.array(ref)).max() < 1e-12


def test_rotated_domain_attention_equals_plain_attention():
    """The algebra the fused decode uses: q.k_hat = (SRFT(q) * lambda) . (code * scale), and
    sum_t p_t v_hat_t = inverse_SRFT(lambda * sum_t p_t code_t scale_t)."""
    d, S, G = 128, 50, 3
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 1, 1, S, d)).astype(np.float16)
    q = rng.standard_normal((1, G, d)).astype(np.float16)
    sk = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    sv = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    lk = np.exp(rng.uniform(-1, 1, d))
    lv = np.exp(rng.uniform(-1, 1, d))
    kc, ks = O.quantize(x[0], sk, lk, 8)
    vc, vs = O.quantize(x[1], sv, lv, 4)
    o = O.decode_attention_quantized(q, kc, ks, vc, vs, sk, sv, lk, lv, S)
    qh = O.srft(q[0].astype(float), sk) * lk / np.sqrt(d)
    kr = kc[0, 0] * np.repeat(ks[0, 0].astype(float), 16, axis=-1)
    vr = vc[0, 0] * np.repeat(vs[0, 0].astype(float), 16, axis=-1)
    logits = qh @ kr.T
    p = np.exp(logits - logits.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    orot = lv * (p @ vr)
    assert np.abs(O.inverse_srft(orot, sv) - o[0]).max() < 1e-12
