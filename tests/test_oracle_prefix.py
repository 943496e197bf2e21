"""Pins of the oracle's multi-token (causal) and sliding-window attention (readings R14, R15):
torch's scaled_dot_product_attention in float64 with an explicit position mask (a library
routine), scalar loops on a tiny cache, and the special cases the definition fixes."""
import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O


def _rand(rng, B, T, Hkv, G, S, d):
    q = rng.standard_normal((B, T, Hkv * G, d))
    k = rng.standard_normal((B, Hkv, S, d)) * 1.5
    v = rng.standard_normal((B, Hkv, S, d))
    return q, k, v


def _sdpa(q, k, v, lens, T, window):
    """torch SDPA (float64, CPU) per sequence with a boolean mask built from positions; rows whose
    position is negative are left at zero."""
    B, _, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for b in range(B):
        L = int(lens[b])
        pos = np.arange(T) + L - T
        t = np.arange(L)
        mask = t[None, :] <= pos[:, None]
        if window >= 1:
            mask &= t[None, :] >= pos[:, None] - window + 1
        live = pos >= 0
        if not live.any():
            continue
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)[:, live]                       # [Hq, T', d]
        kt = torch.from_numpy(np.repeat(k[b, :, :L], G, axis=0))                     # [Hq, L, d]
        vt = torch.from_numpy(np.repeat(v[b, :, :L], G, axis=0))
        m = torch.from_numpy(mask[live])[None].expand(Hq, -1, -1)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
        out[b, live] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("T,window", [(1, 0), (3, 0), (8, 0), (1, 7), (4, 5), (6, 1), (5, 300)])
def test_prefix_attention_matches_torch_sdpa(T, window):
    rng = np.random.default_rng(T * 31 + window)
    B, Hkv, G, S, d = 3, 2, 3, 40, 16
    q, k, v = _rand(rng, B, T, Hkv, G, S, d)
    lens = np.array([40, 17, T])
    got = O.prefix_attention(q, k, v, lens, T, window)
    ref = _sdpa(q, k, v, lens, T, window)
    assert np.abs(got - ref).max() < 1e-12


def test_prefix_attention_scalar_loops():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 2, 1, 1, 6, 4)
    L, T, W = 6, 2, 3
    got = O.prefix_attention(q, k, v, L, T, W)
    for i in range(T):
        p = L - T + i
        ts = list(range(max(0, p - W + 1), p + 1))
        logits = [sum(q[0, i, 0, c] * k[0, 0, t, c] for c in range(4)) / 2.0 for t in ts]
        mx = max(logits)
        w = [np.exp(x - mx) for x in logits]
        z = sum(w)
        for c in range(4):
            assert abs(got[0, i, 0, c] - sum(wi * v[0, 0, t, c] for wi, t in zip(w, ts)) / z) < 1e-12


def test_special_cases():
    rng = np.random.default_rng(11)
    B, Hkv, G, S, d = 2, 2, 2, 30, 8
    q, k, v = _rand(rng, B, 5, Hkv, G, S, d)
    lens = np.array([30, 12])
    # one query token and no window: single-token decode attention
    assert np.abs(O.prefix_attention(q[:, -1:], k, v, lens, 1) - O.decode_attention(q[:, -1], k, v, lens)[:, None]).max() < 1e-12
    # window 1: each query returns the value at its own position
    o = O.prefix_attention(q, k, v, lens, 5, 1)
    for b in range(B):
        for i in range(5):
            p = lens[b] - 5 + i
            assert np.abs(o[b, i] - np.repeat(v[b, :, p], G, axis=0)).max() < 1e-15
    # a window longer than the sequence is no window
    assert np.abs(O.prefix_attention(q, k, v, lens, 5, 1000) - O.prefix_attention(q, k, v, lens, 5, 0)).max() < 1e-15
    # causality: keys and values past a query's position do not change its output (sequence 0
    # holds its queries at positions 25..29; positions 27.. are perturbed)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 27:] += 5.0
    v2[0, :, 27:] -= 3.0
    o1 = O.prefix_attention(q, k, v, lens, 5, 0)
    o2 = O.prefix_attention(q, k2, v2, lens, 5, 0)
    assert np.array_equal(o1[0, :2], o2[0, :2])
    assert all(not np.allclose(o1[0, i], o2[0, i]) for i in range(2, 5))
    # queries before the start of a short sequence get zeros
    o = O.prefix_attention(q, k, v, np.array([30, 3]), 5, 0)
    assert np.all(o[1, :2] == 0.0) and np.all(np.abs(o[1, 2:]).sum(axis=-1) > 0)


def test_full_causal_self_attention():
    """T = L and no window is ordinary causal self-attention over the sequence."""
    rng = np.random.default_rng(5)
    L, H, d = 9, 2, 8
    q, k, v = _rand(rng, 1, L, H, 1, L, d)
    got = O.prefix_attention(q, k, v, L, L, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q[0]).permute(1, 0, 2),
                                                           torch.from_numpy(k[0]), torch.from_numpy(v[0]),
                                                           is_causal=True)
    assert np.abs(got[0] - ref.permute(1, 0, 2).numpy()).max() < 1e-12


def test_quantized_prefix_attention_uses_dequantized_cache():
    rng = np.random.default_rng(8)
    B, Hkv, G, S, d, T = 1, 1, 2, 50, 128, 4
    x = rng.standard_normal((B, Hkv, S, d)).astype(np.float16)
    y = rng.standard_normal((B, Hkv, S, d)).astype(np.float16)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    kc, ks = O.quantize(x, s, 1.0, 4)
    vc, vs = O.quantize(y, s, 1.0, 4)
    q = rng.standard_normal((B, T, Hkv * G, d)).astype(np.float16)
    got = O.prefix_attention_quantized(q, kc, ks, vc, vs, s, s, 1.0, 1.0, S, T, 20)
    ref = O.prefix_attention(q.astype(np.float64), O.dequantize(kc, ks, s, 1.0), O.dequantize(vc, vs, s, 1.0), S, T, 20)
    assert np.abs(got - ref).max() < 1e-13
