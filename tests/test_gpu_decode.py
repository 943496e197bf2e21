"""GPU parity of the fused decode attention (kvq_decode_attn) and the fp16 comparator
(kvq_decode_attn_fp16) against the CPU oracle, through the C ABI.

The quantized decode is compared on the oracle's own planes, so its tolerance measures the
read path alone (the write path's rounding-tie freedom is judged in the quantize tests)."""
import numpy as np
import pytest

from kv_cache_quantization_srft_amd import synth
from oracle import kvq_oracle as O

from gpu_parity import ATTN_ATOL, gpu_decode, gpu_decode_fp16, say

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def _case(rng, B, Hkv, G, S, d, k_bits, lam=True, dist="t4"):
    Hq = Hkv * G
    if dist == "t4":
        k = synth.to_fp16(rng.standard_t(4, size=(B, Hkv, S, d)) * np.where(rng.random((B, Hkv, 1, d)) < 0.03, 20, 1))
    else:
        k = synth.to_fp16(rng.standard_normal((B, Hkv, S, d)))
    v = synth.to_fp16(rng.standard_normal((B, Hkv, S, d)))
    q = synth.to_fp16(rng.standard_normal((B, Hq, d)))
    sk = synth.random_signs(int(rng.integers(1 << 30)), d)
    sv = synth.random_signs(int(rng.integers(1 << 30)), d)
    lk = O.calibrate_lambda(k, sk, min(S, 512)).astype(np.float32) if lam else None
    lv = O.calibrate_lambda(v, sv, min(S, 512)).astype(np.float32) if lam else None
    return q, k, v, sk, sv, lk, lv


def _check(q, k, v, sk, sv, lk, lv, k_bits, seq_len, seq_lens=None, label="", v_bits=4):
    B, Hkv, S, d = k.shape
    lkb = None if lk is None else lk[:, :, None, :]
    lvb = None if lv is None else lv[:, :, None, :]
    kc, ks = O.quantize(k, sk, 1.0 if lk is None else lkb, k_bits)
    vc, vs = O.quantize(v, sv, 1.0 if lv is None else lvb, v_bits)
    # device lengths are clamped to [0, seq_len]; a length-0 sequence has a zero output (API rule)
    lens = np.full(B, seq_len) if seq_lens is None else np.clip(np.asarray(seq_lens), 0, seq_len)
    say("decode", label, (B, Hkv, q.shape[1], S, d), k_bits, seq_len)
    got = gpu_decode(q, kc, ks, vc, vs, k_bits, sk, sv, lk, lv, seq_len, seq_lens,
                     lambda_bs=0 if lk is None else Hkv * d, v_bits=v_bits)
    ref = np.zeros_like(got)
    live = lens > 0
    if live.any():
        sel = lambda a: a if np.ndim(a) == 0 else a[live]
        ref[live] = O.decode_attention_quantized(q[live], kc[live], ks[live], vc[live], vs[live], sk, sv,
                                                 1.0 if lk is None else sel(lkb), 1.0 if lv is None else sel(lvb),
                                                 lens[live])
    err = np.abs(got - ref).max()
    assert np.isfinite(got).all(), label
    assert err <= ATTN_ATOL, f"{label}: max-abs {err:.3g}"
    return err


@pytest.mark.parametrize("G", [1, 2, 3, 4, 6, 8, 12])
def test_gqa_ratios_d128_int4(G):
    rng = np.random.default_rng(G)
    args = _case(rng, 2, 2, G, 777, 128, 4)
    _check(*args, 4, 777, label=f"G{G}")


@pytest.mark.parametrize("G", [1, 4])
def test_d256_k8v4(G):
    rng = np.random.default_rng(100 + G)
    args = _case(rng, 1, 2, G, 1030, 256, 8, lam=False, dist="normal")
    _check(*args, 8, 1030, label=f"k8v4 G{G}")


@pytest.mark.parametrize("d,kb,G,S,lens", [(128, 4, 6, 1111, [1111, 300]), (128, 8, 4, 700, None),
                                           (128, 4, 16, 515, [515, 1]), (256, 4, 4, 900, [900, 77]),
                                           (256, 8, 2, 600, None)])
def test_int8_values(d, kb, G, S, lens):
    """The other bit pairings: int8 V codes (K4V8, K8V8)."""
    rng = np.random.default_rng(d + kb + G)
    B = 2
    args = _case(rng, B, 2, G, S, d, kb, lam=True)
    _check(*args, kb, S, seq_lens=lens, label=f"K{kb}V8 d{d} G{G}", v_bits=8)


@pytest.mark.parametrize("d", [128, 256])
def test_int8_values_large_scales(d):
    """int8 V whose group scales exceed 512 (tiny lambda_V makes u = SRFT(v) / lambda ~ 1e5, while
    the dequantized values stay O(1)): the superblocks that hold such scales take the
    range-safe form (scale / 128 in B, p * 128 in A)."""
    rng = np.random.default_rng(7 + d)
    q, k, v, sk, sv, lk, lv = _case(rng, 2, 2, 4, 600, d, 4, lam=True)
    lv = np.full_like(lv, 1e-5)
    lv[1, 1] = O.calibrate_lambda(v, sv, 256)[1, 1]  # one row of ordinary scales beside them
    _check(q, k, v, sk, sv, lk, lv, 4, 600, seq_lens=[600, 333], label=f"K4V8 big scales d{d}", v_bits=8)


def test_tiny_workload_and_single_token():
    w = W[1]
    s = synth.signs(w)
    k = synth.kv(w, 0, synth.K_TENSOR)
    v = synth.kv(w, 0, synth.V_TENSOR)
    q = synth.query(w, 0)
    _check(q, k, v, s, s, None, None, 4, 256, label="tiny")
    _check(q, k, v, s, s, None, None, 4, 1, label="tiny len1")


def test_ragged_sequence_lengths():
    rng = np.random.default_rng(7)
    q, k, v, sk, sv, lk, lv = _case(rng, 4, 2, 3, 1500, 128, 4)
    _check(q, k, v, sk, sv, lk, lv, 4, 1500, seq_lens=[1500, 1, 0, 999], label="seq_lens")
    _check(q, k, v, sk, sv, lk, lv, 4, 1000, seq_lens=[1000, 5000, -3, 257], label="clamped seq_lens")


def test_qwen_like_layers_folded_into_batch():
    """Two layers of the Qwen-like workload folded into the batch with per-row lambda."""
    w = W[2]
    s = synth.signs(w)
    ks, vs, qs, lks, lvs = [], [], [], [], []
    for layer in (0, 13):
        k = synth.kv(w, layer, synth.K_TENSOR)
        v = synth.kv(w, layer, synth.V_TENSOR)
        ks.append(k)
        vs.append(v)
        qs.append(synth.query(w, layer))
        lks.append(O.calibrate_lambda(k, s, w.n_cal).astype(np.float32))
        lvs.append(O.calibrate_lambda(v, s, w.n_cal).astype(np.float32))
    k = np.concatenate(ks)
    v = np.concatenate(vs)
    q = np.concatenate(qs)
    _check(q, k, v, s, s, np.concatenate(lks), np.concatenate(lvs), 4, w.seq_len, label="qwen 2 layers")


def test_sm_scale_override():
    rng = np.random.default_rng(12)
    q, k, v, sk, sv, lk, lv = _case(rng, 1, 1, 2, 300, 128, 4)
    kc, ks = O.quantize(k, sk, lk[:, :, None, :], 4)
    vc, vs = O.quantize(v, sv, lv[:, :, None, :], 4)
    say("decode sm_scale")
    got = gpu_decode(q, kc, ks, vc, vs, 4, sk, sv, lk, lv, 300, sm_scale=0.05, lambda_bs=128)
    ref = O.decode_attention_quantized(q, kc, ks, vc, vs, sk, sv, lk[:, :, None, :], lv[:, :, None, :], 300,
                                       sm_scale=0.05)
    assert np.abs(got - ref).max() <= ATTN_ATOL


@pytest.mark.parametrize("d,G", [(128, 1), (128, 6), (256, 4)])
def test_fp16_decode(d, G):
    rng = np.random.default_rng(d + G)
    B, Hkv, S = 2, 2, 901
    k = synth.to_fp16(rng.standard_normal((B, Hkv, S, d)) * 2)
    v = synth.to_fp16(rng.standard_normal((B, Hkv, S, d)))
    q = synth.to_fp16(rng.standard_normal((B, Hkv * G, d)))
    say("fp16 decode", d, G)
    got = gpu_decode_fp16(q, k, v, S, seq_lens=[S, 17])
    ref = O.decode_attention(q, k, v, [S, 17])
    assert np.abs(got - ref).max() <= ATTN_ATOL


def test_shared_workspace_across_shapes():
    """One workspace, zeroed once, serves a sequence of quantized and fp16 calls of different
    shapes (unit and chunk counts change between calls); every call matches the oracle and the
    completion counters are back at zero afterwards (the workspace contract of the C ABI)."""
    import torch
    from kv_cache_quantization_srft_amd import kvq

    rng = np.random.default_rng(31)
    lay_big = kvq.make_layout(6, 4, 24, 256, 3000, k_bits=8, v_bits=4)
    ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay_big, 3000), dtype=torch.uint8, device="cuda")
    shapes = [(2, 2, 6, 1200, 128, 4), (6, 4, 3, 3000, 128, 4), (1, 1, 4, 700, 256, 8), (2, 2, 6, 1200, 128, 4),
              (5, 3, 2, 2100, 128, 8)]
    for i, (B, Hkv, G, S, d, kb) in enumerate(shapes):
        q, k, v, sk, sv, lk, lv = _case(rng, B, Hkv, G, S, d, kb)
        kc, ks = O.quantize(k, sk, lk[:, :, None, :], kb)
        vc, vs = O.quantize(v, sv, lv[:, :, None, :], 4)
        say("shared workspace", i, (B, Hkv, G, S, d, kb))
        got = gpu_decode(q, kc, ks, vc, vs, kb, sk, sv, lk, lv, S, lambda_bs=Hkv * d, ws=ws)
        ref = O.decode_attention_quantized(q, kc, ks, vc, vs, sk, sv, lk[:, :, None, :], lv[:, :, None, :], S)
        assert np.abs(got - ref).max() <= ATTN_ATOL, f"call {i}"
        assert int(ws[:65536].count_nonzero()) == 0, f"counters not reset after call {i}"
        if i % 2 == 0:
            got16 = gpu_decode_fp16(q, k, v, S, ws=ws)
            assert np.abs(got16 - O.decode_attention(q, k, v, S)).max() <= ATTN_ATOL, f"fp16 call {i}"
            assert int(ws[:65536].count_nonzero()) == 0, f"counters not reset after fp16 call {i}"


@pytest.mark.parametrize("seed", [1634, 7, 2024])
def test_keys_beyond_a_wide_calibrated_lambda(seed):
    """Student-t (nu = 3) keys with x20 outlier channels and lambda_K calibrated on the first 256
    tokens: lambda_K spans more than a decade and later keys exceed it, so the rotated query has
    a wide dynamic range across channels.  The query digits must keep the score error small
    relative to the largest channel (a 16-bit query gave 2.9e-3 here, over the 2e-3 bar)."""
    rng = np.random.default_rng(seed)
    B, Hkv, G, S, d = 4, 2, 6, 1500, 128
    k = synth.to_fp16(rng.standard_t(3, size=(B, Hkv, S, d)) * np.where(rng.random((B, Hkv, 1, d)) < 0.03, 20, 1))
    v = synth.to_fp16(rng.standard_normal((B, Hkv, S, d)))
    q = synth.to_fp16(rng.standard_normal((B, Hkv * G, d)))
    sk = synth.random_signs(seed * 5 + 1, d)
    sv = synth.random_signs(seed * 5 + 2, d)
    lk = O.calibrate_lambda(k, sk, 256).astype(np.float32)
    lv = O.calibrate_lambda(v, sv, 256).astype(np.float32)
    _check(q, k, v, sk, sv, lk, lv, 4, S, [1500, 700, 257, 1], label=f"wide lambda seed {seed}")
