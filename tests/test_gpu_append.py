"""GPU parity of kvq_decode_attn_append (one launch: the write path on the step's new K/V
vectors at position L - 1 of every row, then decode attention over the cache holding them)
against the CPU oracle, through the C ABI.

Bars: the new token's bytes meet the write path's bar (packing bit-exact, codes within the tie
rule); every other byte of the planes is untouched; the output matches the oracle's attention
over the planes the GPU left (the same planes for both sides) within 2e-3 max-abs; rows of
length 0 are neither written nor attended.  With uniform lengths the fused call and the
unfused sequence (kvq_quantize + kvq_quantize + kvq_decode_attn) are compared as well."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_srft_amd import kvq, synth
from oracle import kvq_oracle as O

from gpu_parity import ATTN_ATOL, check_quantize, dev, say

pytestmark = pytest.mark.gpu


def _inputs(seed, B, Hkv, G, S, d, lam, transform):
    rng = np.random.default_rng(seed)
    k = synth.to_fp16(rng.standard_t(3, size=(B, Hkv, S, d)) * np.where(rng.random((B, Hkv, 1, d)) < 0.03, 20, 1))
    v = synth.to_fp16(rng.standard_normal((B, Hkv, S, d)))
    q = synth.to_fp16(rng.standard_normal((B, Hkv * G, d)))
    sk = synth.random_signs(seed * 7 + 1, d)
    sv = synth.random_signs(seed * 7 + 2, d)
    lk = O.calibrate_lambda(k, sk, min(S, 256), transform).astype(np.float32) if lam else None
    lv = O.calibrate_lambda(v, sv, min(S, 256), transform).astype(np.float32) if lam else None
    return k, v, q, sk, sv, lk, lv


def _planes(k, v, sk, sv, lk, lv, kb, transform, vb=4):
    l4 = lambda x: 1.0 if x is None else x[:, :, None, :]
    kc, ks = O.quantize(k, sk, l4(lk), kb, transform=transform)
    vc, vs = O.quantize(v, sv, l4(lv), vb, transform=transform)
    return O.pack_codes(kc, kb), ks.copy(), O.pack_codes(vc, vb), vs.copy()


def _run_append(lay, q, k_new, v_new, pl, seq_len, lens, sk, sv, lk, lv):
    B, Hkv, d = lay.batch, lay.kv_heads, lay.head_dim
    kcb, ksb, vcb, vsb = (dev(a) for a in (pl[0], pl[1].view(np.int16), pl[2], pl[3].view(np.int16)))
    ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay, seq_len), dtype=torch.uint8, device="cuda")
    out = torch.full((B, lay.q_heads, d), float("nan"), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attn_append(lay, dev(q), dev(k_new), dev(v_new), kcb, ksb, vcb, vsb, seq_len,
                               None if lens is None else dev(np.asarray(lens, np.int32)), dev(sk), dev(sv), 0,
                               None if lk is None else dev(lk), None if lv is None else dev(lv),
                               0 if lk is None else Hkv * d, 0.0, ws, out)
    torch.cuda.synchronize()
    got = (kcb.cpu().numpy(), ksb.cpu().numpy().view(np.float16), vcb.cpu().numpy(),
           vsb.cpu().numpy().view(np.float16))
    return got, out.cpu().numpy().astype(np.float64)


CASES = [
    # d, G, k_bits, S, lens, lambda, transform, v_bits
    (128, 6, 4, 1500, [1500, 700, 257, 1], True, "srft", 4),
    (128, 1, 4, 256, None, False, "srft", 4),
    (256, 4, 8, 900, [900, 1, 513], False, "srft", 4),
    (128, 16, 4, 600, [600, 0, 65], True, "srft", 4),
    (128, 6, 4, 1100, [1100, 64], True, "srht", 4),
    (256, 4, 4, 700, [700, 300], True, "srht", 4),
    (128, 6, 4, 800, [800, 129], True, "srft", 8),
    (256, 2, 8, 500, [500, 3], True, "srft", 8),
]


@pytest.mark.parametrize("d,G,kb,S,lens,lam,transform,vb", CASES)
def test_append_parity(d, G, kb, S, lens, lam, transform, vb):
    Hkv = 2
    B = 1 if lens is None else len(lens)
    k, v, q, sk, sv, lk, lv = _inputs(d + G + S, B, Hkv, G, S, d, lam, transform)
    L = np.full(B, S) if lens is None else np.clip(np.asarray(lens), 0, S)
    pl = _planes(k, v, sk, sv, lk, lv, kb, transform, vb)
    # the step's new vectors and, at their slots, stale bytes that the call must overwrite
    rng = np.random.default_rng(5)
    k_new = synth.to_fp16(rng.standard_normal((B, Hkv, d)) * 3)
    v_new = synth.to_fp16(rng.standard_normal((B, Hkv, d)))
    before = [a.copy() for a in pl]
    for b in range(B):
        if L[b] >= 1:
            k_new[b] = k[b, :, L[b] - 1]
            for a in before:
                a[b, :, L[b] - 1] = np.array(0xAB, a.dtype) if a.dtype == np.uint8 else np.float16(-7.5)
    lay = kvq.make_layout(B, Hkv, Hkv * G, d, S, k_bits=kb, v_bits=vb, transform=transform)
    say("append", d, G, kb, vb, S, lens, lam, transform)
    got, out = _run_append(lay, q, k_new, v_new, before, S, lens, sk, sv, lk, lv)
    # untouched elsewhere, bit-exact
    for b in range(B):
        keep = np.ones(S, bool)
        if L[b] >= 1:
            keep[L[b] - 1] = False
        for g_, bf in zip(got, before):
            assert np.array_equal(g_[b][:, keep].view(np.uint8), bf[b][:, keep].view(np.uint8)), f"row {b} touched"
    # the new token meets the write path's bar
    live = np.nonzero(L >= 1)[0]
    l4 = lambda x: 1.0 if x is None else x[live][:, :, None, :]
    uk = O.rotated_scaled(k_new[live][:, :, None, :], sk, l4(lk), transform=transform)
    uv = O.rotated_scaled(v_new[live][:, :, None, :], sv, l4(lv), transform=transform)
    sel = lambda a: np.stack([a[b][:, L[b] - 1:L[b]] for b in live])
    check_quantize(sel(got[0]), sel(got[1]), uk, kb, label="append K")
    check_quantize(sel(got[2]), sel(got[3]), uv, vb, label="append V")
    # attention over the planes the GPU left, on both sides
    ref = np.zeros_like(out)
    kc = O.unpack_codes(got[0], kb)
    vc = O.unpack_codes(got[2], vb)
    ref[live] = O.decode_attention_quantized(q[live], kc[live], got[1][live], vc[live], got[3][live], sk, sv,
                                             l4(lk), l4(lv), L[live], transform=transform)
    assert np.abs(out - ref).max() <= ATTN_ATOL
    assert np.all(out[L == 0] == 0.0)


@pytest.mark.parametrize("d,G,kb,S", [(128, 6, 4, 1000), (256, 4, 8, 600), (128, 2, 8, 300)])
def test_append_matches_unfused(d, G, kb, S):
    """Uniform lengths: the fused call leaves the same planes as kvq_quantize at pos = S - 1
    (up to the write path's tie rule) and returns the decode of those planes."""
    Hkv, B = 2, 2
    k, v, q, sk, sv, lk, lv = _inputs(d * G + S, B, Hkv, G, S, d, True, "srft")
    pl = _planes(k, v, sk, sv, lk, lv, kb, "srft")
    k_new = np.ascontiguousarray(k[:, :, S - 1])
    v_new = np.ascontiguousarray(v[:, :, S - 1])
    lay = kvq.make_layout(B, Hkv, Hkv * G, d, S, k_bits=kb, v_bits=4)
    say("append vs unfused", d, G, kb, S)
    got, out = _run_append(lay, q, k_new, v_new, pl, S, None, sk, sv, lk, lv)
    # unfused: two single-token quantize calls, then decode, on fresh copies of the planes
    kcb, ksb, vcb, vsb = (dev(a) for a in (pl[0], pl[1].view(np.int16), pl[2], pl[3].view(np.int16)))
    lkt, lvt = dev(lk), dev(lv)
    kvq.kvq_quantize(lay, kb, dev(k_new), S - 1, 1, dev(sk), 0, lkt, Hkv * d, kcb, ksb)
    kvq.kvq_quantize(lay, 4, dev(v_new), S - 1, 1, dev(sv), 0, lvt, Hkv * d, vcb, vsb)
    ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay, S), dtype=torch.uint8, device="cuda")
    out2 = torch.empty((B, Hkv * G, d), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attn(lay, dev(q), kcb, ksb, vcb, vsb, S, None, dev(sk), dev(sv), 0, lkt, lvt, Hkv * d, 0.0, ws,
                        out2)
    torch.cuda.synchronize()
    ref_planes = (kcb.cpu().numpy(), ksb.cpu().numpy().view(np.float16), vcb.cpu().numpy(),
                  vsb.cpu().numpy().view(np.float16))
    n_diff = sum(int((a.view(np.uint8) != b_.view(np.uint8)).sum()) for a, b_ in zip(got, ref_planes))
    say("append vs unfused: differing plane bytes", n_diff)
    if n_diff == 0:
        assert np.array_equal(out, out2.cpu().numpy().astype(np.float64))
    else:
        # differences may only come from rounding ties of the new token (checked against the oracle)
        uk = O.rotated_scaled(k_new[:, :, None, :], sk, lk[:, :, None, :])
        check_quantize(got[0][:, :, S - 1:S], got[1][:, :, S - 1:S], uk, kb, label="fused K")
        assert np.abs(out - out2.cpu().numpy()).max() <= ATTN_ATOL
