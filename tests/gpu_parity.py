"""Shared helpers of the GPU parity tests: run the C-ABI entry points on seeded inputs and
compare element by element with the CPU oracle.

Tolerances (fixed by the requirements of the method's port, restated here):
  * packing is bit-exact: re-packing the codes read back from the GPU bytes reproduces them;
  * fp16 scales are bit-equal, or one fp16 ulp apart in at most 0.1% of the groups;
  * in groups whose scales agree, at most 0.1% of codes differ from the oracle's, each by +-1,
    and only where u/scale is within 1e-3 of a rounding tie;
  * in groups whose scales differ by one ulp, codes are valid for the GPU's scale
    (|u/scale - code| <= 0.5 + 1e-3, or u/scale beyond qmax clamped to qmax of its sign);
  * dequantized vectors (from the oracle's planes) within 1e-3 x the vector's max-abs;
  * attention outputs (from the oracle's planes) within 2e-3 max-abs.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from kv_cache_quantization_srft_amd import kvq
from oracle import kvq_oracle as O

CODE_MISMATCH_RATE = 1e-3
TIE_WINDOW = 1e-3
DEQUANT_RTOL = 1e-3
ATTN_ATOL = 2e-3


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def planes(layout, bits, fill=0xAB):
    codes = torch.full((kvq.kvq_codes_bytes(layout, bits),), fill, dtype=torch.uint8, device="cuda")
    scales = torch.full((kvq.kvq_scales_bytes(layout) // 2,), 0x7E00, dtype=torch.int16, device="cuda")  # NaN
    return codes, scales


def gpu_quantize(x16, s, lam, bits, capacity=None, pos=0, sign_bs=0, lambda_bs=None, transform="srft", group=16,
                 entry=None):
    """x16 [B, H, n, d] fp16; lam [B?, H, d] or None.  Returns (codes u8 [B,H,cap,d*bits/8],
    scales f16 [B,H,cap,d/group]) as numpy, plus the layout.  entry: the write-path entry point
    (kvq.kvq_quantize by default, or kvq.kvq_quantize_fft)."""
    B, H, n, d = x16.shape
    cap = capacity or (pos + n)
    lay = kvq.make_layout(B, H, H, d, cap, k_bits=bits, v_bits=4, transform=transform, group_size=group)
    codes, scales = planes(lay, bits)
    lam_t = None if lam is None else dev(np.asarray(lam, np.float32))
    if lambda_bs is None:
        lambda_bs = 0 if lam is None or np.asarray(lam).ndim == 2 else H * d
    (entry or kvq.kvq_quantize)(lay, bits, dev(x16), pos, n, dev(np.asarray(s, np.float32)), sign_bs, lam_t,
                                lambda_bs, codes, scales)
    torch.cuda.synchronize()
    cb = codes.cpu().numpy().reshape(B, H, cap, d * bits // 8)
    sc = scales.cpu().numpy().view(np.float16).reshape(B, H, cap, d // group)
    return cb, sc, lay


def check_quantize(gpu_bytes, gpu_scales, u, bits, label="", group=16):
    """Compare GPU planes (for the vectors whose rotated, lambda-scaled values are u) with the
    oracle's decision.  u: float64 [..., d]; gpu_bytes/scales: matching leading shape."""
    qmax = O.QMAX[bits]
    d = u.shape[-1]
    oc, osc = O.quantize_decision(u, bits, group)
    gc = O.unpack_codes(gpu_bytes, bits)
    # packing: the GPU bytes are exactly the oracle packing of the codes they hold
    assert np.array_equal(O.pack_codes(gc, bits), gpu_bytes), f"{label}: packing not bit-exact"
    assert gc.min() >= -qmax and gc.max() <= qmax, f"{label}: code out of range"
    gs = gpu_scales.reshape(osc.shape)
    ulp = np.abs(gs.view(np.int16).astype(np.int64) - osc.view(np.int16).astype(np.int64))
    assert np.all(np.isfinite(gs.astype(np.float32))), f"{label}: non-finite scale"
    assert ulp.max() <= 1, f"{label}: scale differs by {ulp.max()} ulp"
    n_groups = ulp.size
    assert (ulp > 0).sum() <= max(1, CODE_MISMATCH_RATE * n_groups), f"{label}: {(ulp > 0).sum()} scale ulps"
    same = np.repeat(ulp == 0, group, axis=-1).reshape(gc.shape)
    diff = (gc != oc) & same
    n_diff = int(diff.sum())
    assert n_diff <= max(1, CODE_MISMATCH_RATE * gc.size), f"{label}: {n_diff} codes differ"
    if n_diff:
        assert np.abs(gc[diff].astype(int) - oc[diff].astype(int)).max() == 1, f"{label}: code off by > 1"
        sc = np.repeat(osc.astype(np.float64), group, axis=-1).reshape(u.shape)
        ratio = u[diff] / sc[diff]
        dist = np.abs(np.abs(ratio - np.floor(ratio)) - 0.5)
        assert dist.max() <= TIE_WINDOW, f"{label}: non-tie mismatch (distance {dist.max():.3g})"
    if (~same).any():
        sc = np.repeat(gs.astype(np.float64), group, axis=-1).reshape(u.shape)
        r = u[~same] / np.where(sc[~same] > 0, sc[~same], 1.0)
        err = np.abs(r - gc[~same])
        # a code is valid for the GPU's scale if it is the rounding of u / scale (within the tie
        # window), or the clamp of a ratio beyond qmax to the qmax of the same sign
        clamped = (np.abs(r) > qmax) & (gc[~same] == np.sign(r) * qmax)
        ok = ((sc[~same] == 0) & (gc[~same] == 0)) | (err <= 0.5 + TIE_WINDOW) | clamped
        assert ok.all(), f"{label}: invalid codes in 1-ulp scale groups"
    return n_diff, int((ulp > 0).sum())


def oracle_planes(x16, s, lam, bits):
    """The oracle's planes for x16 [B, H, n, d]: (codes int8, scales fp16)."""
    return O.quantize(x16, s, lam, bits)


def gpu_decode(q16, kc8, ks16, vc8, vs16, k_bits, s_k, s_v, lam_k, lam_v, seq_len, seq_lens=None, sm_scale=0.0,
               capacity=None, sign_bs=0, lambda_bs=0, ws=None, transform="srft", v_bits=4):
    """Run kvq_decode_attn on given unpacked int8 codes (packed here by the oracle's packing)."""
    B, Hkv, S, d = kc8.shape
    Hq = q16.shape[1]
    cap = capacity or S
    lay = kvq.make_layout(B, Hkv, Hq, d, cap, k_bits=k_bits, v_bits=v_bits, transform=transform)
    kb = O.pack_codes(kc8, k_bits)
    vb = O.pack_codes(vc8, v_bits)
    if ws is None:
        ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay, seq_len), dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lk = None if lam_k is None else dev(np.asarray(lam_k, np.float32))
    lv = None if lam_v is None else dev(np.asarray(lam_v, np.float32))
    sl = None if seq_lens is None else dev(np.asarray(seq_lens, np.int32))
    kvq.kvq_decode_attn(lay, dev(q16), dev(kb), dev(ks16.view(np.int16)), dev(vb), dev(vs16.view(np.int16)),
                        seq_len, sl, dev(np.asarray(s_k, np.float32)), dev(np.asarray(s_v, np.float32)), sign_bs,
                        lk, lv, lambda_bs, sm_scale, ws, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def gpu_decode_fp16(q16, k16, v16, seq_len, seq_lens=None, sm_scale=0.0, ws=None):
    B, Hkv, S, d = k16.shape
    Hq = q16.shape[1]
    lay = kvq.make_layout(B, Hkv, Hq, d, S)
    if ws is None:
        ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay, seq_len), dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    sl = None if seq_lens is None else dev(np.asarray(seq_lens, np.int32))
    kvq.kvq_decode_attn_fp16(lay, dev(q16), dev(k16), dev(v16), seq_len, sl, sm_scale, ws, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def plan(layout, call, n):
    """The launch plan of a call (kvq_launch_plan) as a dict."""
    p = kvq.kvq_launch_plan(layout, call, n)
    return {f: getattr(p, f) for f, _ in p._fields_}


def gpu_decode_planes(lay, q16, kb, ks16, vb, vs16, seq_len, seq_lens, s_k, s_v, lam_k, lam_v, lambda_bs,
                      sm_scale=0.0, page=None):
    """kvq_decode_attn (or kvq_decode_attn_paged when page = (table [B, pps], page_size, num_pages))
    on packed planes given as numpy arrays; returns the output [B, Hq, d] as float64."""
    B, Hq, d = lay.batch, lay.q_heads, lay.head_dim
    ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay, seq_len), dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    args = (dev(kb), dev(ks16.view(np.int16)), dev(vb), dev(vs16.view(np.int16)))
    sl = None if seq_lens is None else dev(np.asarray(seq_lens, np.int32))
    lk = None if lam_k is None else dev(np.asarray(lam_k, np.float32))
    lv = None if lam_v is None else dev(np.asarray(lam_v, np.float32))
    if page is None:
        kvq.kvq_decode_attn(lay, dev(q16), *args, seq_len, sl, dev(s_k), dev(s_v), 0, lk, lv, lambda_bs, sm_scale, ws,
                            out)
    else:
        table, page_size, num_pages = page
        kvq.kvq_decode_attn_paged(lay, dev(q16), None, None, *args, dev(np.asarray(table, np.int32)), table.shape[1],
                                  page_size, num_pages, seq_len, sl, dev(s_k), dev(s_v), 0, lk, lv, lambda_bs,
                                  sm_scale, ws, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def oracle_unit(q16, kb, ks16, vb, vs16, k_bits, v_bits, s_k, s_v, lk_row, lv_row, L, sm_scale=None,
                transform="srft"):
    """The oracle's decode attention of one (sequence, kv head): q16 [G, d]; kb, vb packed code rows
    [>= L, bytes]; ks16, vs16 [>= L, d/16]; lk_row, lv_row [d] or None.  Returns [G, d] float64."""
    G, d = q16.shape
    if L == 0:
        return np.zeros((G, d))
    kc = O.unpack_codes(kb[:L], k_bits)[None, None]
    vc = O.unpack_codes(vb[:L], v_bits)[None, None]
    lk = 1.0 if lk_row is None else np.asarray(lk_row, np.float64)[None, None, None, :]
    lv = 1.0 if lv_row is None else np.asarray(lv_row, np.float64)[None, None, None, :]
    return O.decode_attention_quantized(q16[None], kc, ks16[:L][None, None], vc, vs16[:L][None, None], s_k, s_v,
                                        lk, lv, L, sm_scale=sm_scale, transform=transform)[0]
