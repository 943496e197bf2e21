"""GPU parity at the full sizes of the two largest workloads, in the launch configurations the
benchmark times (all layers folded into the batch, one launch per call):

  * 48 layers x 16 kv heads x 16 query heads, d = 128, 16384 tokens, int4, per-channel lambda
  * serving shard: 32 layers x 8 sequences x 8 kv heads x 32 query heads, d = 128, 32768 tokens, int4

Decode: the cache is random in-range code bytes and fp16 scales drawn on the device with a seeded
generator (10.7 GB of planes for the serving shard); sampled (sequence, kv head) units are read
back and compared with the oracle's attention over those planes, 2e-3 max-abs.  The fused
append (the benchmark's decode step) is checked the same way plus the new token's bytes, and so
are the serving shard's multi-token attention (4 query tokens, causal) and 4096-position window,
and the paged decode over the cache cut into shuffled 256-token pages.

Write path: the whole prefill of one tensor (K) is quantized in one call from fp16 values drawn on
the device; sampled vectors (random ones, the first and last vectors of work-group ranges and
rows) are compared with the oracle under the write path's bar."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_srft_amd import kvq, synth
from oracle import kvq_oracle as O

from gpu_parity import ATTN_ATOL, check_quantize, dev, oracle_unit, plan, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
W = synth.WORKLOADS


def _layout(w):
    return kvq.make_layout(w.layers * w.batch, w.kv_heads, w.q_heads, w.head_dim, w.seq_len, k_bits=w.k_bits,
                           v_bits=w.v_bits)


def _device_planes(w, seed):
    lay = _layout(w)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    kc = synth.torch_random_code_bytes(g, kvq.kvq_codes_bytes(lay, w.k_bits), w.k_bits, "cuda")
    vc = synth.torch_random_code_bytes(g, kvq.kvq_codes_bytes(lay, w.v_bits), w.v_bits, "cuda")
    n_sc = kvq.kvq_scales_bytes(lay) // 2
    # K scales wide enough that each query's softmax is dominated by tens of tokens (outputs of
    # order 1 over 32768 random keys), V scales giving values of order 1
    ks = synth.torch_random_scales(g, n_sc, 0.3, 1.6, "cuda").view(torch.int16)
    vs = synth.torch_random_scales(g, n_sc, 0.15, 0.8, "cuda").view(torch.int16)
    return lay, (kc, ks, vc, vs)


def _row(t, lay, b, j, width, np_dtype):
    """Plane row (sequence b, kv head j) of a flat device plane, as numpy [capacity, width]."""
    v = t.view(lay.batch, lay.kv_heads, lay.capacity, width)[b, j].cpu().numpy()
    return v.view(np_dtype)


def _sample_units(rng, lay, n):
    picks = {(0, 0), (lay.batch - 1, lay.kv_heads - 1), (lay.batch // 2, 0)}
    while len(picks) < n:
        picks.add((int(rng.integers(lay.batch)), int(rng.integers(lay.kv_heads))))
    return sorted(picks)


@pytest.mark.parametrize("cid", [4, 5])
@pytest.mark.parametrize("append", [False, True])
def test_decode_full_size(cid, append):
    w = W[cid]
    rng = np.random.default_rng(cid * 10 + append)
    lay, (kc, ks, vc, vs) = _device_planes(w, 1000 + cid)
    call = "decode_append" if append else "decode"
    pl = plan(lay, call, w.seq_len)
    say("full-size decode", w.name, call, pl)
    assert pl["n_chunks"] == 1 and pl["superblocks_per_wave"] == w.seq_len // 256, pl
    LB, H, G, d, S = lay.batch, lay.kv_heads, w.q_heads // w.kv_heads, w.head_dim, w.seq_len
    q = synth.to_fp16(rng.standard_normal((LB, w.q_heads, d)))
    s = synth.signs(w)
    lk = synth.random_lambda(rng, (LB, H, d), 0.5, 2.0) if w.calibrate else None
    lv = synth.random_lambda(rng, (LB, H, d), 0.5, 2.0) if w.calibrate else None
    lbs = H * d if w.calibrate else 0
    ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay, S), dtype=torch.uint8, device="cuda")
    out = torch.full((LB, w.q_heads, d), float("nan"), dtype=torch.float32, device="cuda")
    lkt = None if lk is None else dev(lk)
    lvt = None if lv is None else dev(lv)
    units = _sample_units(rng, lay, 5 if append else 8)
    if append:
        k_new = synth.to_fp16(rng.standard_normal((LB, H, d)) * 2)
        v_new = synth.to_fp16(rng.standard_normal((LB, H, d)))
        kvq.kvq_decode_attn_append(lay, dev(q), dev(k_new), dev(v_new), kc, ks, vc, vs, S, None, dev(s), dev(s), 0,
                                   lkt, lvt, lbs, 0.0, ws, out)
    else:
        kvq.kvq_decode_attn(lay, dev(q), kc, ks, vc, vs, S, None, dev(s), dev(s), 0, lkt, lvt, lbs, 0.0, ws, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    worst = 0.0
    for b, j in units:
        rows = (_row(kc, lay, b, j, d * w.k_bits // 8, np.uint8), _row(ks, lay, b, j, d // 16, np.float16),
                _row(vc, lay, b, j, d * w.v_bits // 8, np.uint8), _row(vs, lay, b, j, d // 16, np.float16))
        if append:
            lkb = 1.0 if lk is None else lk[b, j][None, None, :]
            lvb = 1.0 if lv is None else lv[b, j][None, None, :]
            uk = O.rotated_scaled(k_new[b, j][None, None, None, :], s, lkb)
            uv = O.rotated_scaled(v_new[b, j][None, None, None, :], s, lvb)
            check_quantize(rows[0][None, None, S - 1:], rows[1][None, None, S - 1:], uk, w.k_bits, "new K")
            check_quantize(rows[2][None, None, S - 1:], rows[3][None, None, S - 1:], uv, w.v_bits, "new V")
        ref = oracle_unit(q[b, j * G:(j + 1) * G], *rows, w.k_bits, w.v_bits, s, s,
                          None if lk is None else lk[b, j], None if lv is None else lv[b, j], S)
        err = float(np.abs(got[b, j * G:(j + 1) * G] - ref).max())
        worst = max(worst, err)
        assert err <= ATTN_ATOL, f"{w.name} unit ({b}, {j}): max-abs {err:.3g}"
    say("full-size decode", w.name, call, "worst max-abs", f"{worst:.3g}", "max |out|", f"{np.abs(got).max():.3g}")


def _paged_copy(planes, LB, H, S, page, seed):
    """The planes cut into pages of `page` tokens and stored in a shuffled page order; returns the
    paged planes and the page table [LB, S / page]."""
    pps = S // page
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    perm = torch.randperm(LB * pps, generator=g).to("cuda")
    out = []
    for t in planes:
        wb = t.numel() // (LB * H * S)
        nat = t.view(LB, H, pps, page, wb).permute(0, 2, 1, 3, 4).reshape(LB * pps, H, page, wb)
        pg = torch.empty_like(nat)
        pg[perm] = nat
        out.append(pg.view(-1))
    return out, perm.view(LB, pps).to(torch.int32).contiguous()


@pytest.mark.parametrize("cid", [4, 5])
def test_paged_decode_full_size(cid):
    """kvq_decode_attn_paged over the full cache cut into 256-token pages in a shuffled order, as
    benchmarked; sampled units against the oracle over the logical rows."""
    w = W[cid]
    rng = np.random.default_rng(70 + cid)
    lay, planes = _device_planes(w, 1000 + cid)
    LB, H, G, d, S = lay.batch, lay.kv_heads, w.q_heads // w.kv_heads, w.head_dim, w.seq_len
    page = 256
    paged, table = _paged_copy(planes, LB, H, S, page, 9 + cid)
    pl = plan(lay, "decode_paged", S)
    say("full-size paged decode", w.name, pl)
    q = synth.to_fp16(rng.standard_normal((LB, w.q_heads, d)))
    s = synth.signs(w)
    lk = synth.random_lambda(rng, (LB, H, d), 0.5, 2.0) if w.calibrate else None
    lv = synth.random_lambda(rng, (LB, H, d), 0.5, 2.0) if w.calibrate else None
    lbs = H * d if w.calibrate else 0
    ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay, S), dtype=torch.uint8, device="cuda")
    out = torch.full((LB, w.q_heads, d), float("nan"), dtype=torch.float32, device="cuda")
    kvq.kvq_decode_attn_paged(lay, dev(q), None, None, *paged, table, S // page, page, LB * (S // page), S, None,
                              dev(s), dev(s), 0, None if lk is None else dev(lk), None if lv is None else dev(lv), lbs,
                              0.0, ws, out)
    torch.cuda.synchronize()
    del paged
    assert int(ws[:65536].count_nonzero()) == 0, "completion counters not left at zero"
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    kc, ks, vc, vs = planes
    worst = 0.0
    for b, j in _sample_units(rng, lay, 5):
        rows = (_row(kc, lay, b, j, d * w.k_bits // 8, np.uint8), _row(ks, lay, b, j, d // 16, np.float16),
                _row(vc, lay, b, j, d * w.v_bits // 8, np.uint8), _row(vs, lay, b, j, d // 16, np.float16))
        ref = oracle_unit(q[b, j * G:(j + 1) * G], *rows, w.k_bits, w.v_bits, s, s,
                          None if lk is None else lk[b, j], None if lv is None else lv[b, j], S)
        err = float(np.abs(got[b, j * G:(j + 1) * G] - ref).max())
        worst = max(worst, err)
        assert err <= ATTN_ATOL, f"{w.name} paged unit ({b}, {j}): max-abs {err:.3g}"
    say("full-size paged decode", w.name, "worst max-abs", f"{worst:.3g}", "max |out|", f"{np.abs(got).max():.3g}")


@pytest.mark.parametrize("T,window", [(4, 0), (1, 4096)])
def test_attn_full_size(T, window):
    """kvq_attn on the full serving-shard cache in the benchmark's configuration: 4 query tokens per
    sequence (causal, speculative verification) and a 4096-position sliding window."""
    w = W[5]
    rng = np.random.default_rng(50 + T + window)
    lay, (kc, ks, vc, vs) = _device_planes(w, 1005)
    LB, H, G, d, S = lay.batch, lay.kv_heads, w.q_heads // w.kv_heads, w.head_dim, w.seq_len
    opts = kvq.make_attn_opts(n_query=T, window=window)
    p = kvq.kvq_attn_launch_plan(lay, opts, S)
    pl = {f: getattr(p, f) for f, _ in p._fields_}
    say("full-size attn", w.name, T, window, pl)
    q = synth.to_fp16(rng.standard_normal((LB, T, w.q_heads, d)))
    s = synth.signs(w)
    ws = torch.zeros(kvq.kvq_attn_workspace_bytes(lay, opts, S), dtype=torch.uint8, device="cuda")
    out = torch.full((LB, T, w.q_heads, d), float("nan"), dtype=torch.float32, device="cuda")
    kvq.kvq_attn(lay, opts, dev(q), kc, ks, vc, vs, None, 0, 0, 0, S, None, dev(s), dev(s), 0, None, None, 0, 0.0,
                 ws, out)
    torch.cuda.synchronize()
    assert int(ws[:65536].count_nonzero()) == 0, "completion counters not left at zero"
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    worst = 0.0
    for b, j in _sample_units(rng, lay, 5):
        kb = _row(kc, lay, b, j, d * w.k_bits // 8, np.uint8)
        kss = _row(ks, lay, b, j, d // 16, np.float16)
        vb = _row(vc, lay, b, j, d * w.v_bits // 8, np.uint8)
        vss = _row(vs, lay, b, j, d // 16, np.float16)
        # a window reads only the latest positions: the oracle takes those (and 64 before them)
        t0 = max(S - window - 64, 0) if window else 0
        kcodes = O.unpack_codes(kb[t0:S], w.k_bits)[None, None]
        vcodes = O.unpack_codes(vb[t0:S], w.v_bits)[None, None]
        ref = O.prefix_attention_quantized(q[b:b + 1, :, j * G:(j + 1) * G], kcodes, kss[t0:S][None, None], vcodes,
                                           vss[t0:S][None, None], s, s, 1.0, 1.0, S - t0, T, window)[0]
        err = float(np.abs(got[b, :, j * G:(j + 1) * G] - ref).max())
        worst = max(worst, err)
        assert err <= ATTN_ATOL, f"{w.name} T {T} window {window} unit ({b}, {j}): max-abs {err:.3g}"
    say("full-size attn", w.name, T, window, "worst max-abs", f"{worst:.3g}", "max |out|", f"{np.abs(got).max():.3g}")


def _device_values(w, seed):
    """fp16 [layers x batch, kv_heads, seq, d] drawn on the device: Student-t-like heavy tails
    (a normal over the root of a chi-square of 4 degrees) with a per-channel log-uniform spread."""
    LB, H, S, d = w.layers * w.batch, w.kv_heads, w.seq_len, w.head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.empty((LB, H, S, d), dtype=torch.float16, device="cuda")
    std = torch.exp(torch.empty((LB, H, 1, d), device="cuda").uniform_(np.log(0.5), np.log(4.0), generator=g))
    for i in range(LB):
        z = torch.randn((H, S, d), generator=g, device="cuda")
        c = sum(torch.randn((H, S, d), generator=g, device="cuda") ** 2 for _ in range(4)) / 4.0
        x[i] = (z / torch.sqrt(c) * std[i]).clamp_(-65504.0, 65504.0).half()
    return x


@pytest.mark.parametrize("cid", [4, 5])
def test_quantize_full_size(cid):
    w = W[cid]
    rng = np.random.default_rng(40 + cid)
    lay = _layout(w)
    LB, H, S, d = lay.batch, lay.kv_heads, w.seq_len, w.head_dim
    pl = plan(lay, "quantize", S)
    say("full-size quantize", w.name, pl)
    assert pl["blocks_per_work_group"] >= 1000, pl
    x = _device_values(w, 2000 + cid)
    s = synth.signs(w)
    lam = synth.random_lambda(rng, (LB, H, d), 0.5, 8.0) if w.calibrate else None
    codes = torch.full((kvq.kvq_codes_bytes(lay, w.k_bits),), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((kvq.kvq_scales_bytes(lay) // 2,), 0x7E00, dtype=torch.int16, device="cuda")
    kvq.kvq_quantize(lay, w.k_bits, x, 0, S, dev(s), 0, None if lam is None else dev(lam), 0 if lam is None else H * d,
                     codes, scales)
    torch.cuda.synchronize()
    # sampled vectors: random, plus the first and last vector of every 97th work-group range and
    # the vectors around row boundaries
    n_vec = LB * H * S
    nblk, grid = pl["blocks"], pl["work_groups"]
    idx = set(rng.integers(0, n_vec, 3000).tolist())
    for wg in range(0, grid, 97):
        lo, hi = wg * nblk // grid * 16, min((wg + 1) * nblk // grid * 16, n_vec)
        idx |= {lo, lo + 1, hi - 2, hi - 1}
    for r in rng.integers(1, LB * H, 64):
        idx |= {int(r) * S - 1, int(r) * S}
    idx = np.array(sorted(i for i in idx if 0 <= i < n_vec))
    it = torch.from_numpy(idx).cuda()
    xs = x.view(n_vec, d)[it].cpu().numpy()
    cw = d * w.k_bits // 8
    cs = codes.view(n_vec, cw)[it].cpu().numpy()
    ss = scales.view(n_vec, d // 16)[it].cpu().numpy().view(np.float16)
    row = idx // S
    lam_s = 1.0 if lam is None else lam.reshape(LB * H, d)[row].astype(np.float64)
    u = O.rotated_scaled(xs, s, lam_s)
    n_diff, n_ulp = check_quantize(cs, ss, u, w.k_bits, f"full-size quantize {w.name}")
    say("full-size quantize", w.name, len(idx), "vectors; tie flips", n_diff, "scale ulps", n_ulp)
    del x
