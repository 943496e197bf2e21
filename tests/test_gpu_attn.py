"""GPU parity of kvq_attn -- several query tokens per sequence with a causal mask, sliding windows,
ring-buffer rows and paged caches -- against the oracle's prefix attention (readings R14-R16),
through the C ABI.

The caches are random in-range code bytes and fp16 scales (synth's random planes).  The oracle
works on logical rows; ring-buffer and paged planes are laid out from those rows here, so the
storage conventions are checked by the same comparison.  Sampled (sequence, kv head) units are
compared element by element, 2e-3 max-abs; every test asserts the launch shape it exercises."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_srft_amd import kvq, synth
from oracle import kvq_oracle as O

from gpu_parity import ATTN_ATOL, dev, gpu_decode_planes, say

pytestmark = pytest.mark.gpu

K4, K8, V4, V8 = (0.15, 0.8), (0.01, 0.06), (0.15, 0.8), (0.01, 0.06)


def _cache(rng, B, Hkv, S, d, kb, vb, lam=(0.5, 2.0)):
    kbytes = synth.random_code_bytes(rng, (B, Hkv, S, d * kb // 8), kb)
    vbytes = synth.random_code_bytes(rng, (B, Hkv, S, d * vb // 8), vb)
    ks = synth.random_scales(rng, (B, Hkv, S, d // 16), *(K4 if kb == 4 else K8))
    vs = synth.random_scales(rng, (B, Hkv, S, d // 16), *(V4 if vb == 4 else V8))
    lk = None if lam is None else synth.random_lambda(rng, (B, Hkv, d), *lam)
    lv = None if lam is None else synth.random_lambda(rng, (B, Hkv, d), *lam)
    return kbytes, ks, vbytes, vs, lk, lv


def _oracle_unit(q, cache, b, j, G, L, T, W, kb, vb, sk, sv):
    """Oracle output of unit (b, j): [T, G, d]."""
    kbytes, ks, vbytes, vs, lk, lv = cache
    n = max(L, 1)
    kc = O.unpack_codes(kbytes[b, j, :n], kb)[None, None]
    vc = O.unpack_codes(vbytes[b, j, :n], vb)[None, None]
    lkb = 1.0 if lk is None else lk[b, j][None, None, None, :].astype(np.float64)
    lvb = 1.0 if lv is None else lv[b, j][None, None, None, :].astype(np.float64)
    return O.prefix_attention_quantized(q[b:b + 1, :, j * G:(j + 1) * G], kc, ks[b, j, :n][None, None], vc,
                                        vs[b, j, :n][None, None], sk, sv, lkb, lvb, L, T, W)[0]


def _run_attn(lay, opts, q, planes, seq_len, lens, sk, sv, lk, lv, page=None):
    """planes: (kbytes, ks, vbytes, vs) numpy in the call's storage; page = (table, page_size,
    num_pages) or None.  Returns out [B, T, Hq, d] float64."""
    B, T, Hq, d = q.shape
    ws = torch.zeros(kvq.kvq_attn_workspace_bytes(lay, opts, seq_len), dtype=torch.uint8, device="cuda")
    out = torch.full((B, T, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    kbytes, ks, vbytes, vs = planes
    tbl, ps, npg = (None, 0, 0) if page is None else (dev(np.asarray(page[0], np.int32)), page[1], page[2])
    pps = 0 if page is None else page[0].shape[1]
    kvq.kvq_attn(lay, opts, dev(q), dev(kbytes), dev(ks.view(np.int16)), dev(vbytes), dev(vs.view(np.int16)), tbl,
                 pps, ps, npg, seq_len, None if lens is None else dev(np.asarray(lens, np.int32)), dev(sk), dev(sv), 0,
                 None if lk is None else dev(lk), None if lv is None else dev(lv),
                 0 if lk is None else lay.kv_heads * d, 0.0, ws, out)
    torch.cuda.synchronize()
    assert int(ws[:65536].count_nonzero()) == 0, "completion counters not left at zero"
    return out.cpu().numpy().astype(np.float64)


def _lengths(rng, B, S, T):
    special = [S, 0, 1, T - 1, T, T + 1, 63, 64, 65, 257, S - 1]
    lens = rng.integers(1, S + 1, size=B)
    lens[: min(B, len(special))] = [min(max(x, 0), S) for x in special[:B]]
    return lens


def _units(rng, B, Hkv, n):
    n = min(n, B * Hkv)
    picks = {(0, 0), (B - 1, Hkv - 1)}
    picks |= {(b, int(rng.integers(Hkv))) for b in range(min(B, 11))}
    while len(picks) < n:
        picks.add((int(rng.integers(B)), int(rng.integers(Hkv))))
    return sorted(picks)


def _check(got, q, cache, units, lens, S, T, W, kb, vb, sk, sv, G, label):
    worst = 0.0
    for b, j in units:
        L = S if lens is None else int(np.clip(lens[b], 0, S))
        ref = _oracle_unit(q, cache, b, j, G, L, T, W, kb, vb, sk, sv)
        err = float(np.abs(got[b, :, j * G:(j + 1) * G] - ref).max())
        worst = max(worst, err)
        assert err <= ATTN_ATOL, f"{label}: unit ({b}, {j}) L={L} max-abs {err:.3g}"
    say(label, "worst", f"{worst:.3g}", "max |out|", f"{np.abs(got).max():.3g}")


# d, k_bits, v_bits, B, Hkv, G, S, T, window
CASES = [
    (128, 4, 4, 6, 2, 4, 900, 4, 0),      # speculative verification, G 4: one tile of 16 rows
    (128, 4, 4, 6, 2, 6, 700, 3, 0),      # G 6: two token tiles, the second one partial
    (128, 4, 4, 4, 2, 1, 800, 16, 0),     # G 1, 16 query tokens in one tile
    (128, 4, 4, 4, 2, 1, 1000, 13, 200),  # window
    (128, 4, 4, 5, 2, 4, 1200, 40, 0),    # 40 query tokens: ten token tiles
    (128, 4, 4, 8, 2, 4, 1500, 1, 100),   # sliding-window decode
    (128, 4, 4, 4, 2, 4, 300, 1, 1),      # window of one position
    (128, 4, 8, 6, 2, 2, 900, 5, 64),
    (256, 8, 4, 6, 2, 4, 700, 2, 0),
    (256, 4, 4, 5, 1, 8, 600, 3, 130),
    (128, 8, 4, 6, 2, 12, 500, 2, 0),     # G 12: rows 12 x 1 token per tile
]


@pytest.mark.parametrize("d,kb,vb,B,Hkv,G,S,T,W", CASES)
def test_attn_matches_oracle(d, kb, vb, B, Hkv, G, S, T, W):
    rng = np.random.default_rng(d + kb * 7 + vb + B + G * 3 + S + T * 11 + W)
    lay = kvq.make_layout(B, Hkv, Hkv * G, d, S, k_bits=kb, v_bits=vb)
    opts = kvq.make_attn_opts(T, W)
    pl = kvq.kvq_attn_launch_plan(lay, opts, S)
    say("attn", (d, kb, vb, B, Hkv, G, S, T, W), "tiles", pl.head_tile, pl.query_tile, pl.query_tiles, "chunks",
        pl.n_chunks, "sb/wave", pl.superblocks_per_wave)
    assert pl.head_tile * pl.query_tile <= (16 if d == 128 else 8)
    cache = _cache(rng, B, Hkv, S, d, kb, vb)
    q = synth.to_fp16(rng.standard_normal((B, T, Hkv * G, d)))
    sk, sv = synth.random_signs(int(rng.integers(1 << 20)), d), synth.random_signs(int(rng.integers(1 << 20)), d)
    lens = _lengths(rng, B, S, T)
    got = _run_attn(lay, opts, q, cache[:4], S, lens, sk, sv, cache[4], cache[5])
    assert np.isfinite(got).all()
    _check(got, q, cache, _units(rng, B, Hkv, 12), lens, S, T, W, kb, vb, sk, sv, G, f"attn T{T} W{W} G{G} d{d}")


@pytest.mark.parametrize("d,kb,G", [(128, 4, 4), (128, 4, 1), (256, 8, 4)])
def test_single_query_without_window_is_the_decode(d, kb, G):
    """n_query 1 and no window: the same plan and kernel as kvq_decode_attn, bit for bit."""
    rng = np.random.default_rng(5 + d + G)
    B, Hkv, S = 3, 2, 1100
    lay = kvq.make_layout(B, Hkv, Hkv * G, d, S, k_bits=kb, v_bits=4)
    cache = _cache(rng, B, Hkv, S, d, kb, 4)
    q = synth.to_fp16(rng.standard_normal((B, 1, Hkv * G, d)))
    sk, sv = synth.random_signs(1, d), synth.random_signs(2, d)
    lens = np.array([S, 517, 1])
    say("attn vs decode", d, kb, G)
    got = _run_attn(lay, kvq.make_attn_opts(1, 0), q, cache[:4], S, lens, sk, sv, cache[4], cache[5])
    ref = gpu_decode_planes(lay, q[:, 0], *cache[:4], S, lens, sk, sv, cache[4], cache[5], Hkv * d)
    assert np.array_equal(got[:, 0], ref)


def _ring_planes(logical, C, lens):
    """Ring layout of logical rows [B, Hkv, L_max, w]: slot s of row b holds the latest position
    t < lens[b] with t % C == s (older positions were overwritten)."""
    B, Hkv, Lmax, w = logical.shape
    ring = np.zeros((B, Hkv, C, w), logical.dtype)
    for b in range(B):
        L = int(lens[b])
        for t in range(max(0, L - C), L):
            ring[b, :, t % C] = logical[b, :, t]
    return ring


@pytest.mark.parametrize("d,G,T,W,C,page", [(128, 4, 1, 512, 640, 0), (128, 4, 4, 300, 512, 0),
                                            (128, 1, 8, 200, 256, 0), (256, 4, 2, 333, 448, 0),
                                            (128, 4, 3, 400, 512, 128), (128, 2, 1, 640, 640, 64)])
def test_ring_buffer_wraps(d, G, T, W, C, page):
    """Sequences several times longer than the ring's capacity C: the planes hold only the latest C
    positions of every row, at slot t % C (or in pages through the table, page = page size); the
    window reaches back across the wrap point."""
    rng = np.random.default_rng(d + G + T + W + C + page)
    B, Hkv = 4, 2
    kb = 8 if d == 256 else 4
    Lmax = 3 * C + 101
    lens = np.array([Lmax, 2 * C + 5, C - 7, T + W + 64])
    logical = _cache(rng, B, Hkv, Lmax, d, kb, 4)
    lay = kvq.make_layout(B, Hkv, Hkv * G, d, C, k_bits=kb, v_bits=4)
    opts = kvq.make_attn_opts(T, W, ring=True)
    ring = tuple(_ring_planes(a, C, lens) for a in logical[:4])
    q = synth.to_fp16(rng.standard_normal((B, T, Hkv * G, d)))
    sk, sv = synth.random_signs(3, d), synth.random_signs(4, d)
    pg = None
    if page:
        pps = C // page
        n_pages = B * pps + 3
        perm = rng.permutation(n_pages)[: B * pps]
        table = perm.reshape(B, pps).astype(np.int32)

        def paged(a):
            w = a.shape[-1]
            out = np.zeros((n_pages, Hkv, page, w), a.dtype)
            out[perm] = a.reshape(B, Hkv, pps, page, w).transpose(0, 2, 1, 3, 4).reshape(B * pps, Hkv, page, w)
            return out

        ring = tuple(paged(a) for a in ring)
        pg = (table, page, n_pages)
    pl = kvq.kvq_attn_launch_plan(lay, opts, Lmax, paged=bool(page))
    say("ring", (d, G, T, W, C, page), "chunks", pl.n_chunks, "sb/wave", pl.superblocks_per_wave)
    got = _run_attn(lay, opts, q, ring, Lmax, lens, sk, sv, logical[4], logical[5], page=pg)
    _check(got, q, logical, [(b, j) for b in range(B) for j in range(Hkv)], lens, Lmax, T, W, kb, 4, sk, sv, G,
           f"ring C{C} W{W} T{T} page{page}")


@pytest.mark.parametrize("T,W", [(4, 0), (6, 700)])
def test_paged_multi_token(T, W):
    rng = np.random.default_rng(100 + T + W)
    B, Hkv, G, S, d, ps = 4, 2, 4, 1000, 128, 128
    pps = -(-S // ps)
    cache = _cache(rng, B, Hkv, S, d, 4, 4)
    lay = kvq.make_layout(B, Hkv, Hkv * G, d, pps * ps)
    opts = kvq.make_attn_opts(T, W)
    n_pages = B * pps
    perm = rng.permutation(n_pages)
    table = perm.reshape(B, pps).astype(np.int32)

    def paged(a):
        w = a.shape[-1]
        nat = np.concatenate([a, np.zeros((B, Hkv, pps * ps - S, w), a.dtype)], 2)
        out = np.empty((n_pages, Hkv, ps, w), a.dtype)
        out[perm] = nat.reshape(B, Hkv, pps, ps, w).transpose(0, 2, 1, 3, 4).reshape(n_pages, Hkv, ps, w)
        return out

    q = synth.to_fp16(rng.standard_normal((B, T, Hkv * G, d)))
    sk, sv = synth.random_signs(5, d), synth.random_signs(6, d)
    lens = np.array([S, 333, T, 64])
    say("paged multi-token", T, W)
    got = _run_attn(lay, opts, q, tuple(paged(a) for a in cache[:4]), S, lens, sk, sv, cache[4], cache[5],
                    page=(table, ps, n_pages))
    _check(got, q, cache, [(b, j) for b in range(B) for j in range(Hkv)], lens, S, T, W, 4, 4, sk, sv, G,
           f"paged T{T} W{W}")


@pytest.mark.parametrize("T,W", [(4, 0), (4, 2000), (1, 1500)])
def test_attn_deep(T, W):
    """Many units and long rows: several superblocks per wave with windows and causal rows."""
    rng = np.random.default_rng(7 + T + W)
    B, Hkv, G, S, d = 64, 8, 4, 6000, 128
    lay = kvq.make_layout(B, Hkv, Hkv * G, d, S)
    opts = kvq.make_attn_opts(T, W)
    pl = kvq.kvq_attn_launch_plan(lay, opts, S)
    say("attn deep", T, W, "chunks", pl.n_chunks, "sb/wave", pl.superblocks_per_wave, "work-groups", pl.work_groups)
    assert pl.superblocks_per_wave >= 4
    cache = _cache(rng, B, Hkv, S, d, 4, 4)
    q = synth.to_fp16(rng.standard_normal((B, T, Hkv * G, d)))
    sk, sv = synth.random_signs(8, d), synth.random_signs(9, d)
    lens = _lengths(rng, B, S, T)
    got = _run_attn(lay, opts, q, cache[:4], S, lens, sk, sv, cache[4], cache[5])
    _check(got, q, cache, _units(rng, B, Hkv, 14), lens, S, T, W, 4, 4, sk, sv, G, f"attn deep T{T} W{W}")
