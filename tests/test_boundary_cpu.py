"""The C-ABI library loads, exports every declared symbol, and validates arguments on the host.

No GPU is needed: every call here fails validation, which happens before any HIP call, so the
fake device pointers below are never dereferenced.
"""
import ctypes
import os
import re
import subprocess
import sys
import threading

import pytest

from kv_cache_quantization_srft_amd import kvq
from oracle import kvq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

P = ctypes.c_void_p
GOOD = P(1 << 20)      # aligned fake device pointer (never dereferenced)
MIS = P((1 << 20) + 4)  # 4-byte aligned, not 16-byte aligned
NULL = P(0)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")
    return kvq.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(kvq.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(kvq_\w+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_version_and_status_strings(L):
    assert kvq.kvq_version() >= 100
    for code, name in kvq.STATUS_NAMES.items():
        assert L.kvq_status_string(code).decode() == name


def layout(**kw):
    base = dict(batch=2, kv_heads=2, q_heads=12, head_dim=128, capacity=64, k_bits=4, v_bits=4)
    base.update(kw)
    return kvq.make_layout(**base)


def test_footprint_matches_oracle(L):
    for d, kb, vb in ((128, 4, 4), (256, 8, 4)):
        lay = layout(head_dim=d, k_bits=kb, v_bits=vb, capacity=4096, batch=3)
        total = kvq.kvq_codes_bytes(lay, kb) + kvq.kvq_codes_bytes(lay, vb) + 2 * kvq.kvq_scales_bytes(lay)
        assert total == O.quantized_kv_bytes(1, 2, d, 4096, kb, vb, batch=3)
    assert kvq.kvq_codes_bytes(layout(head_dim=96), 4) == 0
    assert kvq.kvq_codes_bytes(layout(), 3) == 0


def test_workspace_bytes_monotonic(L):
    lay = layout()
    sizes = [kvq.kvq_decode_attn_workspace_bytes(lay, s) for s in (1, 64, 4096, 65536)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    assert kvq.kvq_decode_attn_workspace_bytes(layout(q_heads=5), 64) == 0


def quantize(L, lay, bits=4, x=GOOD, pos=0, n_tok=4, sign=GOOD, sbs=0, lam=NULL, lbs=0, codes=GOOD, scales=GOOD):
    return L.kvq_quantize(ctypes.byref(lay), bits, x, pos, n_tok, sign, sbs, lam, lbs, codes, scales, NULL)


def msg(L):
    return L.kvq_last_error_message().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(lay=dict(head_dim=96)), 2, "head_dim"),
    (dict(lay=dict(head_dim=64)), 2, "head_dim"),
    (dict(lay=dict(batch=0)), 1, "batch"),
    (dict(bits=3), 2, "bits"),
    (dict(pos=62, n_tok=4), 1, "token range"),
    (dict(pos=-1), 1, "token range"),
    (dict(n_tok=0), 1, "token range"),
    (dict(x=NULL), 1, "x is NULL"),
    (dict(x=MIS), 3, "x is not 16-byte"),
    (dict(codes=MIS), 3, "codes"),
    (dict(scales=NULL), 1, "scales"),
    (dict(sign=P((1 << 20) + 2)), 3, "sign"),
    (dict(sbs=-1), 1, "stride"),
])
def test_quantize_validation(L, kw, status, needle):
    lay = layout(**kw.pop("lay", {}))
    st = quantize(L, lay, **kw)
    assert st == status
    assert needle in msg(L)


def test_group_size_unsupported(L):
    lay = layout()
    lay.group_size = 32
    assert quantize(L, lay) == 2 and "group_size" in msg(L)


@pytest.mark.parametrize("d", [128, 256])
def test_per_token_group_is_a_write_path_mode(L, d):
    """group_size == head_dim (one scale per vector): accepted by the write path, dequantize and
    the sizing calls (one fp16 scale per token), rejected by both quantized decode calls."""
    lay = layout(head_dim=d, group_size=d)
    assert kvq.kvq_scales_bytes(lay) == 2 * 2 * 64 * 2
    assert kvq.kvq_scales_bytes(layout(head_dim=d)) == 2 * 2 * 64 * (d // 16) * 2
    assert quantize(L, lay, x=MIS) == 3  # validation passes the group check, stops at x
    st = L.kvq_dequantize(ctypes.byref(lay), 4, GOOD, GOOD, 0, 1, GOOD, 0, NULL, 0, MIS, NULL)
    assert st == 3 and "out" in msg(L)
    assert decode(L, lay) == 2 and "group_size" in msg(L)
    st = L.kvq_decode_attn_append(ctypes.byref(lay), GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 16, NULL, GOOD,
                                  GOOD, 0, NULL, NULL, 0, ctypes.c_float(0), GOOD, 1 << 30, GOOD, NULL)
    assert st == 2 and "group_size" in msg(L)


def test_transform_field(L):
    lay = layout(transform="srht")
    assert lay.transform == 1 and layout().transform == 0
    lay.transform = 2
    assert quantize(L, lay) == 2 and "transform" in msg(L)
    assert decode(L, lay) == 2 and "transform" in msg(L)


def test_dequantize_and_calibrate_validation(L):
    lay = layout()
    st = L.kvq_dequantize(ctypes.byref(lay), 8, GOOD, GOOD, 0, 65, GOOD, 0, NULL, 0, GOOD, NULL)
    assert st == 1 and "token range" in msg(L)
    st = L.kvq_dequantize(ctypes.byref(lay), 4, GOOD, GOOD, 0, 1, GOOD, 0, NULL, 0, MIS, NULL)
    assert st == 3 and "out" in msg(L)
    st = L.kvq_calibrate_lambda(ctypes.byref(lay), GOOD, 16, 17, GOOD, 0, GOOD, NULL)
    assert st == 1 and "n_cal" in msg(L)
    st = L.kvq_calibrate_lambda(ctypes.byref(lay), GOOD, 16, 0, GOOD, 0, GOOD, NULL)
    assert st == 1


def decode(L, lay, q=GOOD, seq_len=16, seq_lens=NULL, sm=0.0, ws=GOOD, ws_bytes=1 << 30, out=GOOD, kc=GOOD,
           lam=NULL):
    return L.kvq_decode_attn(ctypes.byref(lay), q, kc, GOOD, GOOD, GOOD, seq_len, seq_lens, GOOD, GOOD, 0, lam,
                             lam, 0, ctypes.c_float(sm), ws, ws_bytes, out, NULL)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(lay=dict(q_heads=5)), 1, "multiple of kv_heads"),
    (dict(lay=dict(q_heads=2 * 65)), 2, "GQA"),
    (dict(lay=dict(v_bits=3)), 2, "v_bits"),
    (dict(lay=dict(k_bits=2)), 2, "k_bits"),
    (dict(seq_len=0), 1, "seq_len"),
    (dict(seq_len=65), 1, "seq_len"),
    (dict(q=MIS), 3, "q is not"),
    (dict(out=NULL), 1, "out"),
    (dict(ws=P((1 << 20) + 16)), 3, "workspace"),
    (dict(ws_bytes=16), 4, "workspace has 16 bytes"),
    (dict(sm=float("nan")), 1, "sm_scale"),
    (dict(kc=MIS), 3, "k_codes"),
    (dict(seq_lens=P((1 << 20) + 2)), 3, "seq_lens"),
    (dict(lay=dict(batch=16385)), 2, "exceeds 16384"),
    (dict(lay=dict(batch=2049, kv_heads=2, q_heads=16 * 2 * 4)), 2, "exceeds 16384"),
])
def test_decode_validation(L, kw, status, needle):
    lay = layout(**kw.pop("lay", {}))
    assert decode(L, lay, **kw) == status
    assert needle in msg(L)


def test_fp16_decode_validation(L):
    lay = layout()
    st = L.kvq_decode_attn_fp16(ctypes.byref(lay), GOOD, MIS, GOOD, 16, NULL, ctypes.c_float(0), GOOD, 1 << 30,
                                GOOD, NULL)
    assert st == 3 and "k is not" in msg(L)
    st = L.kvq_decode_attn_fp16(ctypes.byref(lay), GOOD, GOOD, GOOD, 65, NULL, ctypes.c_float(0), GOOD, 1 << 30,
                                GOOD, NULL)
    assert st == 1


def test_error_message_is_thread_local(L):
    lay = layout(head_dim=96)
    assert quantize(L, lay) == 2
    main_msg = msg(L)
    seen = {}

    def worker():
        seen["before"] = L.kvq_last_error_message().decode()
        quantize(L, layout(), bits=3)
        seen["after"] = L.kvq_last_error_message().decode()

    t = threading.Thread(target=worker)
    t.start()
    t.join()
    assert seen["before"] == ""
    assert "bits" in seen["after"]
    assert msg(L) == main_msg


def test_binding_requires_device_tensors(L):
    torch = pytest.importorskip("torch")
    lay = layout()
    x = torch.zeros(2 * 2 * 4 * 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        kvq.kvq_quantize(lay, 4, x, 0, 4, x, 0, None, 0, x, x, stream=0)


def append(L, lay, q=GOOD, k_new=GOOD, v_new=GOOD, seq_len=16, ws_bytes=1 << 30, kc=GOOD):
    return L.kvq_decode_attn_append(ctypes.byref(lay), q, k_new, v_new, kc, GOOD, GOOD, GOOD, seq_len, NULL, GOOD,
                                    GOOD, 0, NULL, NULL, 0, ctypes.c_float(0.0), GOOD, ws_bytes, GOOD, NULL)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(k_new=NULL), 1, "k_new is NULL"),
    (dict(v_new=MIS), 3, "v_new is not"),
    (dict(kc=MIS), 3, "k_codes"),
    (dict(seq_len=65), 1, "seq_len"),
    (dict(lay=dict(v_bits=3)), 2, "v_bits"),
    (dict(ws_bytes=16), 4, "workspace has 16 bytes"),
])
def test_append_validation(L, kw, status, needle):
    lay = layout(**kw.pop("lay", {}))
    assert append(L, lay, **kw) == status
    assert needle in msg(L)


def test_append_head_tile_limit(L):
    # G = 16 at d = 128: kvq_decode_attn uses one head tile of 16, the appending call two of 8
    # (rows 14 and 15 of its query rotation carry the new K and V), so its unit count doubles
    # (both calls fail validation: the first only at the workspace size, after the unit check)
    lay = layout(batch=8193, kv_heads=1, q_heads=16)
    assert decode(L, lay, ws_bytes=16) == 4 and "workspace has 16 bytes" in msg(L)
    assert append(L, lay, ws_bytes=16) == 2 and "exceeds 16384" in msg(L)


def paged(L, lay, q=GOOD, kn=NULL, vn=NULL, table=GOOD, pps=4, psz=16, npages=9, seq_len=16, ws_bytes=1 << 30):
    return L.kvq_decode_attn_paged(ctypes.byref(lay), q, kn, vn, GOOD, GOOD, GOOD, GOOD, table, pps, psz, npages,
                                   seq_len, NULL, GOOD, GOOD, 0, NULL, NULL, 0, ctypes.c_float(0), GOOD, ws_bytes,
                                   GOOD, NULL)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(psz=16), 2, "page_size"),
    (dict(psz=96, pps=2, lay=dict(capacity=192)), 2, "page_size"),
    (dict(psz=64, pps=0), 1, "pages_per_seq"),
    (dict(psz=64, pps=1, npages=0), 1, "num_pages"),
    (dict(psz=64, pps=2), 1, "capacity"),
    (dict(psz=64, pps=1, table=NULL), 1, "page_table"),
    (dict(psz=64, pps=1, table=P((1 << 20) + 2)), 3, "page_table"),
    (dict(psz=64, pps=1, kn=GOOD), 1, "v_new"),
    (dict(psz=64, pps=1, seq_len=65), 1, "seq_len"),
    (dict(psz=64, pps=1, lay=dict(group_size=128)), 2, "group_size"),
])
def test_paged_decode_validation(L, kw, status, needle):
    """capacity = 64 unless set: one 64-token page per sequence is the valid base case."""
    lay = layout(**kw.pop("lay", {}))
    assert paged(L, lay, **kw) == status
    assert needle in msg(L)


def test_paged_workspace_covers_long_chunks(L):
    """A paged call caps a work-group's chunk at 64 superblocks per wave (16384 tokens), so with
    many units and long sequences it needs more chunk partials than a contiguous call; the
    workspace query covers both."""
    lay = layout(batch=512, kv_heads=1, q_heads=1, capacity=65536)
    need = kvq.kvq_decode_attn_workspace_bytes(lay, 65536)
    assert need > 0
    assert paged(L, lay, pps=1024, psz=64, npages=512 * 1024, seq_len=65536, ws_bytes=need - 1) == 4


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; --gpus N > 1 prints a one-line JSON error and exits 2 before
    touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = r.stdout.strip().splitlines()[-1]
    assert "one GPU" in line and line.startswith("{")


def test_launch_plan_shapes(L):
    """kvq_launch_plan describes the split the calls launch with (host only)."""
    # serving shard folded into the batch: 2048 units cover the GPU, one chunk of 32768 tokens each
    p = kvq.kvq_launch_plan(kvq.make_layout(256, 8, 32, 128, 32768), "decode", 32768)
    assert (p.work_groups, p.head_tile, p.head_tiles, p.chunk, p.n_chunks) == (2048, 4, 1, 32768, 1)
    assert (p.wave_tokens, p.superblocks_per_wave) == (64, 128)
    # few units: the sequence is split into chunks, every chunk a multiple of 4 waves x 64 tokens
    p = kvq.kvq_launch_plan(kvq.make_layout(1, 2, 12, 128, 4096), "decode", 4096)
    assert p.head_tile == 6 and p.chunk % 256 == 0 and p.n_chunks * p.chunk >= 4096 and p.n_chunks > 1
    # G above the largest head tile: several head tiles per kv head
    p = kvq.kvq_launch_plan(kvq.make_layout(2, 2, 64, 128, 1000), "decode", 1000)
    assert (p.head_tile, p.head_tiles) == (16, 2)
    p = kvq.kvq_launch_plan(kvq.make_layout(2, 2, 64, 128, 1000), "decode_append", 1000)
    assert p.head_tile * p.head_tiles == 32 and p.head_tile <= 14
    # fp16 comparator: 32-token wave superblocks
    p = kvq.kvq_launch_plan(kvq.make_layout(64, 8, 8, 128, 1000), "decode_fp16", 1000)
    assert p.wave_tokens == 32 and p.superblocks_per_wave == p.chunk // 128
    # write path: 16-vector blocks in contiguous ranges over at most 3 x 256 work-groups (d 128)
    p = kvq.kvq_launch_plan(kvq.make_layout(3, 9, 9, 128, 5000), "quantize", 5000)
    assert (p.work_groups, p.blocks) == (768, (3 * 9 * 5000 + 15) // 16)
    assert p.blocks_per_work_group == -(-p.blocks // 768)
    p = kvq.kvq_launch_plan(kvq.make_layout(1, 1, 1, 256, 40), "quantize", 40)
    assert (p.work_groups, p.blocks, p.blocks_per_work_group) == (3, 3, 1)


def test_launch_plan_errors(L):
    out = kvq.kvq_plan()
    lay = kvq.make_layout(2, 2, 12, 128, 64)
    assert L.kvq_launch_plan(ctypes.byref(lay), 1, 65, ctypes.byref(out)) == 1   # seq_len > capacity
    assert L.kvq_launch_plan(ctypes.byref(lay), 0, 0, ctypes.byref(out)) == 1    # n_tok < 1
    assert L.kvq_launch_plan(ctypes.byref(lay), 9, 8, ctypes.byref(out)) == 1    # unknown call
    assert L.kvq_launch_plan(ctypes.byref(lay), 1, 8, None) == 1
    bad = kvq.make_layout(2, 2, 5, 128, 64)
    assert L.kvq_launch_plan(ctypes.byref(bad), 1, 8, ctypes.byref(out)) == 1    # q_heads % kv_heads
    assert L.kvq_launch_plan(ctypes.byref(kvq.make_layout(2, 2, 2, 96, 64)), 0, 8, ctypes.byref(out)) == 2


def attn(L, lay, opts, seq_len=64, table=NULL, pps=0, ps=0, npg=0, ws=GOOD, ws_bytes=1 << 30, q=GOOD):
    return L.kvq_attn(ctypes.byref(lay), opts if opts is None else ctypes.byref(opts), q, GOOD, GOOD, GOOD, GOOD, table,
                      pps, ps, npg, seq_len, NULL, GOOD, GOOD, 0, NULL, NULL, 0, 0.0, ws, ws_bytes, GOOD, NULL)


def test_attn_validation(L):
    """kvq_attn rejects bad options on the host (status codes from kvq.h), before any HIP call."""
    lay = layout(capacity=640)
    ok_opts = kvq.make_attn_opts(4, 0)
    assert attn(L, lay, None) == 1                                          # opts NULL
    assert attn(L, lay, kvq.make_attn_opts(0, 0)) == 1                      # n_query < 1
    assert attn(L, lay, kvq.make_attn_opts(2, -1)) == 1                     # window < 0
    assert attn(L, lay, ok_opts, seq_len=641) == 1                          # beyond capacity, no ring
    assert attn(L, lay, kvq.make_attn_opts(1, 0, ring=True), seq_len=5000) == 1   # ring needs a window
    assert attn(L, lay, kvq.make_attn_opts(4, 638, ring=True), seq_len=5000) == 1  # W + T - 1 > capacity
    assert attn(L, layout(capacity=600), kvq.make_attn_opts(1, 100, ring=True), seq_len=5000) == 2  # capacity % 64
    assert attn(L, lay, ok_opts, table=GOOD, pps=10, ps=100, npg=8) == 2     # page size
    assert attn(L, lay, ok_opts, table=GOOD, pps=4, ps=128, npg=8) == 1      # capacity != pps x page size
    assert attn(L, lay, ok_opts, q=MIS) == 3
    assert attn(L, lay, ok_opts, ws_bytes=1024) == 4
    assert b"workspace" in L.kvq_last_error_message()
    assert attn(L, layout(capacity=640, group_size=128), ok_opts) == 2       # decode reads groups of 16


def test_attn_sizing_and_plan(L):
    lay = kvq.make_layout(8, 2, 8, 128, 65536)
    o = kvq.make_attn_opts(4, 0)
    sizes = [kvq.kvq_attn_workspace_bytes(lay, o, s) for s in (64, 4096, 65536)]
    assert all(s > 0 for s in sizes) and sizes == sorted(sizes)
    # a window bounds the tokens a unit attends, and so the chunks and the workspace
    ow = kvq.make_attn_opts(4, 512)
    assert kvq.kvq_attn_workspace_bytes(lay, ow, 65536) == kvq.kvq_attn_workspace_bytes(lay, ow, 8192)
    assert kvq.kvq_attn_workspace_bytes(lay, kvq.make_attn_opts(0, 0), 64) == 0
    p = kvq.kvq_attn_launch_plan(lay, o, 4096)
    assert (p.head_tile, p.query_tile, p.query_tiles) == (4, 4, 1)            # G 4 x 4 tokens = 16 rows
    p = kvq.kvq_attn_launch_plan(kvq.make_layout(2, 2, 12, 128, 4096), kvq.make_attn_opts(3, 0), 4096)
    assert (p.head_tile, p.query_tile, p.query_tiles) == (6, 2, 2)
    p = kvq.kvq_attn_launch_plan(kvq.make_layout(2, 2, 8, 256, 4096), kvq.make_attn_opts(5, 0), 4096)
    assert p.head_tile * p.query_tile <= 8
    p1 = kvq.kvq_attn_launch_plan(lay, kvq.make_attn_opts(1, 0), 4096)
    p2 = kvq.kvq_launch_plan(lay, "decode", 4096)
    assert (p1.work_groups, p1.chunk, p1.n_chunks, p1.head_tile) == (p2.work_groups, p2.chunk, p2.n_chunks, p2.head_tile)
