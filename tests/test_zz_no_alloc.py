"""kvq_decode_attn_noalloc (the decode with its workspace in the library's built-in device array)
against kvq_decode_attn with a caller workspace, through the C ABI: two calls in a row, the second
smaller, each bit-identical to the workspace call (same kernels, same plan); the first call has
many chunks per unit, so the completion counters and chunk partials of the built-in scratch are
used and must be left ready for the second.  A call needing more than the built-in scratch is
rejected on the host."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_srft_amd import kvq, synth

from gpu_parity import dev, plan, say

pytestmark = pytest.mark.gpu


def _case(rng, B, Hkv, G, S, d, kb):
    lay = kvq.make_layout(B, Hkv, Hkv * G, d, S, k_bits=kb, v_bits=4)
    kc = synth.random_code_bytes(rng, (B, Hkv, S, d * kb // 8), kb)
    vc = synth.random_code_bytes(rng, (B, Hkv, S, d // 2), 4)
    ks = synth.random_scales(rng, (B, Hkv, S, d // 16), 0.15, 0.8) if kb == 4 else \
        synth.random_scales(rng, (B, Hkv, S, d // 16), 0.01, 0.06)
    vs = synth.random_scales(rng, (B, Hkv, S, d // 16), 0.15, 0.8)
    lk = synth.random_lambda(rng, (B, Hkv, d), 0.5, 2.0)
    lv = synth.random_lambda(rng, (B, Hkv, d), 0.5, 2.0)
    q = synth.to_fp16(rng.standard_normal((B, Hkv * G, d)))
    lens = rng.integers(0, S + 1, size=B).astype(np.int32)
    lens[0] = S
    s = synth.random_signs(int(rng.integers(1 << 20)), d)
    args = [dev(q), dev(kc), dev(ks.view(np.int16)), dev(vc), dev(vs.view(np.int16)), S, dev(lens), dev(s), dev(s), 0,
            dev(lk), dev(lv), Hkv * d, 0.0]
    return lay, args


def test_noalloc_matches_workspace_call():
    rng = np.random.default_rng(2027)
    cases = [(4, 2, 6, 3000, 128, 4), (2, 2, 4, 700, 256, 8)]  # the second call is smaller
    for i, (B, Hkv, G, S, d, kb) in enumerate(cases):
        lay, args = _case(rng, B, Hkv, G, S, d, kb)
        pl = plan(lay, "decode", S)
        say("noalloc call", i, (B, Hkv, G, S, d, kb), pl)
        if i == 0:
            assert pl["n_chunks"] >= 8, pl
        ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay, S), dtype=torch.uint8, device="cuda")
        ref = torch.full((B, Hkv * G, d), float("nan"), dtype=torch.float32, device="cuda")
        got = torch.full_like(ref, float("nan"))
        kvq.kvq_decode_attn(lay, *args, ws, ref)
        kvq.kvq_decode_attn_noalloc(lay, *args, got)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref), f"call {i}: max diff {(got - ref).abs().max().item():.3g}"
    # the same large call again after the small one: the scratch was left ready
    lay, args = _case(np.random.default_rng(2027), *cases[0])
    ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay, cases[0][3]), dtype=torch.uint8, device="cuda")
    ref = torch.empty((cases[0][0], cases[0][1] * cases[0][2], cases[0][4]), dtype=torch.float32, device="cuda")
    got = torch.empty_like(ref)
    kvq.kvq_decode_attn(lay, *args, ws, ref)
    kvq.kvq_decode_attn_noalloc(lay, *args, got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_noalloc_rejects_calls_beyond_the_scratch():
    # 16384 units of 16 heads with many chunks need far more than 32 MiB of partials
    lay = kvq.make_layout(1024, 16, 256, 128, 65536)
    need = kvq.kvq_decode_attn_workspace_bytes(lay, 65536)
    assert need > 32 << 20
    t = torch.zeros(16, dtype=torch.uint8, device="cuda")
    f = torch.zeros(4, dtype=torch.float32, device="cuda")
    st = kvq.lib().kvq_decode_attn_noalloc(kvq.ctypes.byref(lay), t.data_ptr(), t.data_ptr(), t.data_ptr(),
                                           t.data_ptr(), t.data_ptr(), 65536, None, f.data_ptr(), f.data_ptr(), 0,
                                           None, None, 0, 0.0, f.data_ptr(), None)
    assert st == 4, st  # KVQ_ERR_WORKSPACE_TOO_SMALL, before any HIP call
    assert b"built-in scratch" in kvq.lib().kvq_last_error_message()
