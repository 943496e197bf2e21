"""GPU parity of the write path (kvq_quantize) on the code paths of bulk calls: every work-group
walks a contiguous range of many 16-vector blocks in halves (staged blocks 1..3 of a shared-sign
half, the next half's loads in flight, the second register set), with rows of the batch ending
inside blocks and inside a work-group's range, so the cached lambda reciprocals are reused
across blocks and refreshed at row boundaries.

Each test asks the library for its launch plan and asserts the blocks per work-group it claims
to reach; every vector is compared with the oracle under the write path's bar (packing
bit-exact, codes within the rounding-tie rule, scales bit-equal or one fp16 ulp apart)."""
import numpy as np
import pytest

from kv_cache_quantization_srft_amd import kvq, synth
from oracle import kvq_oracle as O

from gpu_parity import check_quantize, gpu_quantize, plan, say

pytestmark = pytest.mark.gpu


def _data(rng, B, H, n, d):
    """Student-t (nu = 4) values with a few x20 outlier channels per row and a log-uniform
    per-channel spread, the statistics of the workloads' keys."""
    std = np.exp(rng.uniform(np.log(0.5), np.log(4.0), size=(B, H, 1, d)))
    out = np.where(rng.random((B, H, 1, d)) < 0.03, 20.0, 1.0)
    return synth.to_fp16(rng.standard_t(4, size=(B, H, n, d)) * std * out)


# d, bits, B, H, n, lambda, per-row signs, group, pos, extra capacity, min blocks per work-group
BULK = [
    (128, 4, 3, 9, 5000, True, False, 16, 0, 0, 10),
    (128, 4, 5, 4, 7000, False, True, 16, 37, 100, 10),
    (128, 8, 3, 9, 5000, True, True, 16, 0, 0, 10),
    (128, 4, 4, 6, 5001, True, False, 128, 11, 5, 10),
    (256, 4, 2, 3, 3000, True, False, 16, 0, 0, 4),
    (256, 8, 2, 3, 3000, False, True, 16, 5, 40, 4),
    (256, 8, 3, 2, 2999, True, False, 256, 0, 0, 4),
    # rows of 3 tokens: every block spans several rows, several blocks per work-group
    (128, 4, 128, 80, 3, True, False, 16, 2, 1, 2),
    (256, 8, 64, 50, 3, False, True, 16, 0, 0, 2),
]


@pytest.mark.parametrize("d,bits,B,H,n,lam,per_row_sign,group,pos,extra,min_bpw", BULK)
def test_quantize_bulk(d, bits, B, H, n, lam, per_row_sign, group, pos, extra, min_bpw):
    rng = np.random.default_rng(d + bits + B * H + n + group)
    cap = pos + n + extra
    lay = kvq.make_layout(B, H, H, d, cap, k_bits=bits, group_size=group)
    pl = plan(lay, "quantize", n)
    say("bulk quantize", (d, bits, B, H, n, lam, per_row_sign, group, pos), pl)
    assert pl["blocks_per_work_group"] >= min_bpw, pl
    x = _data(rng, B, H, n, d)
    s = np.stack([synth.random_signs(100 + b, d) for b in range(B)]) if per_row_sign else synth.random_signs(7, d)
    lam_v = synth.random_lambda(rng, (B, H, d), 0.5, 8.0) if lam else None
    cb, sc, _ = gpu_quantize(x, s, lam_v, bits, capacity=cap, pos=pos, sign_bs=d if per_row_sign else 0,
                             lambda_bs=H * d if lam else 0, group=group)
    lam_b = 1.0 if lam_v is None else lam_v[:, :, None, :].astype(np.float64)
    u = O.rotated_scaled(x, s[:, None, None, :] if per_row_sign else s, lam_b)
    n_diff, n_ulp = check_quantize(cb[:, :, pos:pos + n], sc[:, :, pos:pos + n], u, bits,
                                   f"bulk d{d} b{bits} g{group}", group=group)
    say("bulk quantize: tie flips", n_diff, "scale ulps", n_ulp)
    # slots outside [pos, pos + n) keep the fill the planes were created with
    keep = np.ones(cap, bool)
    keep[pos:pos + n] = False
    assert np.all(cb[:, :, keep] == 0xAB)
    assert np.all(np.isnan(sc[:, :, keep].astype(np.float32)))
