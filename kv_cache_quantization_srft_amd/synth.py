"""Seeded synthetic K/V/query/sign generators for the five benchmark workloads.

This module holds no part of the quantization or attention arithmetic: it only draws
random numbers with the shapes and value statistics of each workload, so that the CPU
oracle and the GPU path can be fed identical inputs.

Every tensor is addressed by (workload id, layer, tensor id) and drawn from its own
NumPy PCG64 stream, so any single layer can be regenerated without producing the rest.
``torch_kv`` draws the same *distributions* on a torch device for the largest workloads;
it is seeded and deterministic but is not bit-identical to the NumPy streams.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

K_TENSOR, V_TENSOR, Q_TENSOR, SIGN_TENSOR, SIGN_V_TENSOR = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    """Shapes and value recipe of one workload (per layer: [batch, kv_heads, seq, head_dim])."""
    cid: int
    name: str
    layers: int
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    seq_len: int
    k_bits: int
    v_bits: int
    calibrate: bool            # per-channel lambda from the first `n_cal` tokens
    k_dist: str
    v_dist: str
    n_cal: int = 512
    seq_sweep: tuple = field(default_factory=tuple)

    @property
    def gqa(self) -> int:
        return self.q_heads // self.kv_heads


WORKLOADS = {
    1: Workload(1, "tiny-d128-s256", 1, 1, 1, 1, 128, 256, 4, 4, False,
                "normal_outlier2x15", "normal_outlier2x15"),
    2: Workload(2, "qwen2.5-1.5b-like-kv", 28, 1, 2, 12, 128, 4096, 4, 4, True,
                "t3_outlier4x20", "normal"),
    3: Workload(3, "gemma3-1b-like-kv-k8v4", 26, 1, 1, 4, 256, 4096, 8, 4, False,
                "normal_bern01x10", "normal_bern01x10", seq_sweep=(256, 512, 1024, 2048, 4096)),
    4: Workload(4, "l48-h16-d128-s16384", 48, 1, 16, 16, 128, 16384, 4, 4, True,
                "normal_loguniform_std", "normal_loguniform_std"),
    5: Workload(5, "serving-shard-l32-b8-h8-s32768", 32, 8, 8, 32, 128, 32768, 4, 4, False,
                "t4_outlier4x20", "t4_outlier4x20"),
}


def stream(cid: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cid, layer, tensor])))


def _draw(rng: np.random.Generator, dist: str, batch: int, heads: int, seq: int, d: int) -> np.ndarray:
    shape = (batch, heads, seq, d)
    if dist == "normal":
        return rng.standard_normal(shape)
    if dist == "normal_outlier2x15":
        x = rng.standard_normal(shape)
        return _outlier_channels(rng, x, 2, 15.0)
    if dist == "t3_outlier4x20":
        x = rng.standard_t(3.0, size=shape)
        return _outlier_channels(rng, x, 4, 20.0)
    if dist == "t4_outlier4x20":
        x = rng.standard_t(4.0, size=shape)
        return _outlier_channels(rng, x, 4, 20.0)
    if dist == "normal_bern01x10":
        x = rng.standard_normal(shape)
        mask = rng.random(shape) < 0.01
        return np.where(mask, 10.0 * x, x)
    if dist == "normal_loguniform_std":
        std = np.exp(rng.uniform(np.log(0.5), np.log(8.0), size=(batch, heads, 1, d)))
        return std * rng.standard_normal(shape)
    raise ValueError(f"unknown distribution {dist!r}")


def _outlier_channels(rng, x, count, factor):
    """Multiply `count` rng-chosen channels of every (sequence, head) by `factor`."""
    b, h, _, d = x.shape
    for i in range(b):
        for j in range(h):
            ch = rng.choice(d, size=count, replace=False)
            x[i, j, :, ch] *= factor
    return x


def to_fp16(x: np.ndarray) -> np.ndarray:
    return np.clip(x, -65504.0, 65504.0).astype(np.float16)


def kv(w: Workload, layer: int, tensor: int, seq_len: int | None = None) -> np.ndarray:
    """K (tensor=0) or V (tensor=1) of one layer, fp16 [batch, kv_heads, seq, head_dim]."""
    seq = w.seq_len if seq_len is None else seq_len
    dist = w.k_dist if tensor == K_TENSOR else w.v_dist
    return to_fp16(_draw(stream(w.cid, layer, tensor), dist, w.batch, w.kv_heads, seq, w.head_dim))


def query(w: Workload, layer: int) -> np.ndarray:
    """One decode query per sequence and head, fp16 [batch, q_heads, head_dim] ~ N(0, 1)."""
    return to_fp16(stream(w.cid, layer, Q_TENSOR).standard_normal((w.batch, w.q_heads, w.head_dim)))


def signs(w: Workload, tensor: int = SIGN_TENSOR) -> np.ndarray:
    """The fixed random +-1 vector of the workload (float32 [head_dim]); one per workload."""
    r = stream(w.cid, 0, tensor)
    return np.where(r.random(w.head_dim) < 0.5, -1.0, 1.0).astype(np.float32)


def random_signs(seed: int, d: int) -> np.ndarray:
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 9999])))
    return np.where(r.random(d) < 0.5, -1.0, 1.0).astype(np.float32)


def torch_kv(w: Workload, layer: int, tensor: int, device, seq_len: int | None = None):
    """Same distributions as `kv`, drawn with a seeded torch generator on `device` (fp16)."""
    import torch

    seq = w.seq_len if seq_len is None else seq_len
    dist = w.k_dist if tensor == K_TENSOR else w.v_dist
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * w.cid + 1009 * layer + tensor)
    shape = (w.batch, w.kv_heads, seq, w.head_dim)
    f32 = torch.float32
    if dist == "normal":
        x = torch.randn(shape, generator=g, device=device, dtype=f32)
    elif dist in ("t3_outlier4x20", "t4_outlier4x20", "normal_outlier2x15"):
        z = torch.randn(shape, generator=g, device=device, dtype=f32)
        if dist.startswith("t"):
            nu = 3 if dist.startswith("t3") else 4
            chi2 = torch.zeros(shape, device=device, dtype=f32)
            for _ in range(nu):
                chi2 += torch.randn(shape, generator=g, device=device, dtype=f32) ** 2
            z = z / torch.sqrt(chi2 / nu)
        count, factor = (2, 15.0) if dist == "normal_outlier2x15" else (4, 20.0)
        fac = torch.ones((w.batch, w.kv_heads, 1, w.head_dim), device=device, dtype=f32)
        for i in range(w.batch):
            for j in range(w.kv_heads):
                ch = torch.randperm(w.head_dim, generator=g, device=device)[:count]
                fac[i, j, 0, ch] = factor
        x = z * fac
    elif dist == "normal_bern01x10":
        z = torch.randn(shape, generator=g, device=device, dtype=f32)
        m = torch.rand(shape, generator=g, device=device, dtype=f32) < 0.01
        x = torch.where(m, 10.0 * z, z)
    elif dist == "normal_loguniform_std":
        lo, hi = np.log(0.5), np.log(8.0)
        std = torch.exp(lo + (hi - lo) * torch.rand((w.batch, w.kv_heads, 1, w.head_dim),
                                                     generator=g, device=device, dtype=f32))
        x = std * torch.randn(shape, generator=g, device=device, dtype=f32)
    else:
        raise ValueError(dist)
    return x.clamp_(-65504.0, 65504.0).to(torch.float16)


# ----------------------------------------------------------------------------------------------
# Random cache planes: in-range code bytes and positive fp16 scales drawn directly (no vector is
# quantized to make them), so a large cache costs only random-number generation.  A code plane
# row holds d*bits/8 bytes per token; every int4 nibble and every int8 byte is a two's-complement
# value in [-qmax, qmax] (-8 and -128, which the write path never produces, are replaced by 0).
# ----------------------------------------------------------------------------------------------
def random_code_bytes(rng: np.random.Generator, shape: tuple, bits: int) -> np.ndarray:
    """uint8 array of `shape` (the last axis counts bytes) holding random in-range codes."""
    b = rng.integers(0, 256, size=shape, dtype=np.uint8)
    if bits == 8:
        b[b == 0x80] = 0
        return b
    lo = b & 0x0F
    hi = b >> 4
    lo[lo == 8] = 0
    hi[hi == 8] = 0
    return (lo | (hi << 4)).astype(np.uint8)


def random_scales(rng: np.random.Generator, shape: tuple, lo: float, hi: float) -> np.ndarray:
    """float16 array of `shape`, log-uniform in [lo, hi]."""
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape)).astype(np.float16)


def random_lambda(rng: np.random.Generator, shape: tuple, lo: float = 0.5, hi: float = 8.0) -> np.ndarray:
    """float32 array of `shape`, log-uniform in [lo, hi] (per-channel factors)."""
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape)).astype(np.float32)


def torch_random_code_bytes(gen, numel: int, bits: int, device, chunk: int = 1 << 28):
    """random_code_bytes on a torch device (flat uint8 tensor of `numel` bytes), drawn in chunks
    with the seeded generator `gen`; same recipe, not the same numbers as the NumPy version."""
    import torch

    out = torch.empty(numel, dtype=torch.uint8, device=device)
    for i in range(0, numel, chunk):
        n = min(chunk, numel - i)
        b = torch.randint(0, 256, (n,), generator=gen, device=device, dtype=torch.uint8)
        if bits == 8:
            b[b == 0x80] = 0
        else:
            lo = b & 0x0F
            hi = b >> 4
            lo[lo == 8] = 0
            hi[hi == 8] = 0
            b = lo | (hi << 4)
        out[i:i + n] = b
    return out


def torch_random_scales(gen, numel: int, lo: float, hi: float, device, chunk: int = 1 << 28):
    """random_scales on a torch device: flat fp16 tensor, log-uniform in [lo, hi]."""
    import torch

    out = torch.empty(numel, dtype=torch.float16, device=device)
    a, b = float(np.log(lo)), float(np.log(hi))
    for i in range(0, numel, chunk):
        n = min(chunk, numel - i)
        u = torch.rand((n,), generator=gen, device=device, dtype=torch.float32)
        out[i:i + n] = torch.exp(a + (b - a) * u).to(torch.float16)
    return out
