"""Plain CPU oracle for SRFT-rotated low-bit KV-cache quantization and decode attention.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct reference that the
HIP kernels are checked against.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import it; the product path (the C-ABI library and its Python
binding) never calls it, and it shares no code, table or constant with that path.

Everything is NumPy float64 unless stated otherwise.  The transform is the plain O(d^2)
unitary DFT written out as a sum, not an FFT.

Sources (web pages; cited by title and section):
  [QF]  "When Quantization Is Free: An int4 KV Cache That Outruns fp16 on Apple Silicon",
        gist.science explainer, technical summary ("技术摘要"), Methodology
        ("方法论") items 1 (SRFT), 2 (fused Metal kernel steps) and 3 (per-channel +
        per-group scaling); Key results, memory efficiency ("内存效率").
  [GM]  hotdry blog, "Gemini on-device quantization and KV cache on Apple Silicon",
        sections "INT8/INT4 量化策略" (KV footprint formula, int4 = 25% of fp16) and
        "Flash Attention 与 Metal 内核融合" (tiled attention with online softmax).
  [KS]  xugj520 article on KVSplit, table "内存节省对比（8K上下文）" and section
        "内存优化计算" (K8V4: keys 8-bit, values 4-bit).

Readings taken where the pages are silent (each also listed in the design notes):
  R1  DFT sign/normalisation: X[k] = d^-1/2 * sum_n y[n] exp(-2 pi i k n / d).
  R2  Real layout of the Hermitian half-spectrum, interleaved:
      [Re X0, Re X_{d/2}, sqrt2 Re X1, sqrt2 Im X1, ..., sqrt2 Re X_{d/2-1}, sqrt2 Im X_{d/2-1}].
      The sqrt2 weights make the map orthogonal (norm preserving).
  R3  lambda divides the rotated vector before quantization and multiplies it back after;
      it lives in the rotated domain, one value per (sequence/layer, kv head, channel).
  R4  Groups are 16 consecutive channels of the rotated, lambda-scaled vector.
  R5  Symmetric absmax quantizer, qmax = 7 (int4) or 127 (int8); -8/-128 unused.
  R6  Scales are fp16 (round-to-nearest-even, saturated at 65504); codes are computed
      against the rounded scale; a zero scale gives zero codes.
  R7  The code decision (scale rounding, u/scale, round-half-even) is taken in float32,
      the kernel's precision, on the float64 transform rounded once to float32.
  R8  Nibble order: low nibble = even channel; int4 codes are two's complement nibbles.
  R9  Decode attends cache positions [0, seq_len); query head h reads kv head h // G;
      softmax scale defaults to 1/sqrt(d); output is float in the original domain.
  R10 Calibrated lambda = per-channel absmax of SRFT(x) over the first n_cal tokens;
      a zero absmax is replaced by 1.
  R13 SRHT (the pages' alternative rotation, [QF] Methodology 1 and Key results, SRFT vs
      SRHT): SRHT(x) = d^-1/2 H_d diag(s) x with H_d the Sylvester-ordered Walsh-Hadamard
      matrix, H[i][j] = (-1)^popcount(i & j); everything downstream (lambda, quantizer,
      decode) is unchanged.  Functions take transform="srft" (default) or "srht".
  R14 Several query tokens per sequence (chunked prefill, speculative verification; [GM]
      "Flash Attention 与 Metal 内核融合"): the T new tokens are the last T positions of the
      cache (already written); query i of a sequence of length L sits at position
      p = L - T + i and attends causally, positions t <= p.  A query whose position would be
      negative (L < T) has a zero output.
  R15 Sliding window ([GM] "KV 缓存分片与内存管理": keep the latest tokens): with a window W >= 1
      a query at position p attends the W most recent positions up to its own, t in
      [max(0, p - W + 1), p]; W = 0 means no window.
  R16 Ring buffer: logical position t of a row is stored at plane slot t mod capacity.  This is a
      storage convention only; attention is defined on logical positions (tests lay the planes
      out from the logical rows).
"""
from __future__ import annotations

import numpy as np

GROUP = 16
QMAX = {4: 7, 8: 127}
FP16_MAX = 65504.0


# ----------------------------------------------------------------------------------------
# Transform  [QF] Methodology 1: SRFT(x) = pack(F diag(s) x), F the unitary DFT.
# ----------------------------------------------------------------------------------------
def unitary_dft(y: np.ndarray) -> np.ndarray:
    """X[k] = d^-1/2 * sum_n y[n] * exp(-2 pi i k n / d), over the last axis (reading R1)."""
    y = np.asarray(y, dtype=np.complex128)
    d = y.shape[-1]
    n = np.arange(d)
    w = np.exp(-2j * np.pi * np.outer(n, n) / d) / np.sqrt(d)  # w[k, n]
    return np.einsum("...n,kn->...k", y, w)


def inverse_unitary_dft(X: np.ndarray) -> np.ndarray:
    """y[n] = d^-1/2 * sum_k X[k] * exp(+2 pi i k n / d): the conjugate transpose of unitary_dft."""
    X = np.asarray(X, dtype=np.complex128)
    d = X.shape[-1]
    n = np.arange(d)
    w = np.exp(2j * np.pi * np.outer(n, n) / d) / np.sqrt(d)  # w[n, k]
    return np.einsum("...k,nk->...n", X, w)


def hermitian_pack(X: np.ndarray) -> np.ndarray:
    """Real, norm-preserving layout of the spectrum of a real vector (readings R2).

    [QF] Methodology 2 ("打包"): the Hermitian symmetry of a real input's spectrum is
    unpacked into a real representation.  Only bins 0..d/2 are independent; bins 0 and d/2
    are real.
    """
    d = X.shape[-1]
    m = d // 2
    out = np.empty(X.shape, dtype=np.float64)
    out[..., 0] = X[..., 0].real
    out[..., 1] = X[..., m].real
    for k in range(1, m):
        out[..., 2 * k] = np.sqrt(2.0) * X[..., k].real
        out[..., 2 * k + 1] = np.sqrt(2.0) * X[..., k].imag
    return out


def hermitian_unpack(y: np.ndarray) -> np.ndarray:
    """Inverse of hermitian_pack: rebuild the full conjugate-symmetric spectrum."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    m = d // 2
    X = np.zeros(y.shape, dtype=np.complex128)
    X[..., 0] = y[..., 0]
    X[..., m] = y[..., 1]
    for k in range(1, m):
        X[..., k] = (y[..., 2 * k] + 1j * y[..., 2 * k + 1]) / np.sqrt(2.0)
        X[..., d - k] = np.conj(X[..., k])
    return X


def srft(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """SRFT(x) = pack(F diag(s) x)  ([QF] Methodology 1; sign applied first, Methodology 2)."""
    x = np.asarray(x, dtype=np.float64)
    return hermitian_pack(unitary_dft(np.asarray(s, dtype=np.float64) * x))


def inverse_srft(y: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x = diag(s) F^H unpack(y): the exact inverse of srft (s is +-1 so diag(s) is its own inverse)."""
    z = inverse_unitary_dft(hermitian_unpack(y))
    return np.asarray(s, dtype=np.float64) * z.real


def hadamard_matrix(d: int) -> np.ndarray:
    """Sylvester-ordered Walsh-Hadamard matrix, H[i][j] = (-1)^popcount(i & j) (reading R13)."""
    i = np.arange(d)
    a = np.bitwise_and(i[:, None], i[None, :])
    parity = np.zeros_like(a)
    while a.any():
        parity ^= a & 1
        a >>= 1
    return np.where(parity == 1, -1.0, 1.0)


def srht(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """SRHT(x) = d^-1/2 H diag(s) x (reading R13)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    return (np.asarray(s, dtype=np.float64) * x) @ hadamard_matrix(d).T / np.sqrt(d)


def inverse_srht(y: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x = diag(s) d^-1/2 H y: H H = d I, so this is the exact inverse of srht."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    return np.asarray(s, dtype=np.float64) * (y @ hadamard_matrix(d).T / np.sqrt(d))


def rotate(x: np.ndarray, s: np.ndarray, transform: str = "srft") -> np.ndarray:
    """The rotation of the write path: SRFT (readings R1, R2) or SRHT (R13)."""
    if transform == "srft":
        return srft(x, s)
    if transform == "srht":
        return srht(x, s)
    raise ValueError(f"unknown transform {transform!r}")


def inverse_rotate(y: np.ndarray, s: np.ndarray, transform: str = "srft") -> np.ndarray:
    if transform == "srft":
        return inverse_srft(y, s)
    if transform == "srht":
        return inverse_srht(y, s)
    raise ValueError(f"unknown transform {transform!r}")


# ----------------------------------------------------------------------------------------
# Quantizer  [QF] Methodology 2 ("缩放与量化", "半字节打包") and 3 (per-channel + per-group).
# ----------------------------------------------------------------------------------------
def rotated_scaled(x16: np.ndarray, s: np.ndarray, lam: np.ndarray, transform: str = "srft") -> np.ndarray:
    """u = SRFT(x) / lambda in float64 (reading R3).  x16 is taken as stored (fp16 -> f64)."""
    return rotate(np.asarray(x16).astype(np.float64), s, transform) / np.asarray(lam, dtype=np.float64)


def fp16_saturate(v32: np.ndarray) -> np.ndarray:
    """float32 -> float16, round-to-nearest-even, saturating at 65504 (reading R6)."""
    v32 = np.asarray(v32, dtype=np.float32)
    return np.minimum(v32, np.float32(FP16_MAX)).astype(np.float16)


def quantize_decision(u: np.ndarray, bits: int, group: int = GROUP):
    """Group absmax -> fp16 scale -> signed codes, decided in float32 (readings R4-R7).

    u: [..., d] float64 (the rotated, lambda-scaled vector).
    Returns (codes int8 [..., d], scales float16 [..., d // group]).
    """
    qmax = QMAX[bits]
    u32 = np.asarray(u, dtype=np.float64).astype(np.float32)
    shape = u32.shape
    g = u32.reshape(shape[:-1] + (shape[-1] // group, group))
    absmax = np.abs(g).max(axis=-1)                                   # float32, exact
    scale16 = fp16_saturate(absmax / np.float32(qmax))                # f32 divide, RNE to fp16
    scale32 = scale16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = g / scale32[..., None]                                # f32 divide
    codes = np.where(scale32[..., None] > 0,
                     np.clip(np.rint(ratio), -qmax, qmax), 0).astype(np.int8)
    return codes.reshape(shape), scale16


def quantize(x16: np.ndarray, s: np.ndarray, lam: np.ndarray, bits: int, group: int = GROUP,
             transform: str = "srft"):
    """Full write path for vectors x16 [..., d]: sign -> DFT -> pack -> /lambda -> absmax -> round.

    lam broadcasts against x16 (e.g. [Hkv, 1, d] for x16 [Hkv, n, d]).
    Returns (codes int8, scales float16).
    """
    return quantize_decision(rotated_scaled(x16, s, lam, transform), bits, group)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Byte layout of the code plane (reading R8).

    int4: byte j = (c[2j] & 0xF) | ((c[2j+1] & 0xF) << 4)  -- two int4 per byte ([QF] Methodology 2).
    int8: the two's-complement byte of each code.
    """
    c = np.asarray(codes).astype(np.int64)
    if bits == 8:
        return (c & 0xFF).astype(np.uint8)
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_codes: bytes -> signed codes (int8)."""
    b = np.asarray(packed).astype(np.int64)
    if bits == 8:
        return np.where(b >= 128, b - 256, b).astype(np.int8)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequantize(codes: np.ndarray, scales16: np.ndarray, s: np.ndarray, lam: np.ndarray,
               group: int = GROUP, transform: str = "srft") -> np.ndarray:
    """x_hat = diag(s) F^H unpack(lambda * code * scale), float64 (inverse of the write path)."""
    c = np.asarray(codes).astype(np.float64)
    sc = np.repeat(np.asarray(scales16).astype(np.float64), group, axis=-1)
    y = np.asarray(lam, dtype=np.float64) * (c * sc)
    return inverse_rotate(y, s, transform)


def calibrate_lambda(x16: np.ndarray, s: np.ndarray, n_cal: int, transform: str = "srft") -> np.ndarray:
    """Per-channel absmax of SRFT(x) over the first n_cal tokens (reading R10).

    x16: [..., n, d] -> lambda [..., d] float64.  Zero channels get lambda = 1.
    """
    y = rotate(np.asarray(x16)[..., :n_cal, :].astype(np.float64), s, transform)
    lam = np.abs(y).max(axis=-2)
    return np.where(lam > 0, lam, 1.0)


# ----------------------------------------------------------------------------------------
# Decode attention by definition  ([GM] "Flash Attention 与 Metal 内核融合": attention is
# softmax(q K^T) V; tiling and online softmax change only the order of the sums).
# ----------------------------------------------------------------------------------------
def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens, sm_scale=None):
    """Single-token attention for every (sequence, query head), float64.

    q: [B, Hq, d]; k, v: [B, Hkv, >=max(seq_lens), d] (already dequantized, original domain).
    seq_lens: int or [B].  Query head h uses kv head h // (Hq // Hkv) (reading R9).
    Returns o: [B, Hq, d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    lens = np.broadcast_to(np.asarray(seq_lens), (B,))
    o = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            j = h // G
            logits = sm_scale * (k[b, j, :L] @ q[b, h])
            p = np.exp(logits - logits.max())
            p /= p.sum()
            o[b, h] = p @ v[b, j, :L]
    return o


def decode_attention_quantized(q16, k_codes, k_scales, v_codes, v_scales, s_k, s_v, lam_k, lam_v,
                               seq_lens, sm_scale=None, transform: str = "srft"):
    """Decode attention over a quantized cache: dequantize every K/V vector, then attend.

    Codes are unpacked int8 codes [B, Hkv, S, d]; scales float16 [B, Hkv, S, d/16];
    lam_k, lam_v broadcast against [B, Hkv, 1, d].
    """
    k_hat = dequantize(k_codes, k_scales, s_k, lam_k, transform=transform)
    v_hat = dequantize(v_codes, v_scales, s_v, lam_v, transform=transform)
    return decode_attention(np.asarray(q16).astype(np.float64), k_hat, v_hat, seq_lens, sm_scale)


def prefix_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens, n_query: int, window: int = 0,
                     sm_scale=None):
    """Attention of the last n_query positions of every sequence over its cache (readings R14,
    R15), float64, by definition with explicit loops over sequences, query tokens and heads.

    q: [B, T, Hq, d] (T = n_query); k, v: [B, Hkv, >= max(seq_lens), d] in the original domain.
    Query i of sequence b (length L) sits at p = L - T + i and attends positions
    t in [lo, p] with lo = max(0, p - window + 1) if window >= 1 else 0; p < 0 gives zeros.
    Query head h reads kv head h // (Hq // Hkv).  Returns o: [B, T, Hq, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, Hq, d = q.shape
    assert T == n_query
    Hkv = k.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    lens = np.broadcast_to(np.asarray(seq_lens), (B,))
    o = np.zeros((B, T, Hq, d))
    for b in range(B):
        L = int(lens[b])
        for i in range(T):
            p = L - T + i
            if p < 0:
                continue
            lo = max(0, p - window + 1) if window >= 1 else 0
            for h in range(Hq):
                j = h // G
                logits = sm_scale * (k[b, j, lo:p + 1] @ q[b, i, h])
                w = np.exp(logits - logits.max())
                w /= w.sum()
                o[b, i, h] = w @ v[b, j, lo:p + 1]
    return o


def prefix_attention_quantized(q16, k_codes, k_scales, v_codes, v_scales, s_k, s_v, lam_k, lam_v, seq_lens,
                               n_query: int, window: int = 0, sm_scale=None, transform: str = "srft"):
    """prefix_attention over a quantized cache: dequantize every K/V vector, then attend
    (codes unpacked int8 [B, Hkv, S, d], scales float16 [B, Hkv, S, d/16])."""
    k_hat = dequantize(k_codes, k_scales, s_k, lam_k, transform=transform)
    v_hat = dequantize(v_codes, v_scales, s_v, lam_v, transform=transform)
    return prefix_attention(np.asarray(q16).astype(np.float64), k_hat, v_hat, seq_lens, n_query, window, sm_scale)


# ----------------------------------------------------------------------------------------
# Footprint arithmetic  ([GM] KV cache memory formula; [KS] "内存优化计算"; [QF] memory efficiency)
# ----------------------------------------------------------------------------------------
def fp16_kv_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, batch: int = 1) -> int:
    """2 (K and V) x layers x kv_heads x head_dim x seq_len x 2 bytes."""
    return 2 * layers * kv_heads * head_dim * seq_len * 2 * batch


def quantized_kv_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, k_bits: int,
                       v_bits: int, batch: int = 1, group: int = GROUP, scale_bits: int = 16,
                       with_scales: bool = True) -> float:
    """Codes (k_bits + v_bits per channel) plus one scale_bits scale per group, per K and V."""
    per_elem_bits = k_bits + v_bits
    if with_scales:
        per_elem_bits += 2 * scale_bits / group
    return layers * kv_heads * head_dim * seq_len * batch * per_elem_bits / 8
