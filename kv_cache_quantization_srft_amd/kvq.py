"""ctypes binding of libkvq.so (include/kvq.h).

Each function has the name of the C entry point it calls and takes the same arguments in the
same order; device buffers are passed as torch tensors.  The binding only checks dtype, device,
contiguity and size and passes raw pointers plus the current HIP stream: every step of the
computation runs in the library's kernels.  A missing library raises instead of falling back
to anything else.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK = 0
STATUS_NAMES = {
    0: "KVQ_OK", 1: "KVQ_ERR_INVALID_ARGUMENT", 2: "KVQ_ERR_UNSUPPORTED", 3: "KVQ_ERR_MISALIGNED",
    4: "KVQ_ERR_WORKSPACE_TOO_SMALL", 5: "KVQ_ERR_HIP",
}
EXPORTS = (
    "kvq_version", "kvq_status_string", "kvq_last_error_message", "kvq_codes_bytes", "kvq_scales_bytes",
    "kvq_quantize", "kvq_quantize_fft", "kvq_dequantize", "kvq_calibrate_lambda", "kvq_decode_attn_workspace_bytes",
    "kvq_decode_attn", "kvq_decode_attn_append", "kvq_decode_attn_paged", "kvq_decode_attn_fp16",
    "kvq_launch_plan", "kvq_decode_attn_noalloc", "kvq_attn", "kvq_attn_workspace_bytes", "kvq_attn_launch_plan",
)


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


TRANSFORMS = {"srft": 0, "srht": 1}


class kvq_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "kv_heads", "q_heads", "head_dim", "group_size", "k_bits", "v_bits", "capacity",
                 "transform")]


def make_layout(batch, kv_heads, q_heads, head_dim, capacity, k_bits=4, v_bits=4, group_size=16,
                transform="srft") -> kvq_layout:
    """transform: "srft" (KVQ_TRANSFORM_SRFT) or "srht" (KVQ_TRANSFORM_SRHT), or the enum value."""
    tr = TRANSFORMS[transform] if isinstance(transform, str) else int(transform)
    return kvq_layout(batch, kv_heads, q_heads, head_dim, group_size, k_bits, v_bits, capacity, tr)


CALLS = {"quantize": 0, "decode": 1, "decode_append": 2, "decode_paged": 3, "decode_paged_append": 4,
         "decode_fp16": 5}


class kvq_plan(ctypes.Structure):
    _fields_ = [("work_groups", ctypes.c_int64), ("head_tile", ctypes.c_int32), ("head_tiles", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("n_chunks", ctypes.c_int32), ("wave_tokens", ctypes.c_int32),
                ("superblocks_per_wave", ctypes.c_int32), ("blocks", ctypes.c_int64),
                ("blocks_per_work_group", ctypes.c_int64), ("query_tile", ctypes.c_int32),
                ("query_tiles", ctypes.c_int32)]


class kvq_attn_opts(ctypes.Structure):
    _fields_ = [("n_query", ctypes.c_int32), ("window", ctypes.c_int32), ("ring", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_LP = ctypes.POINTER(kvq_layout)


def lib() -> ctypes.CDLL:
    """Load libkvq.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_quantization_srft_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.kvq_version.restype = _I32
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_status_string.argtypes = [ctypes.c_int]
        L.kvq_last_error_message.restype = ctypes.c_char_p
        L.kvq_codes_bytes.restype = _SZ
        L.kvq_codes_bytes.argtypes = [_LP, _I32]
        L.kvq_scales_bytes.restype = _SZ
        L.kvq_scales_bytes.argtypes = [_LP]
        L.kvq_quantize.restype = ctypes.c_int
        L.kvq_quantize.argtypes = [_LP, _I32, _P, _I32, _I32, _P, _I64, _P, _I64, _P, _P, _P]
        L.kvq_quantize_fft.restype = ctypes.c_int
        L.kvq_quantize_fft.argtypes = [_LP, _I32, _P, _I32, _I32, _P, _I64, _P, _I64, _P, _P, _P]
        L.kvq_dequantize.restype = ctypes.c_int
        L.kvq_dequantize.argtypes = [_LP, _I32, _P, _P, _I32, _I32, _P, _I64, _P, _I64, _P, _P]
        L.kvq_calibrate_lambda.restype = ctypes.c_int
        L.kvq_calibrate_lambda.argtypes = [_LP, _P, _I32, _I32, _P, _I64, _P, _P]
        L.kvq_decode_attn_workspace_bytes.restype = _SZ
        L.kvq_decode_attn_workspace_bytes.argtypes = [_LP, _I32]
        L.kvq_decode_attn.restype = ctypes.c_int
        L.kvq_decode_attn.argtypes = [_LP, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _I64, _P, _P, _I64,
                                      ctypes.c_float, _P, _SZ, _P, _P]
        L.kvq_decode_attn_append.restype = ctypes.c_int
        L.kvq_decode_attn_append.argtypes = [_LP, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _I64, _P, _P,
                                             _I64, ctypes.c_float, _P, _SZ, _P, _P]
        L.kvq_decode_attn_paged.restype = ctypes.c_int
        L.kvq_decode_attn_paged.argtypes = [_LP, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P,
                                            _P, _I64, _P, _P, _I64, ctypes.c_float, _P, _SZ, _P, _P]
        L.kvq_decode_attn_fp16.restype = ctypes.c_int
        L.kvq_decode_attn_fp16.argtypes = [_LP, _P, _P, _P, _I32, _P, ctypes.c_float, _P, _SZ, _P, _P]
        L.kvq_decode_attn_noalloc.restype = ctypes.c_int
        L.kvq_decode_attn_noalloc.argtypes = [_LP, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _I64, _P, _P, _I64,
                                              ctypes.c_float, _P, _P]
        L.kvq_attn.restype = ctypes.c_int
        L.kvq_attn.argtypes = [_LP, ctypes.POINTER(kvq_attn_opts), _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P,
                               _P, _P, _I64, _P, _P, _I64, ctypes.c_float, _P, _SZ, _P, _P]
        L.kvq_attn_workspace_bytes.restype = _SZ
        L.kvq_attn_workspace_bytes.argtypes = [_LP, ctypes.POINTER(kvq_attn_opts), _I32]
        L.kvq_attn_launch_plan.restype = ctypes.c_int
        L.kvq_attn_launch_plan.argtypes = [_LP, ctypes.POINTER(kvq_attn_opts), _I32, _I32, ctypes.POINTER(kvq_plan)]
        L.kvq_launch_plan.restype = ctypes.c_int
        L.kvq_launch_plan.argtypes = [_LP, ctypes.c_int, _I32, ctypes.POINTER(kvq_plan)]
        _lib = L
    return _lib


def _check(status: int):
    if status != KVQ_OK:
        msg = lib().kvq_last_error_message().decode()
        raise KvqError(status, msg or STATUS_NAMES.get(status, str(status)))


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t, dtype, name, numel=None, min_bytes=None):
    """Device pointer of a contiguous tensor (None -> NULL) after dtype/size checks."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, needs {min_bytes}")
    return t.data_ptr()


def _f16():
    import torch
    return torch.float16


def _f32():
    import torch
    return torch.float32


def _u8():
    import torch
    return (torch.uint8, torch.int8)


def _scale_t():
    import torch
    return (torch.float16, torch.int16)


def kvq_version() -> int:
    return lib().kvq_version()


def kvq_codes_bytes(layout: kvq_layout, bits: int) -> int:
    return lib().kvq_codes_bytes(ctypes.byref(layout), bits)


def kvq_scales_bytes(layout: kvq_layout) -> int:
    return lib().kvq_scales_bytes(ctypes.byref(layout))


def kvq_decode_attn_workspace_bytes(layout: kvq_layout, max_seq_len: int) -> int:
    return lib().kvq_decode_attn_workspace_bytes(ctypes.byref(layout), max_seq_len)


def kvq_quantize(layout, bits, x, pos, n_tok, sign, sign_batch_stride, lam, lambda_batch_stride, codes, scales,
                 stream=None):
    _quantize_call(lib().kvq_quantize, layout, bits, x, pos, n_tok, sign, sign_batch_stride, lam,
                   lambda_batch_stride, codes, scales, stream)


def kvq_quantize_fft(layout, bits, x, pos, n_tok, sign, sign_batch_stride, lam, lambda_batch_stride, codes, scales,
                     stream=None):
    _quantize_call(lib().kvq_quantize_fft, layout, bits, x, pos, n_tok, sign, sign_batch_stride, lam,
                   lambda_batch_stride, codes, scales, stream)


def _quantize_call(fn, layout, bits, x, pos, n_tok, sign, sign_batch_stride, lam, lambda_batch_stride, codes, scales,
                   stream):
    d = layout.head_dim
    _check(fn(
        ctypes.byref(layout), bits, _ptr(x, _f16(), "x", layout.batch * layout.kv_heads * n_tok * d), pos, n_tok,
        _ptr(sign, _f32(), "sign"), sign_batch_stride, _ptr(lam, _f32(), "lambda"), lambda_batch_stride,
        _ptr(codes, _u8(), "codes", min_bytes=kvq_codes_bytes(layout, bits)),
        _ptr(scales, _scale_t(), "scales", min_bytes=kvq_scales_bytes(layout)), _stream(stream)))


def kvq_dequantize(layout, bits, codes, scales, pos, n_tok, sign, sign_batch_stride, lam, lambda_batch_stride, out,
                   stream=None):
    d = layout.head_dim
    _check(lib().kvq_dequantize(
        ctypes.byref(layout), bits, _ptr(codes, _u8(), "codes", min_bytes=kvq_codes_bytes(layout, bits)),
        _ptr(scales, _scale_t(), "scales", min_bytes=kvq_scales_bytes(layout)), pos, n_tok,
        _ptr(sign, _f32(), "sign"), sign_batch_stride, _ptr(lam, _f32(), "lambda"), lambda_batch_stride,
        _ptr(out, _f32(), "out", layout.batch * layout.kv_heads * n_tok * d), _stream(stream)))


def kvq_calibrate_lambda(layout, x, n_tok, n_cal, sign, sign_batch_stride, lam, stream=None):
    d = layout.head_dim
    _check(lib().kvq_calibrate_lambda(
        ctypes.byref(layout), _ptr(x, _f16(), "x", layout.batch * layout.kv_heads * n_tok * d), n_tok, n_cal,
        _ptr(sign, _f32(), "sign"), sign_batch_stride,
        _ptr(lam, _f32(), "lambda", layout.batch * layout.kv_heads * d), _stream(stream)))


def kvq_decode_attn(layout, q, k_codes, k_scales, v_codes, v_scales, seq_len, seq_lens, sign_k, sign_v,
                    sign_batch_stride, lambda_k, lambda_v, lambda_batch_stride, sm_scale, workspace, out,
                    stream=None):
    import torch
    d = layout.head_dim
    _check(lib().kvq_decode_attn(
        ctypes.byref(layout), _ptr(q, _f16(), "q", layout.batch * layout.q_heads * d),
        _ptr(k_codes, _u8(), "k_codes", min_bytes=kvq_codes_bytes(layout, layout.k_bits)),
        _ptr(k_scales, _scale_t(), "k_scales", min_bytes=kvq_scales_bytes(layout)),
        _ptr(v_codes, _u8(), "v_codes", min_bytes=kvq_codes_bytes(layout, layout.v_bits)),
        _ptr(v_scales, _scale_t(), "v_scales", min_bytes=kvq_scales_bytes(layout)), seq_len,
        _ptr(seq_lens, torch.int32, "seq_lens", layout.batch), _ptr(sign_k, _f32(), "sign_k"),
        _ptr(sign_v, _f32(), "sign_v"), sign_batch_stride, _ptr(lambda_k, _f32(), "lambda_k"),
        _ptr(lambda_v, _f32(), "lambda_v"), lambda_batch_stride, float(sm_scale),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, _f32(), "out", layout.batch * layout.q_heads * d), _stream(stream)))


def kvq_decode_attn_noalloc(layout, q, k_codes, k_scales, v_codes, v_scales, seq_len, seq_lens, sign_k, sign_v,
                            sign_batch_stride, lambda_k, lambda_v, lambda_batch_stride, sm_scale, out, stream=None):
    import torch
    d = layout.head_dim
    _check(lib().kvq_decode_attn_noalloc(
        ctypes.byref(layout), _ptr(q, _f16(), "q", layout.batch * layout.q_heads * d),
        _ptr(k_codes, _u8(), "k_codes", min_bytes=kvq_codes_bytes(layout, layout.k_bits)),
        _ptr(k_scales, _scale_t(), "k_scales", min_bytes=kvq_scales_bytes(layout)),
        _ptr(v_codes, _u8(), "v_codes", min_bytes=kvq_codes_bytes(layout, layout.v_bits)),
        _ptr(v_scales, _scale_t(), "v_scales", min_bytes=kvq_scales_bytes(layout)), seq_len,
        _ptr(seq_lens, torch.int32, "seq_lens", layout.batch), _ptr(sign_k, _f32(), "sign_k"),
        _ptr(sign_v, _f32(), "sign_v"), sign_batch_stride, _ptr(lambda_k, _f32(), "lambda_k"),
        _ptr(lambda_v, _f32(), "lambda_v"), lambda_batch_stride, float(sm_scale),
        _ptr(out, _f32(), "out", layout.batch * layout.q_heads * d), _stream(stream)))


def kvq_decode_attn_append(layout, q, k_new, v_new, k_codes, k_scales, v_codes, v_scales, seq_len, seq_lens,
                           sign_k, sign_v, sign_batch_stride, lambda_k, lambda_v, lambda_batch_stride, sm_scale,
                           workspace, out, stream=None):
    import torch
    d = layout.head_dim
    n_new = layout.batch * layout.kv_heads * d
    _check(lib().kvq_decode_attn_append(
        ctypes.byref(layout), _ptr(q, _f16(), "q", layout.batch * layout.q_heads * d),
        _ptr(k_new, _f16(), "k_new", n_new), _ptr(v_new, _f16(), "v_new", n_new),
        _ptr(k_codes, _u8(), "k_codes", min_bytes=kvq_codes_bytes(layout, layout.k_bits)),
        _ptr(k_scales, _scale_t(), "k_scales", min_bytes=kvq_scales_bytes(layout)),
        _ptr(v_codes, _u8(), "v_codes", min_bytes=kvq_codes_bytes(layout, layout.v_bits)),
        _ptr(v_scales, _scale_t(), "v_scales", min_bytes=kvq_scales_bytes(layout)), seq_len,
        _ptr(seq_lens, torch.int32, "seq_lens", layout.batch), _ptr(sign_k, _f32(), "sign_k"),
        _ptr(sign_v, _f32(), "sign_v"), sign_batch_stride, _ptr(lambda_k, _f32(), "lambda_k"),
        _ptr(lambda_v, _f32(), "lambda_v"), lambda_batch_stride, float(sm_scale),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, _f32(), "out", layout.batch * layout.q_heads * d), _stream(stream)))


def _page_plane_bytes(layout, bits, num_pages, page_size, scales=False):
    """Bytes of one paged plane [num_pages, kv_heads, page_size, .] (codes, or scales)."""
    per_tok = layout.head_dim // layout.group_size * 2 if scales else layout.head_dim * bits // 8
    return num_pages * layout.kv_heads * page_size * per_tok


def kvq_decode_attn_paged(layout, q, k_new, v_new, k_codes, k_scales, v_codes, v_scales, page_table, pages_per_seq,
                          page_size, num_pages, seq_len, seq_lens, sign_k, sign_v, sign_batch_stride, lambda_k,
                          lambda_v, lambda_batch_stride, sm_scale, workspace, out, stream=None):
    import torch
    d = layout.head_dim
    n_new = layout.batch * layout.kv_heads * d
    _check(lib().kvq_decode_attn_paged(
        ctypes.byref(layout), _ptr(q, _f16(), "q", layout.batch * layout.q_heads * d),
        _ptr(k_new, _f16(), "k_new", n_new), _ptr(v_new, _f16(), "v_new", n_new),
        _ptr(k_codes, _u8(), "k_codes", min_bytes=_page_plane_bytes(layout, layout.k_bits, num_pages, page_size)),
        _ptr(k_scales, _scale_t(), "k_scales",
             min_bytes=_page_plane_bytes(layout, 0, num_pages, page_size, scales=True)),
        _ptr(v_codes, _u8(), "v_codes", min_bytes=_page_plane_bytes(layout, layout.v_bits, num_pages, page_size)),
        _ptr(v_scales, _scale_t(), "v_scales",
             min_bytes=_page_plane_bytes(layout, 0, num_pages, page_size, scales=True)),
        _ptr(page_table, torch.int32, "page_table", layout.batch * pages_per_seq), pages_per_seq, page_size,
        num_pages, seq_len, _ptr(seq_lens, torch.int32, "seq_lens", layout.batch), _ptr(sign_k, _f32(), "sign_k"),
        _ptr(sign_v, _f32(), "sign_v"), sign_batch_stride, _ptr(lambda_k, _f32(), "lambda_k"),
        _ptr(lambda_v, _f32(), "lambda_v"), lambda_batch_stride, float(sm_scale),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, _f32(), "out", layout.batch * layout.q_heads * d), _stream(stream)))


def kvq_decode_attn_fp16(layout, q, k, v, seq_len, seq_lens, sm_scale, workspace, out, stream=None):
    import torch
    d = layout.head_dim
    kv_numel = layout.batch * layout.kv_heads * layout.capacity * d
    _check(lib().kvq_decode_attn_fp16(
        ctypes.byref(layout), _ptr(q, _f16(), "q", layout.batch * layout.q_heads * d),
        _ptr(k, _f16(), "k", kv_numel), _ptr(v, _f16(), "v", kv_numel), seq_len,
        _ptr(seq_lens, torch.int32, "seq_lens", layout.batch), float(sm_scale), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(out, _f32(), "out", layout.batch * layout.q_heads * d),
        _stream(stream)))


def kvq_launch_plan(layout, call, n) -> kvq_plan:
    """call: a key of CALLS ("quantize", "decode", ...) or its enum value; returns the plan struct."""
    c = CALLS[call] if isinstance(call, str) else int(call)
    out = kvq_plan()
    _check(lib().kvq_launch_plan(ctypes.byref(layout), c, n, ctypes.byref(out)))
    return out


def make_attn_opts(n_query=1, window=0, ring=False) -> kvq_attn_opts:
    return kvq_attn_opts(n_query, window, 1 if ring else 0)


def kvq_attn_workspace_bytes(layout, opts, max_seq_len) -> int:
    return lib().kvq_attn_workspace_bytes(ctypes.byref(layout), ctypes.byref(opts), max_seq_len)


def kvq_attn_launch_plan(layout, opts, seq_len, paged=False) -> kvq_plan:
    out = kvq_plan()
    _check(lib().kvq_attn_launch_plan(ctypes.byref(layout), ctypes.byref(opts), seq_len, 1 if paged else 0,
                                      ctypes.byref(out)))
    return out


def kvq_attn(layout, opts, q, k_codes, k_scales, v_codes, v_scales, page_table, pages_per_seq, page_size, num_pages,
             seq_len, seq_lens, sign_k, sign_v, sign_batch_stride, lambda_k, lambda_v, lambda_batch_stride, sm_scale,
             workspace, out, stream=None):
    """page_table None: contiguous rows (planes sized by the layout); otherwise paged planes of
    num_pages pages."""
    import torch
    d = layout.head_dim
    rows = layout.batch * opts.n_query * layout.q_heads * d
    if page_table is None:
        kcb, vcb = kvq_codes_bytes(layout, layout.k_bits), kvq_codes_bytes(layout, layout.v_bits)
        scb = kvq_scales_bytes(layout)
    else:
        kcb = _page_plane_bytes(layout, layout.k_bits, num_pages, page_size)
        vcb = _page_plane_bytes(layout, layout.v_bits, num_pages, page_size)
        scb = _page_plane_bytes(layout, 0, num_pages, page_size, scales=True)
    _check(lib().kvq_attn(
        ctypes.byref(layout), ctypes.byref(opts), _ptr(q, _f16(), "q", rows),
        _ptr(k_codes, _u8(), "k_codes", min_bytes=kcb), _ptr(k_scales, _scale_t(), "k_scales", min_bytes=scb),
        _ptr(v_codes, _u8(), "v_codes", min_bytes=vcb), _ptr(v_scales, _scale_t(), "v_scales", min_bytes=scb),
        _ptr(page_table, torch.int32, "page_table", None if page_table is None else layout.batch * pages_per_seq),
        pages_per_seq, page_size, num_pages, seq_len, _ptr(seq_lens, torch.int32, "seq_lens", layout.batch),
        _ptr(sign_k, _f32(), "sign_k"), _ptr(sign_v, _f32(), "sign_v"), sign_batch_stride,
        _ptr(lambda_k, _f32(), "lambda_k"), _ptr(lambda_v, _f32(), "lambda_v"), lambda_batch_stride,
        float(sm_scale), _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, _f32(), "out", rows), _stream(stream)))
