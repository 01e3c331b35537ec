"""Python binding of libdsa: content-aware dynamic block-sparse causal attention
on AMD MI355X (gfx950).

The functions named ``dsa_*`` mirror the C ABI in ``include/dsa.h`` one to one:
they check that the torch tensors match the shape (dtype, device, size,
contiguity -- the C side cannot see tensor sizes), pass raw device pointers
and the current HIP stream, and raise ``DsaError`` on a non-zero status.
Every step of the computation runs in the HIP library; there is no fallback.
``prefill`` and ``decode`` are conveniences that allocate the outputs and
the workspace with torch and call the fused entry points.
"""

from __future__ import annotations

import ctypes
import functools
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

FORCE_SINK = 1
FORCE_DIAG = 2
DETERMINISTIC = 4  # decode: the same bits on every call (fixed work order)
SELECT_TOPK, SELECT_THRESHOLD, SELECT_ENTROPY = 0, 1, 2
MAX_BLOCKS = 4096

LAYOUT_PREFILL, LAYOUT_DECODE, LAYOUT_PAGED = 0, 1, 2
CHECK_SLOTS = ("rows", "count", "range", "order", "forced", "padding")  # report slots of the selection validator

DSA_OK, DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = 0, -1, -2, -3, -4, -5

EXPORTS = [
    "dsa_kmax",
    "dsa_prefill_kmax",
    "dsa_decode_kmax",
    "dsa_block_means",
    "dsa_block_scores",
    "dsa_block_scores_from_means",
    "dsa_select_topk",
    "dsa_indices_to_bitmap",
    "dsa_check_block_selection",
    "dsa_check_token_selection",
    "dsa_index_kmax",
    "dsa_index_scores",
    "dsa_select_tokens",
    "dsa_token_attn_fwd",
    "dsa_index_topk",
    "dsa_index_workspace_bytes",
    "dsa_index_prefill",
    "dsa_sparse_attn_fwd",
    "dsa_prefill_workspace_bytes",
    "dsa_prefill",
    "dsa_attn_bwd_workspace_bytes",
    "dsa_sparse_attn_bwd",
    "dsa_kv_block_means",
    "dsa_decode_workspace_bytes",
    "dsa_decode",
    "dsa_decode_noalloc",
    "dsa_paged_decode",
    "dsa_paged_kv_append",
    "dsa_paged_kv_block_means",
    "dsa_paged_quantize_fp8",
    "dsa_paged_decode_fp8",
    "dsa_paged_kv_append_fp8",
    "dsa_paged_kv_block_means_fp8",
    "dsa_status_str",
    "dsa_last_error",
]


class Shape(ctypes.Structure):
    """Mirror of ``dsa_shape``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("topk_num", ctypes.c_int32),
        ("topk_den", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("select_mode", ctypes.c_int32),
        ("n_anchor", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("threshold", ctypes.c_float),
        ("k_min", ctypes.c_int32),
        ("k_max", ctypes.c_int32),
    ]

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // self.block)


def make_shape(batch, n_q_heads, n_kv_heads, seq_len, head_dim, block, topk=0, topk_num=0, topk_den=1,
               flags=FORCE_SINK | FORCE_DIAG, select_mode=SELECT_TOPK, n_anchor=0, window=0, threshold=0.0, k_min=0,
               k_max=0) -> Shape:
    return Shape(batch, n_q_heads, n_kv_heads, seq_len, head_dim, block, topk, topk_num, topk_den, flags, select_mode,
                 n_anchor, window, threshold, k_min, k_max)


class IndexShape(ctypes.Structure):
    """Mirror of ``dsa_index_shape``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("n_index_heads", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


def make_index_shape(batch, n_q_heads, n_kv_heads, seq_len, head_dim, n_index_heads, index_dim, topk,
                     flags=FORCE_SINK | FORCE_DIAG) -> IndexShape:
    return IndexShape(batch, n_q_heads, n_kv_heads, seq_len, head_dim, n_index_heads, index_dim, topk, flags)


class DsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libdsa status {code}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load libdsa.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m dynamic_block_sparse_dsa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I32, SZ = ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_size_t
    X = ctypes.POINTER(IndexShape)
    sig = {
        "dsa_kmax": ([S], ctypes.c_int32),
        "dsa_prefill_kmax": ([S, ctypes.POINTER(I32)], ctypes.c_int),
        "dsa_decode_kmax": ([S, ctypes.POINTER(I32)], ctypes.c_int),
        "dsa_block_means": ([S, I32, P, P, P], ctypes.c_int),
        "dsa_block_scores": ([S, P, P, P, P], ctypes.c_int),
        "dsa_block_scores_from_means": ([S, P, P, P, P], ctypes.c_int),
        "dsa_select_topk": ([S, P, P, P, P], ctypes.c_int),
        "dsa_indices_to_bitmap": ([P, P, ctypes.c_int64, I32, I32, P, P], ctypes.c_int),
        "dsa_check_block_selection": ([S, I32, P, P, P, P, P], ctypes.c_int),
        "dsa_check_token_selection": ([X, P, P, P, P], ctypes.c_int),
        "dsa_index_kmax": ([X, ctypes.POINTER(I32)], ctypes.c_int),
        "dsa_index_scores": ([X, P, P, P, P, P], ctypes.c_int),
        "dsa_select_tokens": ([X, P, P, P, P], ctypes.c_int),
        "dsa_token_attn_fwd": ([X, P, P, P, P, P, P, P, P], ctypes.c_int),
        "dsa_index_topk": ([X, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "dsa_index_workspace_bytes": ([X], SZ),
        "dsa_index_prefill": ([X, P, P, P, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "dsa_sparse_attn_fwd": ([S, P, P, P, P, P, P, P, P], ctypes.c_int),
        "dsa_prefill_workspace_bytes": ([S], SZ),
        "dsa_prefill": ([S, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "dsa_attn_bwd_workspace_bytes": ([S], SZ),
        "dsa_sparse_attn_bwd": ([S, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "dsa_kv_block_means": ([S, P, P, P], ctypes.c_int),
        "dsa_decode_workspace_bytes": ([S], SZ),
        "dsa_decode": ([S, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "dsa_decode_noalloc": ([S, P, P, P, P, P, P, P, P], ctypes.c_int),
        "dsa_paged_decode": ([S, P, P, P, P, I32, P, I32, P, P, P, P, P, P], ctypes.c_int),
        "dsa_paged_kv_append": ([S, P, P, P, I32, P, P, P, P, I32, P], ctypes.c_int),
        "dsa_paged_kv_block_means": ([S, P, P, I32, P, P, I32, P], ctypes.c_int),
        "dsa_paged_quantize_fp8": ([S, P, P, I32, P, P, P, P, P], ctypes.c_int),
        "dsa_paged_decode_fp8": ([S, P, P, P, P, P, P, I32, P, I32, P, P, P, P, P, P], ctypes.c_int),
        "dsa_paged_kv_append_fp8": ([S, P, P, P, I32, P, P, P, P, P, P, I32, P], ctypes.c_int),
        "dsa_paged_kv_block_means_fp8": ([S, P, P, P, I32, P, P, I32, P], ctypes.c_int),
        "dsa_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "dsa_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc: int):
    if rc != DSA_OK:
        lib = load()
        raise DsaError(rc, f"{lib.dsa_status_str(rc).decode()}: {lib.dsa_last_error().decode()}")


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def _ptr(t, dtype, shape, name, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _ws(ws, need):
    if need == 0:
        return None, 0
    if ws is None or ws.device.type != "cuda" or not ws.is_contiguous() or ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace must be a contiguous device tensor of at least {need} bytes")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def _key(shape: Shape):
    return tuple(getattr(shape, f) for f, _ in Shape._fields_)


# host-side queries depend only on the shape: cache them per shape
@functools.lru_cache(maxsize=256)
def _query(name: str, key):
    s = Shape(*key)
    lib = load()
    if name == "dsa_kmax":
        rc = int(lib.dsa_kmax(ctypes.byref(s)))
        _check(min(rc, 0))
        return rc
    if name.endswith("kmax"):
        out = ctypes.c_int32(0)
        _check(getattr(lib, name)(ctypes.byref(s), ctypes.byref(out)))
        return out.value
    return int(getattr(lib, name)(ctypes.byref(s)))


# ----------------------------------------------------------------- C ABI mirrors
def dsa_kmax(shape: Shape) -> int:
    """Index width (last dimension of idx) of a prefill or decode of this shape."""
    return _query("dsa_kmax", _key(shape))


def dsa_prefill_kmax(shape: Shape) -> int:
    return _query("dsa_prefill_kmax", _key(shape))


def dsa_decode_kmax(shape: Shape) -> int:
    return _query("dsa_decode_kmax", _key(shape))


def dsa_block_means(shape: Shape, n_heads: int, x, xbar, stream=None):
    B, N, d, nB = shape.batch, shape.seq_len, shape.head_dim, shape.n_blocks
    _check(load().dsa_block_means(ctypes.byref(shape), n_heads, _ptr(x, torch.bfloat16, (B, n_heads, N, d), "x"),
                                  _ptr(xbar, torch.float32, (B, n_heads, nB, d), "xbar"), _stream(stream)))


def dsa_block_scores(shape: Shape, q, k, scores, stream=None):
    B, Hq, Hkv, N, d, nB = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.seq_len, shape.head_dim, shape.n_blocks
    _check(load().dsa_block_scores(ctypes.byref(shape), _ptr(q, torch.bfloat16, (B, Hq, N, d), "q"),
                                   _ptr(k, torch.bfloat16, (B, Hkv, N, d), "k"),
                                   _ptr(scores, torch.float32, (B, Hkv, nB, nB), "scores"), _stream(stream)))


def dsa_block_scores_from_means(shape: Shape, qbar, kbar, scores, stream=None):
    B, Hq, Hkv, d, nB = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_blocks
    _check(load().dsa_block_scores_from_means(ctypes.byref(shape), _ptr(qbar, torch.float32, (B, Hq, nB, d), "qbar"),
                                              _ptr(kbar, torch.float32, (B, Hkv, nB, d), "kbar"),
                                              _ptr(scores, torch.float32, (B, Hkv, nB, nB), "scores"),
                                              _stream(stream)))


def dsa_select_topk(shape: Shape, scores, idx, cnt, stream=None):
    B, Hkv, nB = shape.batch, shape.n_kv_heads, shape.n_blocks
    km = dsa_prefill_kmax(shape)
    _check(load().dsa_select_topk(ctypes.byref(shape), _ptr(scores, torch.float32, (B, Hkv, nB, nB), "scores"),
                                  _ptr(idx, torch.int32, (B, Hkv, nB, km), "idx"),
                                  _ptr(cnt, torch.int32, (B, Hkv, nB), "cnt"), _stream(stream)))


def dsa_index_kmax(shape: IndexShape) -> int:
    out = ctypes.c_int32(0)
    _check(load().dsa_index_kmax(ctypes.byref(shape), ctypes.byref(out)))
    return out.value


def dsa_index_workspace_bytes(shape: IndexShape) -> int:
    return int(load().dsa_index_workspace_bytes(ctypes.byref(shape)))


def _index_dims(shape: IndexShape):
    return (shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.seq_len, shape.head_dim, shape.n_index_heads,
            shape.index_dim)


def dsa_index_scores(shape: IndexShape, qi, ki, wi, scores, stream=None):
    B, _, _, N, _, HI, dI = _index_dims(shape)
    _check(load().dsa_index_scores(ctypes.byref(shape), _ptr(qi, torch.bfloat16, (B, N, HI, dI), "qi"),
                                   _ptr(ki, torch.bfloat16, (B, N, dI), "ki"), _ptr(wi, torch.float32, (B, N, HI), "wi"),
                                   _ptr(scores, torch.float32, (B, N, N), "scores"), _stream(stream)))


def dsa_select_tokens(shape: IndexShape, scores, idx, cnt, stream=None):
    B, N = shape.batch, shape.seq_len
    km = dsa_index_kmax(shape)
    _check(load().dsa_select_tokens(ctypes.byref(shape), _ptr(scores, torch.float32, (B, N, N), "scores"),
                                    _ptr(idx, torch.int32, (B, N, km), "idx"), _ptr(cnt, torch.int32, (B, N), "cnt"),
                                    _stream(stream)))


def dsa_index_topk(shape: IndexShape, qi, ki, wi, idx, cnt, ws, stream=None):
    B, _, _, N, _, HI, dI = _index_dims(shape)
    km = dsa_index_kmax(shape)
    wp, wb = _ws(ws, dsa_index_workspace_bytes(shape))
    _check(load().dsa_index_topk(ctypes.byref(shape), _ptr(qi, torch.bfloat16, (B, N, HI, dI), "qi"),
                                 _ptr(ki, torch.bfloat16, (B, N, dI), "ki"), _ptr(wi, torch.float32, (B, N, HI), "wi"),
                                 _ptr(idx, torch.int32, (B, N, km), "idx"), _ptr(cnt, torch.int32, (B, N), "cnt"),
                                 wp, wb, _stream(stream)))


def dsa_token_attn_fwd(shape: IndexShape, q, k, v, idx, cnt, o, lse=None, stream=None):
    B, Hq, Hkv, N, d, _, _ = _index_dims(shape)
    km = dsa_index_kmax(shape)
    _check(load().dsa_token_attn_fwd(
        ctypes.byref(shape), _ptr(q, torch.bfloat16, (B, Hq, N, d), "q"), _ptr(k, torch.bfloat16, (B, Hkv, N, d), "k"),
        _ptr(v, torch.bfloat16, (B, Hkv, N, d), "v"), _ptr(idx, torch.int32, (B, N, km), "idx"),
        _ptr(cnt, torch.int32, (B, N), "cnt"), _ptr(o, torch.bfloat16, (B, Hq, N, d), "o"),
        _ptr(lse, torch.float32, (B, Hq, N), "lse", optional=True), _stream(stream)))


def dsa_index_prefill(shape: IndexShape, qi, ki, wi, q, k, v, o, lse, idx, cnt, ws, stream=None):
    B, Hq, Hkv, N, d, HI, dI = _index_dims(shape)
    km = dsa_index_kmax(shape)
    wp, wb = _ws(ws, dsa_index_workspace_bytes(shape))
    _check(load().dsa_index_prefill(
        ctypes.byref(shape), _ptr(qi, torch.bfloat16, (B, N, HI, dI), "qi"), _ptr(ki, torch.bfloat16, (B, N, dI), "ki"),
        _ptr(wi, torch.float32, (B, N, HI), "wi"), _ptr(q, torch.bfloat16, (B, Hq, N, d), "q"),
        _ptr(k, torch.bfloat16, (B, Hkv, N, d), "k"), _ptr(v, torch.bfloat16, (B, Hkv, N, d), "v"),
        _ptr(o, torch.bfloat16, (B, Hq, N, d), "o"), _ptr(lse, torch.float32, (B, Hq, N), "lse", optional=True),
        _ptr(idx, torch.int32, (B, N, km), "idx"), _ptr(cnt, torch.int32, (B, N), "cnt"), wp, wb, _stream(stream)))


def dsa_indices_to_bitmap(idx, cnt, n_cols: int, bitmap, stream=None):
    """idx [..., kmax] int32, cnt [...] int32 or None; bitmap [..., ceil(n_cols/32)]
    int32 (the uint32 words' bits)."""
    if not isinstance(idx, torch.Tensor):
        raise TypeError("idx must be a torch tensor")
    lead, km = tuple(idx.shape[:-1]), int(idx.shape[-1])
    n_rows = math.prod(lead)
    _check(load().dsa_indices_to_bitmap(
        _ptr(idx, torch.int32, lead + (km,), "idx"), _ptr(cnt, torch.int32, lead, "cnt", optional=True), n_rows, km,
        n_cols, _ptr(bitmap, torch.int32, lead + ((n_cols + 31) // 32,), "bitmap"), _stream(stream)))


def dsa_check_block_selection(shape: Shape, layout: int, idx, cnt, lengths, report, stream=None):
    """Selection validator (counts into report [6] int64); layouts LAYOUT_*."""
    B, Hkv = shape.batch, shape.n_kv_heads
    nB = -(-shape.seq_len // shape.block)
    if layout == LAYOUT_PREFILL:
        lead, km = (B, Hkv, nB), dsa_prefill_kmax(shape)
    else:
        lead, km = (B, Hkv), dsa_decode_kmax(shape)
    _check(load().dsa_check_block_selection(
        ctypes.byref(shape), layout, _ptr(idx, torch.int32, lead + (km,), "idx"),
        _ptr(cnt, torch.int32, lead, "cnt", optional=True),
        _ptr(lengths, torch.int32, (B,), "lengths", optional=True),
        _ptr(report, torch.int64, (len(CHECK_SLOTS),), "report"), _stream(stream)))


def dsa_check_token_selection(shape: IndexShape, idx, cnt, report, stream=None):
    B, N = shape.batch, shape.seq_len
    _check(load().dsa_check_token_selection(
        ctypes.byref(shape), _ptr(idx, torch.int32, (B, N, dsa_index_kmax(shape)), "idx"),
        _ptr(cnt, torch.int32, (B, N), "cnt", optional=True),
        _ptr(report, torch.int64, (len(CHECK_SLOTS),), "report"), _stream(stream)))


def dsa_sparse_attn_fwd(shape: Shape, q, k, v, idx, cnt, o, lse=None, stream=None):
    B, Hq, Hkv, N, d, nB = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.seq_len, shape.head_dim, shape.n_blocks
    km = dsa_prefill_kmax(shape)
    _check(load().dsa_sparse_attn_fwd(
        ctypes.byref(shape), _ptr(q, torch.bfloat16, (B, Hq, N, d), "q"), _ptr(k, torch.bfloat16, (B, Hkv, N, d), "k"),
        _ptr(v, torch.bfloat16, (B, Hkv, N, d), "v"), _ptr(idx, torch.int32, (B, Hkv, nB, km), "idx"),
        _ptr(cnt, torch.int32, (B, Hkv, nB), "cnt"), _ptr(o, torch.bfloat16, (B, Hq, N, d), "o"),
        _ptr(lse, torch.float32, (B, Hq, N), "lse", optional=True), _stream(stream)))


def dsa_prefill_workspace_bytes(shape: Shape) -> int:
    return _query("dsa_prefill_workspace_bytes", _key(shape))


def dsa_prefill(shape: Shape, q, k, v, o, lse, idx, cnt, ws, stream=None):
    B, Hq, Hkv, N, d, nB = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.seq_len, shape.head_dim, shape.n_blocks
    km = dsa_prefill_kmax(shape)
    wp, wb = _ws(ws, dsa_prefill_workspace_bytes(shape))
    _check(load().dsa_prefill(
        ctypes.byref(shape), _ptr(q, torch.bfloat16, (B, Hq, N, d), "q"), _ptr(k, torch.bfloat16, (B, Hkv, N, d), "k"),
        _ptr(v, torch.bfloat16, (B, Hkv, N, d), "v"), _ptr(o, torch.bfloat16, (B, Hq, N, d), "o"),
        _ptr(lse, torch.float32, (B, Hq, N), "lse", optional=True), _ptr(idx, torch.int32, (B, Hkv, nB, km), "idx"),
        _ptr(cnt, torch.int32, (B, Hkv, nB), "cnt"), wp, wb, _stream(stream)))


def dsa_attn_bwd_workspace_bytes(shape: Shape) -> int:
    return _query("dsa_attn_bwd_workspace_bytes", _key(shape))


def dsa_sparse_attn_bwd(shape: Shape, q, k, v, o, lse, dout, idx, cnt, dq, dk, dv, ws, stream=None):
    B, Hq, Hkv, N, d, nB = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.seq_len, shape.head_dim, shape.n_blocks
    km = dsa_prefill_kmax(shape)
    wp, wb = _ws(ws, dsa_attn_bwd_workspace_bytes(shape))
    _check(load().dsa_sparse_attn_bwd(
        ctypes.byref(shape), _ptr(q, torch.bfloat16, (B, Hq, N, d), "q"), _ptr(k, torch.bfloat16, (B, Hkv, N, d), "k"),
        _ptr(v, torch.bfloat16, (B, Hkv, N, d), "v"), _ptr(o, torch.bfloat16, (B, Hq, N, d), "o"),
        _ptr(lse, torch.float32, (B, Hq, N), "lse"), _ptr(dout, torch.bfloat16, (B, Hq, N, d), "dout"),
        _ptr(idx, torch.int32, (B, Hkv, nB, km), "idx"), _ptr(cnt, torch.int32, (B, Hkv, nB), "cnt"),
        _ptr(dq, torch.bfloat16, (B, Hq, N, d), "dq"), _ptr(dk, torch.bfloat16, (B, Hkv, N, d), "dk"),
        _ptr(dv, torch.bfloat16, (B, Hkv, N, d), "dv"), wp, wb, _stream(stream)))


def dsa_kv_block_means(shape: Shape, k_cache, kbar, stream=None):
    S, Hkv, L, d, nB = shape.batch, shape.n_kv_heads, shape.seq_len, shape.head_dim, shape.n_blocks
    _check(load().dsa_kv_block_means(ctypes.byref(shape), _ptr(k_cache, torch.bfloat16, (S, Hkv, L, d), "k_cache"),
                                     _ptr(kbar, torch.float32, (S, Hkv, nB, d), "kbar"), _stream(stream)))


def dsa_decode_workspace_bytes(shape: Shape) -> int:
    return _query("dsa_decode_workspace_bytes", _key(shape))


def dsa_decode(shape: Shape, q, k_cache, v_cache, kbar, o, lse, idx, ws, stream=None):
    S, Hq, Hkv, L, d, nB = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.seq_len, shape.head_dim, shape.n_blocks
    km = dsa_decode_kmax(shape)
    wp, wb = _ws(ws, dsa_decode_workspace_bytes(shape))
    _check(load().dsa_decode(
        ctypes.byref(shape), _ptr(q, torch.bfloat16, (S, Hq, d), "q"),
        _ptr(k_cache, torch.bfloat16, (S, Hkv, L, d), "k_cache"),
        _ptr(v_cache, torch.bfloat16, (S, Hkv, L, d), "v_cache"), _ptr(kbar, torch.float32, (S, Hkv, nB, d), "kbar"),
        _ptr(o, torch.bfloat16, (S, Hq, d), "o"), _ptr(lse, torch.float32, (S, Hq), "lse", optional=True),
        _ptr(idx, torch.int32, (S, Hkv, km), "idx"), wp, wb, _stream(stream)))


def dsa_decode_noalloc(shape: Shape, q, k_cache, v_cache, kbar, o, lse, idx, stream=None):
    S, Hq, Hkv, L, d, nB = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.seq_len, shape.head_dim, shape.n_blocks
    km = dsa_decode_kmax(shape)
    _check(load().dsa_decode_noalloc(
        ctypes.byref(shape), _ptr(q, torch.bfloat16, (S, Hq, d), "q"),
        _ptr(k_cache, torch.bfloat16, (S, Hkv, L, d), "k_cache"),
        _ptr(v_cache, torch.bfloat16, (S, Hkv, L, d), "v_cache"), _ptr(kbar, torch.float32, (S, Hkv, nB, d), "kbar"),
        _ptr(o, torch.bfloat16, (S, Hq, d), "o"), _ptr(lse, torch.float32, (S, Hq), "lse", optional=True),
        _ptr(idx, torch.int32, (S, Hkv, km), "idx"), _stream(stream)))


def _paged_dims(shape: Shape, k_pool, table):
    n_pages = int(k_pool.shape[0])
    return n_pages, int(table.shape[1])


def dsa_paged_decode(shape: Shape, q, k_pool, v_pool, kbar_pool, block_table, lengths, o, lse, idx, cnt=None,
                     stream=None):
    S, Hq, Hkv, d, b = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.block
    n_pages, mb = _paged_dims(shape, k_pool, block_table)
    km = dsa_decode_kmax(shape)
    _check(load().dsa_paged_decode(
        ctypes.byref(shape), _ptr(q, torch.bfloat16, (S, Hq, d), "q"),
        _ptr(k_pool, torch.bfloat16, (n_pages, Hkv, b, d), "k_pool"),
        _ptr(v_pool, torch.bfloat16, (n_pages, Hkv, b, d), "v_pool"),
        _ptr(kbar_pool, torch.float32, (n_pages, Hkv, d), "kbar_pool"), n_pages,
        _ptr(block_table, torch.int32, (S, mb), "block_table"), mb, _ptr(lengths, torch.int32, (S,), "lengths"),
        _ptr(o, torch.bfloat16, (S, Hq, d), "o"), _ptr(lse, torch.float32, (S, Hq), "lse", optional=True),
        _ptr(idx, torch.int32, (S, Hkv, km), "idx"), _ptr(cnt, torch.int32, (S, Hkv), "cnt", optional=True),
        _stream(stream)))


def dsa_paged_kv_append(shape: Shape, k_new, v_new, block_table, lengths, k_pool, v_pool, kbar_pool, stream=None):
    S, Hkv, d, b = shape.batch, shape.n_kv_heads, shape.head_dim, shape.block
    n_pages, mb = _paged_dims(shape, k_pool, block_table)
    _check(load().dsa_paged_kv_append(
        ctypes.byref(shape), _ptr(k_new, torch.bfloat16, (S, Hkv, d), "k_new"),
        _ptr(v_new, torch.bfloat16, (S, Hkv, d), "v_new"), _ptr(block_table, torch.int32, (S, mb), "block_table"), mb,
        _ptr(lengths, torch.int32, (S,), "lengths"), _ptr(k_pool, torch.bfloat16, (n_pages, Hkv, b, d), "k_pool"),
        _ptr(v_pool, torch.bfloat16, (n_pages, Hkv, b, d), "v_pool"),
        _ptr(kbar_pool, torch.float32, (n_pages, Hkv, d), "kbar_pool"), n_pages, _stream(stream)))


def dsa_paged_kv_block_means(shape: Shape, k_pool, block_table, lengths, kbar_pool, stream=None):
    S, Hkv, d, b = shape.batch, shape.n_kv_heads, shape.head_dim, shape.block
    n_pages, mb = _paged_dims(shape, k_pool, block_table)
    _check(load().dsa_paged_kv_block_means(
        ctypes.byref(shape), _ptr(k_pool, torch.bfloat16, (n_pages, Hkv, b, d), "k_pool"),
        _ptr(block_table, torch.int32, (S, mb), "block_table"), mb, _ptr(lengths, torch.int32, (S,), "lengths"),
        _ptr(kbar_pool, torch.float32, (n_pages, Hkv, d), "kbar_pool"), n_pages, _stream(stream)))


def _fp8_pools(shape: Shape, k8, v8, k_scale, v_scale):
    n_pages = int(k8.shape[0])
    Hkv, d, b = shape.n_kv_heads, shape.head_dim, shape.block
    return n_pages, [_ptr(k8, torch.uint8, (n_pages, Hkv, b, d), "k8"), _ptr(v8, torch.uint8, (n_pages, Hkv, b, d), "v8"),
                     _ptr(k_scale, torch.float32, (n_pages, Hkv, b), "k_scale"),
                     _ptr(v_scale, torch.float32, (n_pages, Hkv, b), "v_scale")]


def dsa_paged_quantize_fp8(shape: Shape, k_pool, v_pool, k8, v8, k_scale, v_scale, stream=None):
    Hkv, d, b = shape.n_kv_heads, shape.head_dim, shape.block
    n_pages, ptrs = _fp8_pools(shape, k8, v8, k_scale, v_scale)
    _check(load().dsa_paged_quantize_fp8(
        ctypes.byref(shape), _ptr(k_pool, torch.bfloat16, (n_pages, Hkv, b, d), "k_pool"),
        _ptr(v_pool, torch.bfloat16, (n_pages, Hkv, b, d), "v_pool"), n_pages, *ptrs, _stream(stream)))


def dsa_paged_decode_fp8(shape: Shape, q, k8, v8, k_scale, v_scale, kbar_pool, block_table, lengths, o, lse, idx,
                         cnt=None, stream=None):
    S, Hq, Hkv, d = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    n_pages, ptrs = _fp8_pools(shape, k8, v8, k_scale, v_scale)
    mb = int(block_table.shape[1])
    km = dsa_decode_kmax(shape)
    _check(load().dsa_paged_decode_fp8(
        ctypes.byref(shape), _ptr(q, torch.bfloat16, (S, Hq, d), "q"), *ptrs,
        _ptr(kbar_pool, torch.float32, (n_pages, Hkv, d), "kbar_pool"), n_pages,
        _ptr(block_table, torch.int32, (S, mb), "block_table"), mb, _ptr(lengths, torch.int32, (S,), "lengths"),
        _ptr(o, torch.bfloat16, (S, Hq, d), "o"), _ptr(lse, torch.float32, (S, Hq), "lse", optional=True),
        _ptr(idx, torch.int32, (S, Hkv, km), "idx"), _ptr(cnt, torch.int32, (S, Hkv), "cnt", optional=True),
        _stream(stream)))


def dsa_paged_kv_append_fp8(shape: Shape, k_new, v_new, block_table, lengths, k8, v8, k_scale, v_scale, kbar_pool,
                            stream=None):
    S, Hkv, d = shape.batch, shape.n_kv_heads, shape.head_dim
    n_pages, ptrs = _fp8_pools(shape, k8, v8, k_scale, v_scale)
    mb = int(block_table.shape[1])
    _check(load().dsa_paged_kv_append_fp8(
        ctypes.byref(shape), _ptr(k_new, torch.bfloat16, (S, Hkv, d), "k_new"),
        _ptr(v_new, torch.bfloat16, (S, Hkv, d), "v_new"), _ptr(block_table, torch.int32, (S, mb), "block_table"), mb,
        _ptr(lengths, torch.int32, (S,), "lengths"), *ptrs,
        _ptr(kbar_pool, torch.float32, (n_pages, Hkv, d), "kbar_pool"), n_pages, _stream(stream)))


def dsa_paged_kv_block_means_fp8(shape: Shape, k8, k_scale, block_table, lengths, kbar_pool, stream=None):
    S, Hkv, d, b = shape.batch, shape.n_kv_heads, shape.head_dim, shape.block
    n_pages = int(k8.shape[0])
    mb = int(block_table.shape[1])
    _check(load().dsa_paged_kv_block_means_fp8(
        ctypes.byref(shape), _ptr(k8, torch.uint8, (n_pages, Hkv, b, d), "k8"),
        _ptr(k_scale, torch.float32, (n_pages, Hkv, b), "k_scale"),
        _ptr(block_table, torch.int32, (S, mb), "block_table"), mb, _ptr(lengths, torch.int32, (S,), "lengths"),
        _ptr(kbar_pool, torch.float32, (n_pages, Hkv, d), "kbar_pool"), n_pages, _stream(stream)))


# ----------------------------------------------------------------- conveniences
def prefill(q, k, v, block: int, topk: int = 0, topk_num: int = 0, topk_den: int = 1,
            flags: int = FORCE_SINK | FORCE_DIAG, want_lse: bool = True, stream=None, **select):
    """Fused prefill; allocates O, LSE, idx, cnt and the workspace.  ``select``:
    select_mode, n_anchor, window, threshold, k_min, k_max (see make_shape)."""
    B, Hq, N, d = q.shape
    shape = make_shape(B, Hq, k.shape[1], N, d, block, topk, topk_num, topk_den, flags, **select)
    km = dsa_prefill_kmax(shape)
    dev = q.device
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if want_lse else None
    idx = torch.empty((B, k.shape[1], shape.n_blocks, km), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, k.shape[1], shape.n_blocks), dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, dsa_prefill_workspace_bytes(shape)), dtype=torch.uint8, device=dev)
    dsa_prefill(shape, q, k, v, o, lse, idx, cnt, ws, stream)
    return o, lse, idx, cnt


def attn_backward(q, k, v, o, lse, dout, idx, cnt, block: int, topk: int = 0, topk_num: int = 0, topk_den: int = 1,
                  flags: int = FORCE_SINK | FORCE_DIAG, stream=None, **select):
    """Gradients of the sparse attention (selection held fixed); allocates
    dq, dk, dv and the workspace.  idx/cnt/o/lse as returned by prefill
    (with the same selection arguments)."""
    B, Hq, N, d = q.shape
    shape = make_shape(B, Hq, k.shape[1], N, d, block, topk, topk_num, topk_den, flags, **select)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(1, dsa_attn_bwd_workspace_bytes(shape)), dtype=torch.uint8, device=q.device)
    dsa_sparse_attn_bwd(shape, q, k, v, o, lse, dout, idx, cnt, dq, dk, dv, ws, stream)
    return dq, dk, dv


def decode(q, k_cache, v_cache, kbar, block: int, topk: int = 0, topk_num: int = 0, topk_den: int = 1,
           flags: int = FORCE_SINK | FORCE_DIAG, want_lse: bool = True, stream=None, n_anchor: int = 0,
           window: int = 0):
    """One decode step; allocates o, lse, idx and the workspace."""
    S, Hq, d = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    shape = make_shape(S, Hq, Hkv, L, d, block, topk, topk_num, topk_den, flags, n_anchor=n_anchor, window=window)
    km = dsa_decode_kmax(shape)
    dev = q.device
    o = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev) if want_lse else None
    idx = torch.empty((S, Hkv, km), dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, dsa_decode_workspace_bytes(shape)), dtype=torch.uint8, device=dev)
    dsa_decode(shape, q, k_cache, v_cache, kbar, o, lse, idx, ws, stream)
    return o, lse, idx


def bitmap(idx, cnt, n_cols: int, stream=None):
    """Selection rows as bit words (int32 storage of uint32 words)."""
    out = torch.empty(tuple(idx.shape[:-1]) + ((n_cols + 31) // 32,), dtype=torch.int32, device=idx.device)
    dsa_indices_to_bitmap(idx, cnt, n_cols, out, stream)
    return out


def check_selection(shape, idx, cnt=None, lengths=None, layout: int = LAYOUT_PREFILL, stream=None) -> dict:
    """Run the selection validator and return its report as a dict (waits for
    the validator to read it).  shape: a Shape (block selection, `layout`) or an
    IndexShape (token selection)."""
    report = torch.empty(len(CHECK_SLOTS), dtype=torch.int64, device=idx.device)
    if isinstance(shape, IndexShape):
        dsa_check_token_selection(shape, idx, cnt, report, stream)
    else:
        dsa_check_block_selection(shape, layout, idx, cnt, lengths, report, stream)
    if stream is not None:
        torch.cuda.synchronize(idx.device)
    return dict(zip(CHECK_SLOTS, report.tolist()))


def index_prefill(qi, ki, wi, q, k, v, topk: int, flags: int = FORCE_SINK | FORCE_DIAG, want_lse: bool = True,
                  stream=None):
    """Token-level indexer -> token selection -> token-gather attention;
    allocates O, LSE, idx, cnt and the workspace."""
    B, N, HI, dI = qi.shape
    shape = make_index_shape(B, q.shape[1], k.shape[1], N, q.shape[3], HI, dI, topk, flags)
    km = dsa_index_kmax(shape)
    dev = q.device
    o = torch.empty_like(q)
    lse = torch.empty((B, q.shape[1], N), dtype=torch.float32, device=dev) if want_lse else None
    idx = torch.empty((B, N, km), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, N), dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, dsa_index_workspace_bytes(shape)), dtype=torch.uint8, device=dev)
    dsa_index_prefill(shape, qi, ki, wi, q, k, v, o, lse, idx, cnt, ws, stream)
    return o, lse, idx, cnt


def paged_decode(q, k_pool, v_pool, kbar_pool, block_table, lengths, block: int, topk: int = 0, topk_num: int = 0,
                 topk_den: int = 1, flags: int = FORCE_SINK | FORCE_DIAG, n_anchor: int = 0, window: int = 0,
                 want_lse: bool = True, stream=None):
    """One decode step over a paged cache (a length per sequence); allocates
    o, lse, idx and cnt."""
    S, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    mb = block_table.shape[1]
    shape = make_shape(S, Hq, Hkv, mb * block, d, block, topk, topk_num, topk_den, flags, n_anchor=n_anchor,
                       window=window)
    km = dsa_decode_kmax(shape)
    dev = q.device
    o = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev) if want_lse else None
    idx = torch.empty((S, Hkv, km), dtype=torch.int32, device=dev)
    cnt = torch.empty((S, Hkv), dtype=torch.int32, device=dev)
    dsa_paged_decode(shape, q, k_pool, v_pool, kbar_pool, block_table, lengths, o, lse, idx, cnt, stream)
    return o, lse, idx, cnt


def paged_shape(k_pool, block_table, n_q_heads: int, batch: int | None = None) -> Shape:
    """A shape for the paged cache calls that need no selection parameters."""
    n_pages, Hkv, b, d = k_pool.shape
    S = block_table.shape[0] if batch is None else batch
    return make_shape(S, n_q_heads, Hkv, block_table.shape[1] * b, d, b, 1)


def kv_block_means(k_cache, block: int, stream=None):
    S, Hkv, L, d = k_cache.shape
    shape = make_shape(S, Hkv, Hkv, L, d, block, 1)
    kbar = torch.empty((S, Hkv, shape.n_blocks, d), dtype=torch.float32, device=k_cache.device)
    dsa_kv_block_means(shape, k_cache, kbar, stream)
    return kbar
