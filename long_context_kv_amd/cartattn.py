"""ctypes binding of libcartattn (the C ABI declared in include/cartattn.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and sizes to the library and
raises ``CartError`` on a non-zero status. All arithmetic runs in the HIP
kernels of libcartattn.so; PyTorch only provides device memory and the
current stream. The library is loaded from this package's directory and the
import fails loudly if it is missing: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import pathlib
from typing import Optional

import torch

_HERE = pathlib.Path(__file__).resolve().parent
LIB_PATH = pathlib.Path(os.environ.get("CARTATTN_LIB", _HERE / "libcartattn.so"))

if not LIB_PATH.exists():
    raise ImportError(
        f"{LIB_PATH} not found: build it with `python -m long_context_kv_amd.build`")

_lib = ctypes.CDLL(str(LIB_PATH))

CART_OK = 0
CART_ERR_INVALID_ARG = 1
CART_ERR_UNSUPPORTED = 2
CART_ERR_ALIGNMENT = 3
CART_ERR_WORKSPACE = 4
CART_ERR_CACHE_NOT_EMPTY = 5
CART_ERR_CACHE_FULL = 6
CART_ERR_GEOMETRY = 7
CART_ERR_HIP = 8

CART_F32 = 0
CART_BF16 = 1

_DTYPES = {torch.float32: CART_F32, torch.bfloat16: CART_BF16}

EXPORTS = [
    "cart_rope_tokens", "cart_rope_tokens_packed", "cart_qk_norm_rope", "cart_qk_norm_rope_bwd", "cart_adam_rows",
    "cart_rows_to_bf16",
    "cart_attn_workspace_size", "cart_parts_rows", "cart_compose_rows",
    "cart_attn_bwd_composed", "cart_write_composed_cache", "cart_attn_fwd", "cart_attn_bwd",
    "cart_cache_create", "cart_cache_destroy", "cart_cache_reset", "cart_cache_seq_len",
    "cart_append_cache", "cart_write_cache", "cart_decode", "cart_decode_workspace_size",
    "cart_decode_verify", "cart_decode_verify_workspace_size", "cart_cache_truncate",
    "cart_decode_noalloc", "cart_decode_noalloc_max_bytes", "cart_attn_schedule_query",
    "cart_decode_schedule_query",
    "cart_timing_enable", "cart_timing_only", "cart_timing_query", "cart_status_string", "cart_last_error",
]


class AttnShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_seq", ctypes.c_int32), ("p", ctypes.c_int32),
        ("frozen_rows", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("scale", ctypes.c_float), ("tok_dtype", ctypes.c_int), ("row_dtype", ctypes.c_int),
        ("window", ctypes.c_int32), ("seg_lens", ctypes.POINTER(ctypes.c_int32)),
    ]


class AttnSchedule(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "fwd_grid", "fwd_key_splits", "bwd_cart_tiles", "bwd_tok_tiles", "bwd_units_per_piece",
        "bwd_cart_pieces", "bwd_tok_pieces_max", "bwd_kv_grid", "bwd_dq_grid",
        "bwd_dq_key_splits", "bwd_tok_units_per_piece")]


class DecodeSchedule(ctypes.Structure):
    _fields_ = [("pages_per_split", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("waves_per_group", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("n_pages", ctypes.c_int32),
        ("dtype", ctypes.c_int), ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
    ]


class Parts(ctypes.Structure):
    _fields_ = [("n_parts", ctypes.c_int32), ("rows", ctypes.POINTER(ctypes.c_int32)),
                ("frozen", ctypes.POINTER(ctypes.c_int32)),
                ("k", ctypes.POINTER(ctypes.c_void_p)), ("v", ctypes.POINTER(ctypes.c_void_p))]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_P = ctypes.POINTER

_lib.cart_rope_tokens.argtypes = [_vp, _vp, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _i32,
                                  _vp, ctypes.c_double, _i32, _vp]
_lib.cart_rope_tokens_packed.argtypes = [_vp, _vp, ctypes.c_int, _i32, _P(_i32), _i32, _i32, _i32,
                                         _i32, ctypes.c_double, _i32, _vp]
_lib.cart_qk_norm_rope.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32,
                                   _i32, _i32, ctypes.c_float, _i32, _vp, ctypes.c_double, _vp]
_lib.cart_qk_norm_rope_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i32,
                                       _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _vp,
                                       ctypes.c_double, _vp]
_lib.cart_adam_rows.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int64, _i32, _i32, _i32,
                                ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                ctypes.c_double, _vp]
_lib.cart_rows_to_bf16.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int64, _i32, _vp]
_lib.cart_attn_workspace_size.argtypes = [_P(AttnShape), _i32]
_lib.cart_parts_rows.argtypes = [_P(Parts)]
_lib.cart_parts_rows.restype = _i32
_lib.cart_compose_rows.argtypes = [_P(Parts), ctypes.c_int, _i32, _i32, _vp, _vp, ctypes.c_int, _vp]
_lib.cart_attn_bwd_composed.argtypes = [_P(AttnShape), _P(Parts), _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]
_lib.cart_write_composed_cache.argtypes = [_vp, _i32, _P(Parts), ctypes.c_int, _i32, _i32, _vp]
_lib.cart_attn_workspace_size.restype = _sz
_lib.cart_attn_fwd.argtypes = [_P(AttnShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.cart_attn_bwd.argtypes = [_P(AttnShape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]
_lib.cart_cache_create.argtypes = [_P(CacheDesc), _P(_vp)]
_lib.cart_cache_destroy.argtypes = [_vp]
_lib.cart_cache_reset.argtypes = [_vp, _i32, _vp]
_lib.cart_cache_seq_len.argtypes = [_vp, _i32]
_lib.cart_cache_seq_len.restype = _i32
_lib.cart_append_cache.argtypes = [_vp, _i32, _vp, _vp, ctypes.c_int, _i32, _i32, _i32, _vp]
_lib.cart_write_cache.argtypes = [_vp, _i32, _vp, _vp, ctypes.c_int, _i32, _i32, _i32, _vp]
_lib.cart_decode.argtypes = [_vp, _vp, _vp, _vp, _i32, ctypes.c_float, _vp, _vp, _sz, _vp]
_lib.cart_decode_workspace_size.argtypes = [_vp, _i32]
_lib.cart_decode_workspace_size.restype = _sz
_lib.cart_decode_verify.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, ctypes.c_float, _vp, _vp, _sz,
                                    _vp]
_lib.cart_decode_verify_workspace_size.argtypes = [_vp, _i32, _i32]
_lib.cart_decode_verify_workspace_size.restype = _sz
_lib.cart_cache_truncate.argtypes = [_vp, _i32, _i32, _vp]
_lib.cart_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i32, ctypes.c_float, _vp, _vp]
_lib.cart_decode_noalloc_max_bytes.argtypes = []
_lib.cart_decode_noalloc_max_bytes.restype = _sz
_lib.cart_attn_schedule_query.argtypes = [_P(AttnShape), _P(AttnSchedule)]
_lib.cart_decode_schedule_query.argtypes = [_vp, _i32, _i32, _P(DecodeSchedule)]
_lib.cart_timing_enable.argtypes = [_i32]
_lib.cart_timing_only.argtypes = [ctypes.c_char_p]
_lib.cart_timing_query.argtypes = [ctypes.c_char_p, _P(ctypes.c_double), _P(_i32)]
_lib.cart_status_string.argtypes = [ctypes.c_int]
_lib.cart_status_string.restype = ctypes.c_char_p
_lib.cart_last_error.argtypes = []
_lib.cart_last_error.restype = ctypes.c_char_p


class CartError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.cart_last_error().decode()
        super().__init__(f"{where}: {_lib.cart_status_string(status).decode()} "
                         f"(status {status}): {msg}")


def _check(status: int, where: str) -> None:
    if status != CART_OK:
        raise CartError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        if not torch.cuda.is_available():
            return ctypes.c_void_p(0)
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def attn_shape(q: torch.Tensor, k_tok: torch.Tensor, p: int, frozen_rows: int = 1,
               scale: float = 0.0, row_dtype: Optional[torch.dtype] = None,
               window: int = 0, seg_lens=None) -> AttnShape:
    """Shape struct from Q [B, n, Hq, d] and token K [B, n, Hkv, d], or, for
    packed segments (seg_lens: their lengths), Q [T, Hq, d] and K [T, Hkv, d].
    A packed shape keeps its length array alive as an attribute."""
    rd = _DTYPES[row_dtype] if row_dtype is not None else _dt(q)
    if seg_lens is None:
        B, n, Hq, d = q.shape
        Hkv = k_tok.shape[2]
        return AttnShape(B, n, p, frozen_rows, Hq, Hkv, d, scale, _dt(q), rd, window, None)
    T, Hq, d = q.shape
    Hkv = k_tok.shape[1]
    lens = (ctypes.c_int32 * len(seg_lens))(*[int(x) for x in seg_lens])
    s = AttnShape(len(seg_lens), max(seg_lens), p, frozen_rows, Hq, Hkv, d, scale, _dt(q), rd,
                  window, lens)
    s._lens = lens
    return s


# ---------------------------------------------------------------- raw calls

def cart_rope_tokens(q: torch.Tensor, k: Optional[torch.Tensor], pos_base: int,
                     pos_offsets: Optional[torch.Tensor] = None, theta: float = 1.0e6,
                     inverse: bool = False, stream=None) -> None:
    """Rotate q [B, S, Hq, d] (and k [B, S, Hkv, d]) in place."""
    B, S, Hq, d = q.shape
    Hkv = k.shape[2] if k is not None else 0
    _check(_lib.cart_rope_tokens(_ptr(q), _ptr(k), _dt(q), B, S, Hq, Hkv, d, pos_base,
                                 _ptr(pos_offsets), theta, int(inverse), _stream(stream)),
           "cart_rope_tokens")


def cart_rope_tokens_packed(q: torch.Tensor, k: Optional[torch.Tensor], seg_lens, pos_base: int,
                            theta: float = 1.0e6, inverse: bool = False, stream=None) -> None:
    """Rotate packed q [T, Hq, d] (and k [T, Hkv, d]) in place; positions
    restart at pos_base in every segment."""
    T, Hq, d = q.shape
    Hkv = k.shape[1] if k is not None else 0
    lens = (ctypes.c_int32 * len(seg_lens))(*[int(x) for x in seg_lens])
    _check(_lib.cart_rope_tokens_packed(_ptr(q), _ptr(k), _dt(q), len(seg_lens), lens, Hq, Hkv, d,
                                        pos_base, theta, int(inverse), _stream(stream)),
           "cart_rope_tokens_packed")


def cart_qk_norm_rope(q_in: torch.Tensor, k_in: Optional[torch.Tensor], q_out: torch.Tensor,
                      k_out: Optional[torch.Tensor], w_q: torch.Tensor,
                      w_k: Optional[torch.Tensor], pos_base: int, eps: float = 1e-6,
                      pos_offsets: Optional[torch.Tensor] = None, theta: float = 1.0e6,
                      stream=None) -> None:
    """q_out/k_out = RoPE(RMSNorm(q_in/k_in)) (may be in place)."""
    B, S, Hq, d = q_in.shape
    Hkv = k_in.shape[2] if k_in is not None else 0
    _check(_lib.cart_qk_norm_rope(_ptr(q_in), _ptr(k_in), _ptr(q_out), _ptr(k_out), _ptr(w_q),
                                  _ptr(w_k), _dt(q_in), B, S, Hq, Hkv, d, eps, pos_base,
                                  _ptr(pos_offsets), theta, _stream(stream)),
           "cart_qk_norm_rope")


def cart_qk_norm_rope_bwd(q_in, k_in, dq_out, dk_out, dq_in, dk_in, w_q, w_k, pos_base: int,
                          eps: float = 1e-6, pos_offsets=None, theta: float = 1.0e6,
                          stream=None) -> None:
    """dq_in/dk_in = input gradients of cart_qk_norm_rope."""
    B, S, Hq, d = q_in.shape
    Hkv = k_in.shape[2] if k_in is not None else 0
    _check(_lib.cart_qk_norm_rope_bwd(_ptr(q_in), _ptr(k_in), _ptr(dq_out), _ptr(dk_out),
                                      _ptr(dq_in), _ptr(dk_in), _ptr(w_q), _ptr(w_k), _dt(q_in),
                                      B, S, Hq, Hkv, d, eps, pos_base, _ptr(pos_offsets), theta,
                                      _stream(stream)),
           "cart_qk_norm_rope_bwd")


def cart_adam_rows(rows: torch.Tensor, grad: torch.Tensor, m: torch.Tensor, v: torch.Tensor,
                   step: int, lr: float, frozen_rows: int = 1, beta1: float = 0.9,
                   beta2: float = 0.999, eps: float = 1e-8,
                   rows_bf16: Optional[torch.Tensor] = None, stream=None) -> None:
    """One Adam step on f32 rows [n_rows, ...] (rows below frozen_rows kept)."""
    n_rows = rows.shape[0]
    row_elems = rows.numel() // max(n_rows, 1)
    _check(_lib.cart_adam_rows(_ptr(rows), _ptr(grad), _ptr(m), _ptr(v), _ptr(rows_bf16),
                               n_rows, row_elems, frozen_rows, step, lr, beta1, beta2, eps,
                               _stream(stream)), "cart_adam_rows")


def cart_rows_to_bf16(k: torch.Tensor, v: torch.Tensor, k_out: torch.Tensor, v_out: torch.Tensor,
                      stream=None) -> None:
    """bf16 copies (nearest even) of f32 cartridge rows k, v [p, ...] into k_out, v_out."""
    n_rows = k.shape[0]
    row_elems = k.numel() // max(n_rows, 1)
    _check(_lib.cart_rows_to_bf16(_ptr(k), _ptr(v), _ptr(k_out), _ptr(v_out), n_rows, row_elems,
                                  _stream(stream)), "cart_rows_to_bf16")


def rows_to_bf16(k: torch.Tensor, v: torch.Tensor, stream=None):
    """Allocate and return the bf16 copies of f32 cartridge rows k, v."""
    k_out = torch.empty(k.shape, dtype=torch.bfloat16, device=k.device)
    v_out = torch.empty(v.shape, dtype=torch.bfloat16, device=v.device)
    cart_rows_to_bf16(k, v, k_out, v_out, stream)
    return k_out, v_out


def cart_attn_workspace_size(shape: AttnShape, for_backward: bool) -> int:
    return int(_lib.cart_attn_workspace_size(ctypes.byref(shape), int(for_backward)))


def cart_attn_fwd(shape: AttnShape, q, k_tok, v_tok, k_cart, v_cart, out, lse, workspace,
                  stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.cart_attn_fwd(ctypes.byref(shape), _ptr(q), _ptr(k_tok), _ptr(v_tok),
                              _ptr(k_cart), _ptr(v_cart), _ptr(out), _ptr(lse),
                              _ptr(workspace), ws_bytes, _stream(stream)), "cart_attn_fwd")


def cart_attn_bwd(shape: AttnShape, q, k_tok, v_tok, k_cart, v_cart, out, lse, dout, dq,
                  dk_tok, dv_tok, dk_cart, dv_cart, accumulate_cart: bool, workspace,
                  stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.cart_attn_bwd(ctypes.byref(shape), _ptr(q), _ptr(k_tok), _ptr(v_tok),
                              _ptr(k_cart), _ptr(v_cart), _ptr(out), _ptr(lse), _ptr(dout),
                              _ptr(dq), _ptr(dk_tok), _ptr(dv_tok), _ptr(dk_cart),
                              _ptr(dv_cart), int(accumulate_cart), _ptr(workspace), ws_bytes,
                              _stream(stream)), "cart_attn_bwd")


def cart_attn_schedule_query(shape: AttnShape) -> AttnSchedule:
    """The work split cart_attn_fwd / cart_attn_bwd will use (host-only)."""
    out = AttnSchedule()
    _check(_lib.cart_attn_schedule_query(ctypes.byref(shape), ctypes.byref(out)),
           "cart_attn_schedule_query")
    return out


def parts_desc(k_parts, v_parts, frozen) -> Parts:
    """A cart_parts description of device tensors (kept alive by the caller).
    The arrays it points to are attached to the returned object."""
    n = len(k_parts)
    rows = (ctypes.c_int32 * n)(*[int(k.shape[0]) for k in k_parts])
    fr = (ctypes.c_int32 * n)(*[int(f) for f in frozen])
    kp = (ctypes.c_void_p * n)(*[k.data_ptr() if k.numel() else None for k in k_parts])
    vp = (ctypes.c_void_p * n)(*[v.data_ptr() if v.numel() else None for v in v_parts])
    d = Parts(n, rows, fr, kp, vp)
    d._keep = (rows, fr, kp, vp)
    return d


def cart_parts_rows(parts: Parts) -> int:
    return int(_lib.cart_parts_rows(ctypes.byref(parts)))


def cart_compose_rows(parts: Parts, src_dtype, n_kv_heads: int, head_dim: int, k_out, v_out,
                      stream=None) -> None:
    _check(_lib.cart_compose_rows(ctypes.byref(parts), _DTYPES[src_dtype], n_kv_heads, head_dim,
                                  _ptr(k_out), _ptr(v_out), _dt(k_out), _stream(stream)),
           "cart_compose_rows")


def cart_attn_bwd_composed(shape: AttnShape, parts: Parts, q, k_tok, v_tok, k_cart, v_cart, out,
                           lse, dout, dq, dk_tok, dv_tok, dk_cart, dv_cart,
                           accumulate_cart: bool, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.cart_attn_bwd_composed(ctypes.byref(shape), ctypes.byref(parts), _ptr(q),
                                       _ptr(k_tok), _ptr(v_tok), _ptr(k_cart), _ptr(v_cart),
                                       _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk_tok),
                                       _ptr(dv_tok), _ptr(dk_cart), _ptr(dv_cart),
                                       int(accumulate_cart), _ptr(workspace), ws_bytes,
                                       _stream(stream)), "cart_attn_bwd_composed")


# ------------------------------------------------------------ conveniences

def workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """Device workspace of at least ``nbytes`` (torch allocation)."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attn_fwd(q, k_tok, v_tok, k_cart, v_cart, frozen_rows: int = 1, scale: float = 0.0,
             stream=None, window: int = 0, seg_lens=None):
    """Allocate O, LSE and the workspace, run cart_attn_fwd, return (O, LSE)."""
    p = 0 if k_cart is None else k_cart.shape[0]
    rd = k_cart.dtype if k_cart is not None else q.dtype
    shape = attn_shape(q, k_tok, p, frozen_rows, scale, rd, window, seg_lens)
    out = torch.empty_like(q)
    B, n, Hq = shape.batch, shape.q_seq, shape.n_q_heads
    lse = torch.empty(B, Hq, n, dtype=torch.float32, device=q.device)
    ws = workspace(cart_attn_workspace_size(shape, False), q.device)
    cart_attn_fwd(shape, q, k_tok, v_tok, k_cart, v_cart, out, lse, ws, stream)
    return out, lse


def attn_bwd(q, k_tok, v_tok, k_cart, v_cart, out, lse, dout, frozen_rows: int = 1,
             scale: float = 0.0, dk_cart=None, dv_cart=None, accumulate_cart: bool = False,
             stream=None, window: int = 0, seg_lens=None):
    """Allocate gradients and workspace, run cart_attn_bwd.

    Returns (dq, dk_tok, dv_tok, dk_cart, dv_cart); cartridge gradients are
    float32 [p, Hkv, d] (the given buffers when passed)."""
    p = 0 if k_cart is None else k_cart.shape[0]
    rd = k_cart.dtype if k_cart is not None else q.dtype
    shape = attn_shape(q, k_tok, p, frozen_rows, scale, rd, window, seg_lens)
    dq = torch.empty_like(q)
    dk_tok = torch.empty_like(k_tok)
    dv_tok = torch.empty_like(v_tok)
    if p > 0:
        if dk_cart is None:
            dk_cart = torch.empty(k_cart.shape, dtype=torch.float32, device=q.device)
        if dv_cart is None:
            dv_cart = torch.empty(v_cart.shape, dtype=torch.float32, device=q.device)
    ws = workspace(cart_attn_workspace_size(shape, True), q.device)
    cart_attn_bwd(shape, q, k_tok, v_tok, k_cart, v_cart, out, lse, dout, dq, dk_tok, dv_tok,
                  dk_cart, dv_cart, accumulate_cart, ws, stream)
    return dq, dk_tok, dv_tok, dk_cart, dv_cart


class PagedCache:
    """A cart_cache handle over torch-allocated pages (bf16, page size 16).

    k_pages/v_pages: [n_pages, Hkv, 16, d]; block_table: [n_seqs, max_pages]
    int32; seq_lens: [n_seqs] int32, zero at creation."""

    def __init__(self, n_seqs: int, n_kv_heads: int, head_dim: int, max_pages_per_seq: int,
                 n_pages: int, block_table: torch.Tensor, device, page_size: int = 16):
        self.k_pages = torch.zeros(n_pages, n_kv_heads, page_size, head_dim,
                                   dtype=torch.bfloat16, device=device)
        self.v_pages = torch.zeros_like(self.k_pages)
        self.block_table = block_table.to(device=device, dtype=torch.int32).contiguous()
        self.seq_lens = torch.zeros(n_seqs, dtype=torch.int32, device=device)
        self.n_kv_heads, self.head_dim = n_kv_heads, head_dim
        desc = CacheDesc(n_seqs, n_kv_heads, head_dim, page_size, max_pages_per_seq, n_pages,
                         CART_BF16, self.k_pages.data_ptr(), self.v_pages.data_ptr(),
                         self.block_table.data_ptr(), self.seq_lens.data_ptr())
        h = ctypes.c_void_p()
        _check(_lib.cart_cache_create(ctypes.byref(desc), ctypes.byref(h)), "cart_cache_create")
        self.handle = h

    def close(self):
        if self.handle:
            _lib.cart_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def seq_len(self, seq: int) -> int:
        return int(_lib.cart_cache_seq_len(self.handle, seq))

    def reset(self, seq: int, stream=None) -> None:
        _check(_lib.cart_cache_reset(self.handle, seq, _stream(stream)), "cart_cache_reset")

    def append(self, seq: int, k: torch.Tensor, v: torch.Tensor, stream=None) -> None:
        n_rows, Hkv, d = k.shape
        _check(_lib.cart_append_cache(self.handle, seq, _ptr(k), _ptr(v), _dt(k), n_rows, Hkv,
                                      d, _stream(stream)), "cart_append_cache")

    def write(self, seq: int, k_cart: torch.Tensor, v_cart: torch.Tensor, stream=None) -> None:
        p, Hkv, d = k_cart.shape
        _check(_lib.cart_write_cache(self.handle, seq, _ptr(k_cart), _ptr(v_cart),
                                     _dt(k_cart), p, Hkv, d, _stream(stream)),
               "cart_write_cache")

    def write_composed(self, seq: int, parts: "Parts", src_dtype, stream=None) -> None:
        _check(_lib.cart_write_composed_cache(self.handle, seq, ctypes.byref(parts),
                                              _DTYPES[src_dtype], self.n_kv_heads, self.head_dim,
                                              _stream(stream)), "cart_write_composed_cache")

    def truncate(self, seq: int, new_len: int, stream=None) -> None:
        _check(_lib.cart_cache_truncate(self.handle, seq, new_len, _stream(stream)),
               "cart_cache_truncate")

    def verify_workspace_size(self, n_tokens: int, n_q_heads: int) -> int:
        return int(_lib.cart_decode_verify_workspace_size(self.handle, n_tokens, n_q_heads))

    def verify(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
               out: torch.Tensor, workspace_t: Optional[torch.Tensor], scale: float = 0.0,
               stream=None) -> None:
        """cart_decode_verify: q [S, k, Hq, d], k_new/v_new [S, k, Hkv, d]."""
        ws_bytes = 0 if workspace_t is None else workspace_t.numel() * workspace_t.element_size()
        _check(_lib.cart_decode_verify(self.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                       q.shape[1], q.shape[2], scale, _ptr(out), _ptr(workspace_t),
                                       ws_bytes, _stream(stream)), "cart_decode_verify")

    def decode_workspace_size(self, n_q_heads: int) -> int:
        return int(_lib.cart_decode_workspace_size(self.handle, n_q_heads))

    def decode_schedule(self, n_q_heads: int, n_tokens: int = 1) -> DecodeSchedule:
        """The split plan of a decode (n_tokens = 1) or verify step (host-only)."""
        out = DecodeSchedule()
        _check(_lib.cart_decode_schedule_query(self.handle, n_tokens, n_q_heads,
                                               ctypes.byref(out)), "cart_decode_schedule_query")
        return out

    def decode(self, q: torch.Tensor, out: torch.Tensor, workspace_t: Optional[torch.Tensor],
               k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
               scale: float = 0.0, stream=None) -> None:
        ws_bytes = 0 if workspace_t is None else workspace_t.numel() * workspace_t.element_size()
        _check(_lib.cart_decode(self.handle, _ptr(q), _ptr(k_new), _ptr(v_new), q.shape[1],
                                scale, _ptr(out), _ptr(workspace_t), ws_bytes, _stream(stream)),
               "cart_decode")


    def decode_noalloc(self, q: torch.Tensor, out: torch.Tensor,
                       k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                       scale: float = 0.0, stream=None) -> None:
        """cart_decode_noalloc: the same step with the library's own scratch."""
        _check(_lib.cart_decode_noalloc(self.handle, _ptr(q), _ptr(k_new), _ptr(v_new),
                                        q.shape[1], scale, _ptr(out), _stream(stream)),
               "cart_decode_noalloc")


def decode_noalloc_max_bytes() -> int:
    return int(_lib.cart_decode_noalloc_max_bytes())


def timing_enable(on: bool) -> None:
    """Start (clearing old records) or stop per-kernel launch timing."""
    _check(_lib.cart_timing_enable(int(on)), "cart_timing_enable")


def timing_only(kernel=None) -> None:
    """Time only launches of `kernel` (None: every kernel)."""
    _check(_lib.cart_timing_only(kernel.encode() if kernel else None), "cart_timing_only")


def timing_query(kernel: str):
    """(total ms, launches) of one kernel name since timing was enabled."""
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    _check(_lib.cart_timing_query(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)),
           "cart_timing_query")
    return ms.value, n.value


def lib() -> ctypes.CDLL:
    return _lib
