"""Python binding of libmiattn.so: exact attention forward and paged split-KV
decode for MI355X (gfx950).

This layer only marshals arguments: it reads shapes, strides and data
pointers from torch tensors, allocates outputs and workspaces with torch when
the caller passes none, and calls the C ABI declared in include/mi_attn.h on
torch's current stream. Every step of the computation runs in the library's
HIP kernels; there is no fallback. If the shared library is missing or fails
to load, every call raises.

Entry points (same names as the C ABI):
  mi_attn_fwd(q, k, v, ...)              -> (out, lse)
  mi_attn_bwd(q, k, v, out, dout, lse, ...) -> (dq, dk, dv)
  mi_attn_decode_splitkv(q, k_cache, v_cache, page_table, ...) -> (out, lse)
  mi_attn_decode_splitkv_noalloc(...)    the same decode with no workspace
                                         (static per-GPU scratch in the library)
  mi_attn_combine(o_partial, lse_partial, ...) -> (out, lse)
  mi_attn_decode_workspace_bytes(...), mi_attn_decode_num_splits(...)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = [
    "MiAttnError", "load", "lib_path", "mi_attn_fwd", "mi_attn_bwd", "mi_attn_bwd_workspace_bytes",
    "BwdParams", "mi_attn_decode_splitkv", "mi_attn_decode_splitkv_noalloc",
    "mi_attn_combine", "mi_attn_decode_workspace_bytes", "mi_attn_decode_num_splits",
    "mi_attn_last_error", "mi_attn_version", "FwdParams", "DecodeParams",
    "MI_ATTN_OK", "MI_ATTN_EINVAL", "MI_ATTN_EUNSUPPORTED", "MI_ATTN_EBOUNDS",
    "MI_ATTN_EWORKSPACE", "MI_ATTN_EHIP", "MI_ATTN_KV_BF16", "MI_ATTN_KV_FP8_E4M3", "MI_ATTN_KV_FP8_E5M2",
]

MI_ATTN_OK = 0
MI_ATTN_EINVAL = -1
MI_ATTN_EUNSUPPORTED = -2
MI_ATTN_EBOUNDS = -3
MI_ATTN_EWORKSPACE = -4
MI_ATTN_EHIP = -5
MI_ATTN_KV_BF16 = 0
MI_ATTN_KV_FP8_E4M3 = 1
MI_ATTN_KV_FP8_E5M2 = 2
_STATUS = {0: "OK", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "EBOUNDS", -4: "EWORKSPACE",
           -5: "EHIP"}

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_PKG_DIR, "libmiattn.so")


class MiAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"mi_attn {_STATUS.get(code, code)}: {message}")
        self.code = code


_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_fp = ctypes.c_void_p  # float* passed as raw address


class FwdParams(ctypes.Structure):
    """Mirror of mi_attn_fwd_params (field order and types must match the header)."""
    _fields_ = [
        ("q", _vp), ("k", _vp), ("v", _vp), ("out", _vp), ("lse", _fp),
        ("q_batch_stride", _i64), ("q_row_stride", _i64), ("q_head_stride", _i64),
        ("k_batch_stride", _i64), ("k_row_stride", _i64), ("k_head_stride", _i64),
        ("v_batch_stride", _i64), ("v_row_stride", _i64), ("v_head_stride", _i64),
        ("o_batch_stride", _i64), ("o_row_stride", _i64), ("o_head_stride", _i64),
        ("batch", _i32), ("seqlen_q", _i32), ("seqlen_k", _i32),
        ("num_heads_q", _i32), ("num_heads_kv", _i32), ("head_dim", _i32),
        ("cu_seqlens_q", _vp), ("cu_seqlens_k", _vp),
        ("total_q", _i32), ("max_seqlen_q", _i32), ("max_seqlen_k", _i32),
        ("page_table", _vp),
        ("softmax_scale", ctypes.c_float),
        ("causal", _i32), ("window_left", _i32), ("window_right", _i32),
        ("seqused_k", _vp),
        ("page_size", _i32), ("num_pages", _i32), ("max_pages_per_seq", _i32),
        ("learnable_sink", _vp),
        ("softcap", ctypes.c_float),
    ]


class BwdParams(ctypes.Structure):
    """Mirror of mi_attn_bwd_params (field order and types must match the header)."""
    _fields_ = [
        ("q", _vp), ("k", _vp), ("v", _vp), ("out", _vp), ("dout", _vp), ("lse", _fp),
        ("dq", _vp), ("dk", _vp), ("dv", _vp),
        *[(f"{t}_{w}_stride", _i64) for t in ("q", "k", "v", "o", "do", "dq", "dk", "dv")
          for w in ("batch", "row", "head")],
        ("batch", _i32), ("seqlen_q", _i32), ("seqlen_k", _i32),
        ("num_heads_q", _i32), ("num_heads_kv", _i32), ("head_dim", _i32),
        ("cu_seqlens_q", _vp), ("cu_seqlens_k", _vp),
        ("total_q", _i32), ("max_seqlen_q", _i32), ("max_seqlen_k", _i32),
        ("softmax_scale", ctypes.c_float),
        ("causal", _i32), ("window_left", _i32), ("window_right", _i32),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
    ]


class DecodeParams(ctypes.Structure):
    """Mirror of mi_attn_decode_params."""
    _fields_ = [
        ("q", _vp), ("k_cache", _vp), ("v_cache", _vp), ("page_table", _vp),
        ("seqused_k", _vp), ("out", _vp), ("lse", _fp),
        ("q_batch_stride", _i64), ("q_head_stride", _i64),
        ("o_batch_stride", _i64), ("o_head_stride", _i64),
        ("batch", _i32), ("num_heads_q", _i32), ("num_heads_kv", _i32), ("head_dim", _i32),
        ("page_size", _i32), ("num_pages", _i32), ("max_pages_per_seq", _i32),
        ("softmax_scale", ctypes.c_float),
        ("causal", _i32), ("window_left", _i32), ("window_right", _i32),
        ("num_splits", _i32),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("kv_dtype", _i32), ("k_descale", _vp), ("v_descale", _vp),
        ("learnable_sink", _vp),
        ("softcap", ctypes.c_float),
        ("cu_seqlens_q", _vp), ("max_seqlen_q", _i32), ("total_q", _i32),
    ]


_LIB = None


def load(path: Optional[str] = None):
    """Loads the shared library (once). Raises if it is missing or incomplete."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or lib_path()
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} not found: build it with `python -m exact_attention_45_amd.build` "
            "(the library has no CPU fallback)")
    lib = ctypes.CDLL(p)
    lib.mi_attn_fwd.argtypes = [ctypes.POINTER(FwdParams), _vp]
    lib.mi_attn_fwd.restype = ctypes.c_int
    lib.mi_attn_decode_splitkv.argtypes = [ctypes.POINTER(DecodeParams), _vp]
    lib.mi_attn_decode_splitkv.restype = ctypes.c_int
    lib.mi_attn_decode_splitkv_noalloc.argtypes = [ctypes.POINTER(DecodeParams), _vp]
    lib.mi_attn_decode_splitkv_noalloc.restype = ctypes.c_int
    lib.mi_attn_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeParams)]
    lib.mi_attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.mi_attn_decode_num_splits.argtypes = [ctypes.POINTER(DecodeParams)]
    lib.mi_attn_decode_num_splits.restype = ctypes.c_int
    lib.mi_attn_bwd.argtypes = [ctypes.POINTER(BwdParams), _vp]
    lib.mi_attn_bwd.restype = ctypes.c_int
    lib.mi_attn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(BwdParams)]
    lib.mi_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.mi_attn_combine.argtypes = [_vp, _vp, _vp, _i64, _vp, _i32, _i32, _i32, _vp]
    lib.mi_attn_combine.restype = ctypes.c_int
    lib.mi_attn_last_error.argtypes = []
    lib.mi_attn_last_error.restype = ctypes.c_char_p
    lib.mi_attn_version.argtypes = []
    lib.mi_attn_version.restype = ctypes.c_char_p
    if path is None:
        _LIB = lib
    return lib


def mi_attn_last_error() -> str:
    return load().mi_attn_last_error().decode()


def mi_attn_version() -> str:
    return load().mi_attn_version().decode()


def _check(rc: int):
    if rc != MI_ATTN_OK:
        raise MiAttnError(rc, mi_attn_last_error())


def _stream_ptr(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _req_bf16(name, t, device=None):
    import torch
    if t.dtype != torch.bfloat16:
        raise MiAttnError(MI_ATTN_EINVAL, f"{name} must be bfloat16 (got {t.dtype})")
    if not t.is_cuda:
        raise MiAttnError(MI_ATTN_EINVAL, f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise MiAttnError(MI_ATTN_EINVAL, f"{name} is on {t.device}, expected {device}")
    if t.stride(-1) != 1:
        raise MiAttnError(MI_ATTN_EINVAL, f"{name} must be contiguous in its last dimension")


def _req_i32(name, t, shape, device):
    import torch
    if t.dtype != torch.int32 or not t.is_cuda or t.device != device:
        raise MiAttnError(MI_ATTN_EINVAL, f"{name} must be an int32 tensor on {device}")
    if not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise MiAttnError(MI_ATTN_EINVAL, f"{name} must be contiguous with shape {tuple(shape)}")


def _win(x: Optional[int]) -> int:
    return -1 if x is None else int(x)


def mi_attn_fwd(q, k, v, out=None, lse=None, cu_seqlens_q=None, cu_seqlens_k=None,
                max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
                softmax_scale: Optional[float] = None, causal: bool = False,
                window_left: Optional[int] = None, window_right: Optional[int] = None,
                return_lse: bool = True, page_table=None, seqused_k=None,
                check_bounds: bool = False, learnable_sink=None,
                softcap: float = 0.0) -> Tuple:
    """Exact attention forward (interface page, `_flash_attn_fwd` contract).

    Dense: q (B, Sq, Hq, D), k/v (B, Sk, Hkv, D); lse (B, Hq, Sq).
    Varlen: q (Tq, Hq, D), k/v (Tk, Hkv, D), cu_seqlens_q/k int32 (B+1,);
    lse (Hq, Tq). max_seqlen_q/k default to the token totals (no device sync).
    Paged: page_table int32 (B, max_pages) with k/v caches
    (num_pages, page_size, Hkv, D), page_size a multiple of 64, seqused_k int32
    (B,) or None (every sequence max_pages * page_size keys); q dense or packed
    by cu_seqlens_q (cu_seqlens_k must be None). check_bounds validates the
    page ids and seqused_k on the host first (one device-to-host copy).
    learnable_sink: bf16 (Hq,) per-head sink logits (see include/mi_attn.h).
    softcap: > 0 caps every scaled score x to softcap * tanh(x / softcap); 0 is none.
    """
    import torch
    lib = load()
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _req_bf16(n, t, dev)
    paged = page_table is not None
    if paged and cu_seqlens_k is not None:
        raise MiAttnError(MI_ATTN_EINVAL, "page_table is not supported with cu_seqlens_k")
    if not paged and seqused_k is not None:
        raise MiAttnError(MI_ATTN_EINVAL, "seqused_k is only used with a page_table")
    varlen = cu_seqlens_q is not None or cu_seqlens_k is not None
    if varlen and not paged and (cu_seqlens_q is None or cu_seqlens_k is None):
        raise MiAttnError(MI_ATTN_EINVAL, "cu_seqlens_q and cu_seqlens_k go together")
    hq, d = q.shape[-2], q.shape[-1]
    hkv = k.shape[-2]
    if v.shape[-1] != d or k.shape[-1] != d:
        raise MiAttnError(MI_ATTN_EUNSUPPORTED, "head_dim of q, k and v must match")
    if paged:
        if k.dim() != 4 or k.shape != v.shape:
            raise MiAttnError(MI_ATTN_EINVAL, "paged k/v must be (num_pages, page_size, Hkv, D)")
        if varlen:
            if q.dim() != 3:
                raise MiAttnError(MI_ATTN_EINVAL, "varlen q must be (tokens, heads, head_dim)")
            batch = cu_seqlens_q.shape[0] - 1
            _req_i32("cu_seqlens_q", cu_seqlens_q, (batch + 1,), dev)
            total_q = q.shape[0]
            max_q = total_q if max_seqlen_q is None else int(max_seqlen_q)
            seq_shape, lse_shape = (total_q,), (hq, total_q)
        else:
            if q.dim() != 4:
                raise MiAttnError(MI_ATTN_EINVAL, "dense q must be (batch, seqlen, heads, head_dim)")
            batch, sq = q.shape[0], q.shape[1]
            total_q, max_q = batch * sq, sq
            seq_shape, lse_shape = (batch, sq), (batch, hq, sq)
        _req_i32("page_table", page_table, (batch, page_table.shape[1]), dev)
        if seqused_k is not None:
            _req_i32("seqused_k", seqused_k, (batch,), dev)
        if check_bounds:
            check_paged_bounds(page_table, seqused_k, k.shape[0], k.shape[1])
        max_k = page_table.shape[1] * k.shape[1]
    elif varlen:
        if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or k.shape != v.shape:
            raise MiAttnError(MI_ATTN_EINVAL, "varlen q/k/v must be (tokens, heads, head_dim)")
        batch = cu_seqlens_q.shape[0] - 1
        _req_i32("cu_seqlens_q", cu_seqlens_q, (batch + 1,), dev)
        _req_i32("cu_seqlens_k", cu_seqlens_k, (batch + 1,), dev)
        total_q = q.shape[0]
        max_q = total_q if max_seqlen_q is None else int(max_seqlen_q)
        max_k = k.shape[0] if max_seqlen_k is None else int(max_seqlen_k)
        seq_shape = (total_q,)
        lse_shape = (hq, total_q)
    else:
        if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
            raise MiAttnError(MI_ATTN_EINVAL, "dense q/k/v must be (batch, seqlen, heads, head_dim)")
        batch, sq = q.shape[0], q.shape[1]
        if k.shape[0] != batch:
            raise MiAttnError(MI_ATTN_EINVAL, "q and k batch sizes differ")
        total_q, max_q, max_k = batch * sq, sq, k.shape[1]
        seq_shape = (batch, sq)
        lse_shape = (batch, hq, sq)
    if out is None:
        out = torch.empty(*seq_shape, hq, d, dtype=torch.bfloat16, device=dev)
    else:
        _req_bf16("out", out, dev)
        if tuple(out.shape) != (*seq_shape, hq, d):
            raise MiAttnError(MI_ATTN_EINVAL, f"out must have shape {(*seq_shape, hq, d)}")
    if lse is None and return_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
    elif lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != lse_shape \
                or lse.device != dev:
            raise MiAttnError(MI_ATTN_EINVAL, f"lse must be contiguous float32 {lse_shape}")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)

    p = FwdParams()
    p.q, p.k, p.v, p.out, p.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(lse)
    if paged:
        if varlen:
            p.q_row_stride, p.q_head_stride = q.stride(0), q.stride(1)
            p.o_row_stride, p.o_head_stride = out.stride(0), out.stride(1)
            p.cu_seqlens_q = cu_seqlens_q.data_ptr()
        else:
            p.q_batch_stride, p.q_row_stride, p.q_head_stride = q.stride(0), q.stride(1), q.stride(2)
            p.o_batch_stride, p.o_row_stride, p.o_head_stride = (out.stride(0), out.stride(1),
                                                                 out.stride(2))
            p.seqlen_q = max_q
        p.k_batch_stride, p.k_row_stride, p.k_head_stride = k.stride(0), k.stride(1), k.stride(2)
        p.v_batch_stride, p.v_row_stride, p.v_head_stride = v.stride(0), v.stride(1), v.stride(2)
        p.page_table, p.seqused_k = page_table.data_ptr(), _ptr(seqused_k)
        p.num_pages, p.page_size, p.max_pages_per_seq = k.shape[0], k.shape[1], page_table.shape[1]
    elif varlen:
        p.q_row_stride, p.q_head_stride = q.stride(0), q.stride(1)
        p.k_row_stride, p.k_head_stride = k.stride(0), k.stride(1)
        p.v_row_stride, p.v_head_stride = v.stride(0), v.stride(1)
        p.o_row_stride, p.o_head_stride = out.stride(0), out.stride(1)
        p.cu_seqlens_q, p.cu_seqlens_k = cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()
    else:
        p.q_batch_stride, p.q_row_stride, p.q_head_stride = q.stride(0), q.stride(1), q.stride(2)
        p.k_batch_stride, p.k_row_stride, p.k_head_stride = k.stride(0), k.stride(1), k.stride(2)
        p.v_batch_stride, p.v_row_stride, p.v_head_stride = v.stride(0), v.stride(1), v.stride(2)
        p.o_batch_stride, p.o_row_stride, p.o_head_stride = (out.stride(0), out.stride(1),
                                                             out.stride(2))
        p.seqlen_q, p.seqlen_k = max_q, max_k
    p.batch, p.num_heads_q, p.num_heads_kv, p.head_dim = batch, hq, hkv, d
    p.total_q, p.max_seqlen_q, p.max_seqlen_k = total_q, max_q, max_k
    p.softmax_scale = scale
    p.causal, p.window_left, p.window_right = int(bool(causal)), _win(window_left), _win(window_right)
    p.learnable_sink = _req_sink(learnable_sink, hq, dev)
    p.softcap = float(softcap)
    _check(lib.mi_attn_fwd(ctypes.byref(p), _stream_ptr(dev)))
    return out, lse


def _bwd_params(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                max_seqlen_k, softmax_scale, causal, window_left, window_right):
    """Checks shapes and fills BwdParams (no workspace yet)."""
    import torch
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq),
                 ("dk", dk), ("dv", dv)):
        _req_bf16(n, t, dev)
    varlen = cu_seqlens_q is not None or cu_seqlens_k is not None
    if varlen and (cu_seqlens_q is None or cu_seqlens_k is None):
        raise MiAttnError(MI_ATTN_EINVAL, "cu_seqlens_q and cu_seqlens_k go together")
    hq, d = q.shape[-2], q.shape[-1]
    hkv = k.shape[-2]
    if k.shape != v.shape or k.shape[-1] != d:
        raise MiAttnError(MI_ATTN_EUNSUPPORTED, "k and v must match q's head_dim and each other")
    for n, t, ref in (("out", out, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k),
                      ("dv", dv, v)):
        if t.shape != ref.shape:
            raise MiAttnError(MI_ATTN_EINVAL, f"{n} must have shape {tuple(ref.shape)}")
    p = BwdParams()
    if varlen:
        if q.dim() != 3 or k.dim() != 3:
            raise MiAttnError(MI_ATTN_EINVAL, "varlen q/k/v must be (tokens, heads, head_dim)")
        batch = cu_seqlens_q.shape[0] - 1
        _req_i32("cu_seqlens_q", cu_seqlens_q, (batch + 1,), dev)
        _req_i32("cu_seqlens_k", cu_seqlens_k, (batch + 1,), dev)
        total_q = q.shape[0]
        max_q = total_q if max_seqlen_q is None else int(max_seqlen_q)
        max_k = k.shape[0] if max_seqlen_k is None else int(max_seqlen_k)
        lse_shape = (hq, total_q)
        p.cu_seqlens_q, p.cu_seqlens_k = cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()
        p.total_q, p.max_seqlen_q, p.max_seqlen_k = total_q, max_q, max_k
    else:
        if q.dim() != 4 or k.dim() != 4:
            raise MiAttnError(MI_ATTN_EINVAL, "dense q/k/v must be (batch, seqlen, heads, head_dim)")
        batch, sq = q.shape[0], q.shape[1]
        if k.shape[0] != batch:
            raise MiAttnError(MI_ATTN_EINVAL, "q and k batch sizes differ")
        lse_shape = (batch, hq, sq)
        p.seqlen_q, p.seqlen_k = sq, k.shape[1]
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != lse_shape \
            or lse.device != dev:
        raise MiAttnError(MI_ATTN_EINVAL, f"lse must be contiguous float32 {lse_shape}")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", out), ("do", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        st = t.stride()
        if varlen:
            setattr(p, f"{name}_row_stride", st[0])
            setattr(p, f"{name}_head_stride", st[1])
        else:
            setattr(p, f"{name}_batch_stride", st[0])
            setattr(p, f"{name}_row_stride", st[1])
            setattr(p, f"{name}_head_stride", st[2])
    p.q, p.k, p.v, p.out, p.dout, p.lse = (q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), dout.data_ptr(), lse.data_ptr())
    p.dq, p.dk, p.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    p.batch, p.num_heads_q, p.num_heads_kv, p.head_dim = batch, hq, hkv, d
    p.softmax_scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    p.causal, p.window_left, p.window_right = int(bool(causal)), _win(window_left), _win(window_right)
    return p


def mi_attn_bwd_workspace_bytes(q, k, v, out, dout, lse, cu_seqlens_q=None, cu_seqlens_k=None,
                                max_seqlen_q=None, max_seqlen_k=None, causal=False) -> int:
    """Workspace bytes mi_attn_bwd needs for these tensors (raises if invalid)."""
    lib = load()
    p = _bwd_params(q, k, v, out, dout, lse, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                    max_seqlen_k, None, causal, None, None)
    n = lib.mi_attn_bwd_workspace_bytes(ctypes.byref(p))
    if n == 0 and mi_attn_last_error():
        # invalid parameters: mi_attn_bwd runs the same checks first and
        # returns their status without launching anything
        _check(lib.mi_attn_bwd(ctypes.byref(p), None))
    return int(n)


def mi_attn_bwd(q, k, v, out, dout, lse, cu_seqlens_q=None, cu_seqlens_k=None,
                max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
                softmax_scale: Optional[float] = None, causal: bool = False,
                window_left: Optional[int] = None, window_right: Optional[int] = None,
                dq=None, dk=None, dv=None, workspace=None) -> Tuple:
    """Backward of mi_attn_fwd (interface page, `_flash_attn_bwd` contract):
    returns (dq, dk, dv) shaped like q, k, v, given the forward's out and lse
    and the output gradient dout. Dense (B, S, H, D) or packed (T, H, D)
    tensors with cu_seqlens_q/k as for mi_attn_fwd; head_dim 64, 96, 128, 192 or 256; no
    paged K/V or learnable sink. workspace: a uint8 device tensor of at least
    mi_attn_bwd_workspace_bytes bytes, or None to allocate one.
    """
    import torch
    lib = load()
    dev = q.device
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    p = _bwd_params(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                    max_seqlen_k, softmax_scale, causal, window_left, window_right)
    need = lib.mi_attn_bwd_workspace_bytes(ctypes.byref(p))
    err = mi_attn_last_error()
    if need == 0 and err:
        _check(lib.mi_attn_bwd(ctypes.byref(p), _stream_ptr(dev)))  # raises with the status
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_cuda or workspace.device != dev:
            raise MiAttnError(MI_ATTN_EINVAL, f"workspace must be a uint8 tensor on {dev}")
        p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _check(lib.mi_attn_bwd(ctypes.byref(p), _stream_ptr(dev)))
    return dq, dk, dv


def _decode_params(q, k_cache, v_cache, page_table, seqused_k, out, lse, softmax_scale,
                   num_splits, window_left, workspace, cu_seqlens_q=None, max_seqlen_q=None,
                   causal=False, window_right=None) -> DecodeParams:
    """q (B, Hq, D), or (total_q, Hq, D) packed by cu_seqlens_q; B is the
    page table's row count."""
    p = DecodeParams()
    p.q, p.k_cache, p.v_cache = _ptr(q), _ptr(k_cache), _ptr(v_cache)
    p.page_table, p.seqused_k, p.out, p.lse = _ptr(page_table), _ptr(seqused_k), _ptr(out), _ptr(lse)
    p.q_batch_stride, p.q_head_stride = q.stride(0), q.stride(1)
    if out is not None:
        p.o_batch_stride, p.o_head_stride = out.stride(0), out.stride(1)
    p.batch, p.num_heads_q, p.head_dim = page_table.shape[0], q.shape[1], q.shape[2]
    p.num_pages, p.page_size, p.num_heads_kv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    p.max_pages_per_seq = page_table.shape[1]
    p.softmax_scale = (1.0 / math.sqrt(q.shape[2]) if softmax_scale is None
                       else float(softmax_scale))
    p.causal, p.window_left, p.window_right = int(bool(causal)), _win(window_left), _win(window_right)
    p.num_splits = int(num_splits)
    if workspace is not None:
        p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    p.kv_dtype = _kv_dtype(k_cache)
    if cu_seqlens_q is not None:
        p.cu_seqlens_q = cu_seqlens_q.data_ptr()
        p.total_q = q.shape[0]
        p.max_seqlen_q = q.shape[0] if max_seqlen_q is None else int(max_seqlen_q)
    return p


def _req_sink(sink, hq: int, device):
    """learnable_sink: bf16 (num_heads_q,) device tensor, or None."""
    if sink is None:
        return None
    _req_bf16("learnable_sink", sink, device)
    if tuple(sink.shape) != (hq,) or not sink.is_contiguous():
        raise MiAttnError(MI_ATTN_EINVAL, f"learnable_sink must be contiguous ({hq},)")
    return sink.data_ptr()


def _kv_dtype(t) -> int:
    """Cache type code from the tensor dtype: float8_e4m3fn (or raw uint8
    bytes, read as e4m3) and float8_e5m2 are fp8 caches, bfloat16 is bf16."""
    import torch
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return MI_ATTN_KV_FP8_E4M3
    if t.dtype == torch.float8_e5m2:
        return MI_ATTN_KV_FP8_E5M2
    return MI_ATTN_KV_BF16


def _is_fp8(t) -> bool:
    return _kv_dtype(t) != MI_ATTN_KV_BF16


def _req_kv(name, t, device, fp8: bool):
    """bf16 cache, or fp8 (float8_e4m3fn, raw uint8 e4m3 bytes, or float8_e5m2)."""
    if not fp8:
        return _req_bf16(name, t, device)
    if not _is_fp8(t):
        raise MiAttnError(MI_ATTN_EINVAL, f"{name} must be an fp8 tensor like k_cache "
                                          f"(got {t.dtype})")
    if not t.is_cuda or t.device != device:
        raise MiAttnError(MI_ATTN_EINVAL, f"{name} must be a device tensor on {device}")


def mi_attn_decode_workspace_bytes(q, k_cache, v_cache, page_table, num_splits: int = 0,
                                   cu_seqlens_q=None, max_seqlen_q: Optional[int] = None) -> int:
    lib = load()
    p = _decode_params(q, k_cache, v_cache, page_table, None, None, None, None, num_splits, None,
                       None, cu_seqlens_q, max_seqlen_q)
    n = lib.mi_attn_decode_workspace_bytes(ctypes.byref(p))
    if n == 0 and mi_attn_last_error():
        # the size query only says "invalid"; the split-count query returns
        # the status itself for the same validation
        rc = lib.mi_attn_decode_num_splits(ctypes.byref(p))
        raise MiAttnError(rc if rc < 0 else MI_ATTN_EINVAL, mi_attn_last_error())
    return n


def mi_attn_decode_num_splits(q, k_cache, v_cache, page_table, num_splits: int = 0,
                              cu_seqlens_q=None, max_seqlen_q: Optional[int] = None) -> int:
    lib = load()
    p = _decode_params(q, k_cache, v_cache, page_table, None, None, None, None, num_splits, None,
                       None, cu_seqlens_q, max_seqlen_q)
    n = lib.mi_attn_decode_num_splits(ctypes.byref(p))
    _check(min(n, 0))
    return n


def check_paged_bounds(page_table, seqused_k, num_pages: int, page_size: int):
    """Host-side check of page-table contents (one device-to-host copy).

    Mirrors the block-table bounds check on the sm_120 PR page: every page a
    sequence uses must be in [0, num_pages), and seqused_k must fit the table.
    """
    pt = page_table.cpu()
    cap = pt.shape[1] * page_size
    used = seqused_k.cpu() if seqused_k is not None else None
    for b in range(pt.shape[0]):
        n = cap if used is None else int(used[b])
        if n < 0 or n > cap:
            raise MiAttnError(MI_ATTN_EBOUNDS, f"seqused_k[{b}] = {n} outside [0, {cap}]")
        npg = -(-n // page_size)
        if npg:
            row = pt[b, :npg]
            if int(row.min()) < 0 or int(row.max()) >= num_pages:
                raise MiAttnError(MI_ATTN_EBOUNDS, f"page_table row {b} references a page "
                                                   f"outside [0, {num_pages})")


def mi_attn_decode_splitkv(q, k_cache, v_cache, page_table, seqused_k=None, out=None, lse=None,
                           softmax_scale: Optional[float] = None, num_splits: int = 0,
                           window_left: Optional[int] = None, workspace=None,
                           return_lse: bool = True, check_bounds: bool = False,
                           k_descale=None, v_descale=None, learnable_sink=None,
                           softcap: float = 0.0, cu_seqlens_q=None,
                           max_seqlen_q: Optional[int] = None, causal: bool = False,
                           window_right: Optional[int] = None):
    """Query tokens against a paged cache, split along keys, then combined.

    q (B, Hq, D): one token per sequence; or (total_q, Hq, D) with cu_seqlens_q
    int32 (B+1,) packing a few tokens per sequence (aligned bottom-right to
    its keys; causal / window_right then apply), max_seqlen_q their maximum
    (None: total_q, which is safe but sizes the launch for it).
    k/v cache (num_pages, page_size, Hkv, D) contiguous, bf16 or fp8
    (float8_e4m3fn, raw uint8 e4m3 bytes, or float8_e5m2; then k_descale /
    v_descale are float32 (B, Hkv) or None for 1); page_table int32
    (B, max_pages); seqused_k int32 (B,) or None. softcap as for mi_attn_fwd
    (on the descaled scores). Returns out shaped like q (bf16) and lse
    (q.shape[0], Hq) float32.
    """
    return _decode(False, q, k_cache, v_cache, page_table, seqused_k, out, lse, softmax_scale,
                   num_splits, window_left, workspace, return_lse, check_bounds, k_descale,
                   v_descale, learnable_sink, softcap, cu_seqlens_q, max_seqlen_q, causal,
                   window_right)


def mi_attn_decode_splitkv_noalloc(q, k_cache, v_cache, page_table, seqused_k=None, out=None,
                                   lse=None, softmax_scale: Optional[float] = None,
                                   num_splits: int = 0, window_left: Optional[int] = None,
                                   return_lse: bool = True, check_bounds: bool = False,
                                   k_descale=None, v_descale=None, learnable_sink=None,
                                   softcap: float = 0.0, cu_seqlens_q=None,
                                   max_seqlen_q: Optional[int] = None, causal: bool = False,
                                   window_right: Optional[int] = None):
    """mi_attn_decode_splitkv through the C entry point that allocates
    nothing: the split partials go to the library's static per-GPU scratch
    (64 MiB; larger requests raise EWORKSPACE) instead of a workspace. Calls
    that may overlap on one GPU race on that scratch. Pass out (and lse) to
    keep this call free of allocations on the Python side as well."""
    return _decode(True, q, k_cache, v_cache, page_table, seqused_k, out, lse, softmax_scale,
                   num_splits, window_left, None, return_lse, check_bounds, k_descale,
                   v_descale, learnable_sink, softcap, cu_seqlens_q, max_seqlen_q, causal,
                   window_right)


def _decode(noalloc, q, k_cache, v_cache, page_table, seqused_k, out, lse, softmax_scale,
            num_splits, window_left, workspace, return_lse, check_bounds, k_descale, v_descale,
            learnable_sink, softcap, cu_seqlens_q=None, max_seqlen_q=None, causal=False,
            window_right=None):
    import torch
    lib = load()
    dev = q.device
    _req_bf16("q", q, dev)
    fp8 = _is_fp8(k_cache)
    _req_kv("k_cache", k_cache, dev, fp8)
    _req_kv("v_cache", v_cache, dev, fp8)
    if fp8 and _kv_dtype(v_cache) != _kv_dtype(k_cache):
        raise MiAttnError(MI_ATTN_EINVAL, "k_cache and v_cache must have the same fp8 format")
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise MiAttnError(MI_ATTN_EINVAL, "q must be (B, Hq, D) and caches (pages, page_size, Hkv, D)")
    if not k_cache.is_contiguous() or not v_cache.is_contiguous():
        raise MiAttnError(MI_ATTN_EINVAL, "k_cache and v_cache must be contiguous")
    T, hq, d = q.shape  # T: query tokens (one per sequence, or packed)
    B = page_table.shape[0]
    if cu_seqlens_q is None:
        if T != B:
            raise MiAttnError(MI_ATTN_EINVAL, f"q has {T} rows but page_table {B} sequences")
    else:
        _req_i32("cu_seqlens_q", cu_seqlens_q, (B + 1,), dev)
    _req_i32("page_table", page_table, (B, page_table.shape[1]), dev)
    if seqused_k is not None:
        _req_i32("seqused_k", seqused_k, (B,), dev)
    if check_bounds:
        check_paged_bounds(page_table, seqused_k, k_cache.shape[0], k_cache.shape[1])
    if out is None:
        out = torch.empty(T, hq, d, dtype=torch.bfloat16, device=dev)
    else:
        _req_bf16("out", out, dev)
        if tuple(out.shape) != (T, hq, d):
            raise MiAttnError(MI_ATTN_EINVAL, f"out must have shape {(T, hq, d)}")
    if lse is None and return_lse:
        lse = torch.empty(T, hq, dtype=torch.float32, device=dev)
    elif lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (T, hq) \
                or not lse.is_cuda or lse.device != dev:
            raise MiAttnError(MI_ATTN_EINVAL, f"lse must be a contiguous float32 {(T, hq)} "
                                              f"tensor on {dev}")
    if workspace is None and not noalloc:
        nbytes = mi_attn_decode_workspace_bytes(q, k_cache, v_cache, page_table, num_splits,
                                                cu_seqlens_q, max_seqlen_q)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    p = _decode_params(q, k_cache, v_cache, page_table, seqused_k, out, lse, softmax_scale,
                       num_splits, window_left, workspace, cu_seqlens_q, max_seqlen_q, causal,
                       window_right)
    for n, t in (("k_descale", k_descale), ("v_descale", v_descale)):
        if t is None:
            continue
        if not fp8:
            raise MiAttnError(MI_ATTN_EINVAL, f"{n} applies to an fp8 cache only")
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, k_cache.shape[2]) \
                or t.device != dev:
            raise MiAttnError(MI_ATTN_EINVAL, f"{n} must be contiguous float32 {(B, k_cache.shape[2])}")
    p.k_descale, p.v_descale = _ptr(k_descale), _ptr(v_descale)
    p.learnable_sink = _req_sink(learnable_sink, hq, dev)
    p.softcap = float(softcap)
    entry = lib.mi_attn_decode_splitkv_noalloc if noalloc else lib.mi_attn_decode_splitkv
    _check(entry(ctypes.byref(p), _stream_ptr(dev)))
    return out, lse


def mi_attn_combine(o_partial, lse_partial, out=None, lse=None, return_lse: bool = True):
    """LSE-weighted merge (interface page, `flash_attn_combine`).

    o_partial float32 (rows, splits, D) contiguous, lse_partial float32
    (rows, splits) contiguous. Returns out (rows, D) bf16 and lse (rows,).
    """
    import torch
    lib = load()
    dev = o_partial.device
    if o_partial.dtype != torch.float32 or lse_partial.dtype != torch.float32:
        raise MiAttnError(MI_ATTN_EINVAL, "partials must be float32")
    if not (o_partial.is_contiguous() and lse_partial.is_contiguous()) or o_partial.dim() != 3 \
            or tuple(lse_partial.shape) != tuple(o_partial.shape[:2]):
        raise MiAttnError(MI_ATTN_EINVAL, "o_partial (rows, splits, D) and lse_partial "
                                          "(rows, splits) must be contiguous")
    rows, splits, d = o_partial.shape
    if out is None:
        out = torch.empty(rows, d, dtype=torch.bfloat16, device=dev)
    else:
        _req_bf16("out", out, dev)
    if lse is None and return_lse:
        lse = torch.empty(rows, dtype=torch.float32, device=dev)
    rc = lib.mi_attn_combine(o_partial.data_ptr(), lse_partial.data_ptr(), out.data_ptr(),
                             out.stride(0), _ptr(lse), rows, splits, d, _stream_ptr(dev))
    _check(rc)
    return out, lse
