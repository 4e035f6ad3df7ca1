"""MI355X (gfx950) FlashAttention forward: thin PyTorch binding over libattnfwd.so.

The calls carry the names of the C ABI (include/attn_fwd.h).  This module
only marshals arguments: it checks tensor placement and layout, allocates the
outputs with torch.empty, and passes raw device pointers plus the current HIP
stream to the library.  Every step of the computation runs in the library's
kernels; there is no other implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import math
from typing import List, Optional, Sequence, Tuple

from . import _lib

__all__ = ["attn_fwd_varlen", "attn_fwd_dense", "attn_fwd_padded", "attn_unpad_gather",
           "attn_pad_scatter", "attn_bwd_varlen", "attn_bwd_dense", "attn_bwd_workspace_bytes",
           "attn_fwd_paged", "attn_fwd_paged_workspace_bytes", "paged_workspace",
           "attn_mask_to_varlen", "attn_fwd_fp8_varlen", "attn_fwd_fp8_dense",
           "attn_fwd_paged_fp8kv",
           "attn_fwd_workspace_bytes", "workspace", "abi_version", "AttnError"]

AttnError = _lib.AttnError


def _torch():
    import torch
    return torch


def _stream_ptr(device, stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _check_bf16(name, t):
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError(f"{name} must hold bfloat16 (or its 16-bit storage), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def abi_version() -> int:
    return int(_lib.load().attn_abi_version())


def attn_fwd_workspace_bytes(num_seqs: int, max_seqlen: int, num_heads_q: int, head_dim: int,
                             causal: bool) -> int:
    """Bytes of workspace that let a launch of this shape split long key ranges (0: none)."""
    return int(_lib.load().attn_fwd_workspace_bytes(int(num_seqs), int(max_seqlen),
                                                     int(num_heads_q), int(head_dim),
                                                     int(bool(causal))))


def workspace(num_seqs: int, max_seqlen: int, num_heads_q: int, head_dim: int, causal: bool,
              device="cuda"):
    """A device buffer of attn_fwd_workspace_bytes for the shape, or None when none is needed."""
    n = attn_fwd_workspace_bytes(num_seqs, max_seqlen, num_heads_q, head_dim, causal)
    if n <= 0:
        return None
    return _torch().empty(n, dtype=_torch().uint8, device=device)


def attn_fwd_launch_plan(varlen: bool, num_seqs: int, total_q: int, max_seqlen: int,
                         num_heads_q: int, head_dim: int, causal: bool,
                         workspace_bytes: int = 0) -> dict:
    """The library's launch choice for a forward shape: tile policy, workgroup
    order, key-range parts per query block and queries per block."""
    plan = (ctypes.c_int32 * 4)()
    _lib.check("attn_fwd_launch_plan", _lib.load().attn_fwd_launch_plan(
        int(bool(varlen)), int(num_seqs), int(total_q), int(max_seqlen), int(num_heads_q),
        int(head_dim), int(bool(causal)), int(workspace_bytes), plan))
    return {"policy": plan[0], "order": plan[1], "n_split": plan[2], "bm": plan[3]}


def attn_fwd_tile_policy_compiled(policy: int, head_dim: int) -> bool:
    """Whether ATTN_FWD_TILE=<policy> can force that tile policy at head_dim."""
    return bool(_lib.load().attn_fwd_tile_policy_compiled(int(policy), int(head_dim)))


def _ws_args(ws):
    if ws is None:
        return None, 0
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return _ptr(ws), int(ws.numel() * ws.element_size())


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen: int,
                    scale: Optional[float] = None, causal: bool = False,
                    out=None, lse=None, return_lse: bool = True, stream=None,
                    workspace=None):
    """Packed variable-length attention.  q (Tq, Hq, D), k/v (Tk, Hkv, D) bf16.

    ``workspace`` (optional, see ``workspace()``) lets the library split the
    key loop of long query blocks over several workgroups.
    Returns (out (Tq, Hq, D) fp32, lse (Hq, Tq) fp32 or None).
    """
    torch = _torch()
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(n, t)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or k.shape != v.shape:
        raise ValueError("q must be (Tq, Hq, D) and k, v (Tk, Hkv, D)")
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    if dk != d:
        raise ValueError("head_dim of q and k differ")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((tq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
            cu_seqlens_q.numel() - 1, tq, tk, hq, hkv, d, int(max_seqlen),
            float(scale), int(bool(causal)), _ptr(out), _ptr(lse))
    if workspace is None:
        st = lib.attn_fwd_varlen(*args, _stream_ptr(q.device, stream))
        _lib.check("attn_fwd_varlen", st)
    else:
        st = lib.attn_fwd_varlen_ws(*args, *_ws_args(workspace), _stream_ptr(q.device, stream))
        _lib.check("attn_fwd_varlen_ws", st)
    return out, lse


def attn_fwd_dense(q, k, v, scale: Optional[float] = None, causal: bool = False,
                   out=None, lse=None, return_lse: bool = True, stream=None, workspace=None):
    """Dense batched attention.  q (B, Sq, Hq, D), k/v (B, Sk, Hkv, D) bf16.

    Non-contiguous q/k/v/out are accepted when the head_dim stride is 1 (their
    strides are passed through).  Returns (out (B, Sq, Hq, D) fp32, lse
    (B, Hq, Sq) fp32 or None).
    """
    torch = _torch()
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise ValueError(f"{n} must be a bfloat16 GPU tensor")
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{n} must be 4-D with a unit head_dim stride")
    b, sq, hq, d = q.shape
    _, sk, hkv, _ = k.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[3] != d:
        raise ValueError("k and v must be (B, Sk, Hkv, D) matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((b, sq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    strides = (ctypes.c_int64 * 12)(*(list(q.stride()[:3]) + list(k.stride()[:3]) +
                                      list(v.stride()[:3]) + list(out.stride()[:3])))
    args = (_ptr(q), _ptr(k), _ptr(v), b, sq, sk, hq, hkv, d,
            ctypes.cast(strides, ctypes.c_void_p), float(scale), int(bool(causal)),
            _ptr(out), _ptr(lse))
    if workspace is None:
        st = lib.attn_fwd_dense(*args, _stream_ptr(q.device, stream))
        _lib.check("attn_fwd_dense", st)
    else:
        st = lib.attn_fwd_dense_ws(*args, *_ws_args(workspace), _stream_ptr(q.device, stream))
        _lib.check("attn_fwd_dense_ws", st)
    return out, lse


def attn_fwd_padded(q, k, v, indices, cu_seqlens, max_seqlen: int,
                    scale: Optional[float] = None, causal: bool = False,
                    out=None, lse=None, return_lse: bool = True, stream=None):
    """The padded path in one call: q (..., Hq, D), k/v (..., Hkv, D) padded bf16
    (leading dims flattened to rows), int32 ``indices`` of the valid rows and
    ``cu_seqlens`` over them.  Returns (out shaped like q, fp32, padding rows
    +0.0; lse (Hq, n_valid) fp32 or None)."""
    torch = _torch()
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(n, t)
    if k.shape != v.shape or q.shape[:-2] != k.shape[:-2] or q.shape[-1] != k.shape[-1]:
        raise ValueError("q (..., Hq, D) and k, v (..., Hkv, D) must share leading dims and D")
    for n, t in (("indices", indices), ("cu_seqlens", cu_seqlens)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    hq, d = q.shape[-2], q.shape[-1]
    hkv = k.shape[-2]
    n_rows = int(math.prod(q.shape[:-2]))
    n_valid = indices.numel()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, n_valid), dtype=torch.float32, device=q.device)
    st = lib.attn_fwd_padded(_ptr(q), _ptr(k), _ptr(v), _ptr(indices), _ptr(cu_seqlens),
                             cu_seqlens.numel() - 1, n_valid, n_rows, hq, hkv, d,
                             int(max_seqlen), float(scale), int(bool(causal)), _ptr(out),
                             _ptr(lse), _stream_ptr(q.device, stream))
    _lib.check("attn_fwd_padded", st)
    return out, lse


def attn_unpad_gather(srcs: Sequence, indices, row_dims: int = 2, outs=None,
                      stream=None) -> List:
    """Gathers rows of 1..3 tensors by one shared int32 index list.

    A row is the trailing ``row_dims`` dimensions (H, D by default), so a
    (B, total_len, H, D) tensor has B * total_len rows.  Returns one
    (n_valid, *row_shape) tensor per source.
    """
    torch = _torch()
    lib = _lib.load()
    srcs = list(srcs)
    if not 1 <= len(srcs) <= 3:
        raise ValueError("between 1 and 3 tensors per call")
    if indices.dtype != torch.int32 or not indices.is_cuda or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous int32 GPU tensor")
    row_shape = tuple(srcs[0].shape[-row_dims:])
    row_bytes = int(math.prod(row_shape)) * srcs[0].element_size()
    n_rows = srcs[0].numel() // max(1, int(math.prod(row_shape)))
    for s in srcs:
        if not s.is_cuda or not s.is_contiguous():
            raise ValueError("sources must be contiguous GPU tensors")
        if tuple(s.shape[-row_dims:]) != row_shape or s.dtype != srcs[0].dtype \
                or s.numel() != srcs[0].numel():
            raise ValueError("all sources must share shape and dtype")
    n_valid = indices.numel()
    if outs is None:
        outs = [torch.empty((n_valid,) + row_shape, dtype=s.dtype, device=s.device) for s in srcs]
    src_arr = (ctypes.c_void_p * len(srcs))(*[_ptr(s) for s in srcs])
    dst_arr = (ctypes.c_void_p * len(outs))(*[_ptr(o) for o in outs])
    st = lib.attn_unpad_gather(ctypes.cast(src_arr, ctypes.c_void_p),
                               ctypes.cast(dst_arr, ctypes.c_void_p), len(srcs), _ptr(indices),
                               n_valid, n_rows, row_bytes, _stream_ptr(srcs[0].device, stream))
    _lib.check("attn_unpad_gather", st)
    return outs


def attn_pad_scatter(src, indices, n_rows_total: int, out_shape: Optional[Tuple[int, ...]] = None,
                     out=None, stream=None):
    """Scatters compact rows (n_valid, *row_shape) back to n_rows_total rows.

    Rows that no index names are written as zeros.  ``out_shape`` (default
    (n_rows_total, *row_shape)) reshapes the result, e.g. to (B, total_len, H, D).
    """
    torch = _torch()
    lib = _lib.load()
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    if indices.dtype != torch.int32 or not indices.is_cuda or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous int32 GPU tensor")
    n_valid = indices.numel()
    if src.shape[0] != n_valid:
        raise ValueError("src must have one row per index")
    row_shape = tuple(src.shape[1:])
    row_bytes = int(math.prod(row_shape)) * src.element_size()
    if out is None:
        shape = out_shape if out_shape is not None else (n_rows_total,) + row_shape
        out = torch.empty(shape, dtype=src.dtype, device=src.device)
    st = lib.attn_pad_scatter(_ptr(src), _ptr(out), _ptr(indices), n_valid, int(n_rows_total),
                              row_bytes, _stream_ptr(src.device, stream))
    _lib.check("attn_pad_scatter", st)
    return out


def attn_bwd_workspace_bytes(total_q: int, num_heads_q: int) -> int:
    """Bytes of workspace the backward calls need (4 per query row and head)."""
    return int(_lib.load().attn_bwd_workspace_bytes(int(total_q), int(num_heads_q)))


def _bwd_outputs(q, k, v, dq, dk, dv, ws, total_q, hq):
    torch = _torch()
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    for n, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != ref.shape:
            raise ValueError(f"{n} must be a contiguous fp32 tensor shaped like its input")
    if ws is None:
        ws = torch.empty(max(attn_bwd_workspace_bytes(total_q, hq), 16), dtype=torch.uint8,
                         device=q.device)
    return dq, dk, dv, ws


def _check_fp32(name, t, shape):
    torch = _torch()
    if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous fp32 GPU tensor of shape {tuple(shape)}")


def attn_bwd_varlen(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                    max_seqlen_k: Optional[int] = None, scale: Optional[float] = None,
                    causal: bool = False, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of attn_fwd_varlen.  out / lse are that call's results for the
    same inputs; dout (Tq, Hq, D) bf16 is the gradient of out.
    Returns (dq, dk, dv) fp32 shaped like q, k, v."""
    torch = _torch()
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_bf16(n, t)
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or dout.shape != q.shape:
        raise ValueError("q, dout must be (Tq, Hq, D) and k, v (Tk, Hkv, D)")
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    _check_fp32("out", out, q.shape)
    _check_fp32("lse", lse, (hq, tq))
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if max_seqlen_k is None:
        max_seqlen_k = max_seqlen_q
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv, ws = _bwd_outputs(q, k, v, dq, dk, dv, workspace, tq, hq)
    st = lib.attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                             _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), cu_seqlens_q.numel() - 1,
                             tq, tk, hq, hkv, d, int(max_seqlen_q), int(max_seqlen_k),
                             float(scale), int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv),
                             *_ws_args(ws), _stream_ptr(q.device, stream))
    _lib.check("attn_bwd_varlen", st)
    return dq, dk, dv


def attn_bwd_dense(q, k, v, out, lse, dout, scale: Optional[float] = None, causal: bool = False,
                   dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of attn_fwd_dense for contiguous q, k, v (B, S, H, D) bf16.
    Returns (dq, dk, dv) fp32 shaped like q, k, v."""
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_bf16(n, t)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or dout.shape != q.shape:
        raise ValueError("q, dout must be (B, Sq, Hq, D) and k, v (B, Sk, Hkv, D)")
    b, sq, hq, d = q.shape
    _, sk, hkv, _ = k.shape
    _check_fp32("out", out, q.shape)
    _check_fp32("lse", lse, (b, hq, sq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv, ws = _bwd_outputs(q, k, v, dq, dk, dv, workspace, b * sq, hq)
    st = lib.attn_bwd_dense(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), b, sq,
                            sk, hq, hkv, d, float(scale), int(bool(causal)), _ptr(dq), _ptr(dk),
                            _ptr(dv), *_ws_args(ws), _stream_ptr(q.device, stream))
    _lib.check("attn_bwd_dense", st)
    return dq, dk, dv


def attn_fwd_paged_workspace_bytes(num_seqs: int, max_seqlen_q: int, max_seqlen_k: int,
                                   num_heads_q: int, num_heads_k: int, head_dim: int) -> int:
    """Bytes of workspace that let attn_fwd_paged split long key ranges (0: none)."""
    return int(_lib.load().attn_fwd_paged_workspace_bytes(int(num_seqs), int(max_seqlen_q),
                                                           int(max_seqlen_k), int(num_heads_q),
                                                           int(num_heads_k), int(head_dim)))


def paged_workspace(num_seqs: int, max_seqlen_q: int, max_seqlen_k: int, num_heads_q: int,
                    num_heads_k: int, head_dim: int, device="cuda"):
    """A device buffer of attn_fwd_paged_workspace_bytes, or None when none is needed."""
    n = attn_fwd_paged_workspace_bytes(num_seqs, max_seqlen_q, max_seqlen_k, num_heads_q,
                                       num_heads_k, head_dim)
    if n <= 0:
        return None
    return _torch().empty(n, dtype=_torch().uint8, device=device)


def attn_fwd_paged(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table,
                   max_seqlen_q: int, max_seqlen_k: int, scale: Optional[float] = None,
                   causal: bool = True, out=None, lse=None, return_lse: bool = True,
                   workspace=None, stream=None):
    """New queries q (Tq, Hq, D) bf16 over a paged cache k_cache / v_cache
    (num_pages, page_size, Hkv, D) bf16 with block_table (num_seqs, max_pages)
    and seqlens_k (num_seqs) int32.  Returns (out (Tq, Hq, D) fp32, lse (Hq, Tq)
    fp32 or None)."""
    torch = _torch()
    lib = _lib.load()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_bf16(n, t)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be (Tq, Hq, D) and the caches (num_pages, page_size, Hkv, D)")
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("seqlens_k", seqlens_k),
                 ("block_table", block_table)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    tq, hq, d = q.shape
    num_pages, page_size, hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError("head_dim of q and the caches differ")
    nseq = cu_seqlens_q.numel() - 1
    if seqlens_k.numel() != nseq or block_table.dim() != 2 or block_table.shape[0] != nseq:
        raise ValueError("seqlens_k must be (num_seqs,) and block_table (num_seqs, max_pages)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((tq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    ws_ptr, ws_bytes = _ws_args(workspace)
    st = lib.attn_fwd_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q),
                            _ptr(seqlens_k), _ptr(block_table), nseq, tq, num_pages, page_size,
                            block_table.shape[1], hq, hkv, d, int(max_seqlen_q),
                            int(max_seqlen_k), float(scale), int(bool(causal)), _ptr(out),
                            _ptr(lse), ws_ptr, ws_bytes, _stream_ptr(q.device, stream))
    _lib.check("attn_fwd_paged", st)
    return out, lse


def attn_fwd_paged_noalloc(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table,
                           max_seqlen_q: int, max_seqlen_k: int, out, lse=None,
                           scale: Optional[float] = None, causal: bool = True, stream=None):
    """attn_fwd_paged with the library's own static scratch instead of a
    workspace; `out` (Tq, Hq, D) fp32 and `lse` (Hq, Tq) fp32 or None are
    passed in, so this call allocates nothing."""
    torch = _torch()
    lib = _lib.load()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_bf16(n, t)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be (Tq, Hq, D) and the caches (num_pages, page_size, Hkv, D)")
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("seqlens_k", seqlens_k),
                 ("block_table", block_table)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    tq, hq, d = q.shape
    num_pages, page_size, hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError("head_dim of q and the caches differ")
    nseq = cu_seqlens_q.numel() - 1
    if seqlens_k.numel() != nseq or block_table.dim() != 2 or block_table.shape[0] != nseq:
        raise ValueError("seqlens_k must be (num_seqs,) and block_table (num_seqs, max_pages)")
    _check_fp32("out", out, (tq, hq, d))
    if lse is not None:
        _check_fp32("lse", lse, (hq, tq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.attn_fwd_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q),
                                    _ptr(seqlens_k), _ptr(block_table), nseq, tq, num_pages,
                                    page_size, block_table.shape[1], hq, hkv, d,
                                    int(max_seqlen_q), int(max_seqlen_k), float(scale),
                                    int(bool(causal)), _ptr(out), _ptr(lse),
                                    _stream_ptr(q.device, stream))
    _lib.check("attn_fwd_paged_noalloc", st)
    return out, lse


def attn_mask_to_varlen(mask, stream=None):
    """mask (B, L) bool/uint8/int8 GPU tensor, nonzero = valid row.  Returns
    (indices (B*L,) int32 whose first n_valid entries are the valid rows,
    cu_seqlens (B+1,) int32, stats (2,) int32 = [n_valid, max_seqlen]), all on
    the GPU; nothing is synchronised."""
    torch = _torch()
    lib = _lib.load()
    if not mask.is_cuda or mask.dim() != 2 or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous 2-D GPU tensor")
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    if mask.element_size() != 1:
        raise ValueError("mask must hold bytes (bool, uint8 or int8)")
    b, l = mask.shape
    indices = torch.empty(max(b * l, 1), dtype=torch.int32, device=mask.device)
    cu = torch.empty(b + 1, dtype=torch.int32, device=mask.device)
    stats = torch.empty(2, dtype=torch.int32, device=mask.device)
    st = lib.attn_mask_to_varlen(_ptr(mask), b, l, _ptr(indices), _ptr(cu), _ptr(stats),
                                 _stream_ptr(mask.device, stream))
    _lib.check("attn_mask_to_varlen", st)
    return indices, cu, stats


def _check_u8(name, t):
    torch = _torch()
    if not t.is_cuda or t.element_size() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor of E4M3 bytes "
                         "(uint8 or float8_e4m3fn)")
    if t.dtype not in (torch.uint8, torch.int8, getattr(torch, "float8_e4m3fn", torch.uint8)):
        raise ValueError(f"{name} must hold E4M3 bytes")


def attn_fwd_fp8_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen: int,
                        scale: Optional[float] = None, q_scale: float = 1.0, k_scale: float = 1.0,
                        v_scale: float = 1.0, causal: bool = False, out=None, lse=None,
                        return_lse: bool = True, stream=None):
    """Packed attention on E4M3 bytes q (Tq, Hq, D), k/v (Tk, Hkv, D) with
    per-tensor factors.  Returns (out fp32, lse (Hq, Tq) fp32 or None)."""
    torch = _torch()
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_u8(n, t)
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError("q must be (Tq, Hq, D) and k, v (Tk, Hkv, D)")
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((tq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    st = lib.attn_fwd_fp8_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                 cu_seqlens_q.numel() - 1, tq, tk, hq, hkv, d, int(max_seqlen),
                                 float(scale), float(q_scale), float(k_scale), float(v_scale),
                                 int(bool(causal)), _ptr(out), _ptr(lse),
                                 _stream_ptr(q.device, stream))
    _lib.check("attn_fwd_fp8_varlen", st)
    return out, lse


def attn_fwd_fp8_dense(q, k, v, scale: Optional[float] = None, q_scale: float = 1.0,
                       k_scale: float = 1.0, v_scale: float = 1.0, causal: bool = False, out=None,
                       lse=None, return_lse: bool = True, stream=None):
    """Dense attention on E4M3 bytes q (B, Sq, Hq, D), k/v (B, Sk, Hkv, D),
    contiguous.  Returns (out (B, Sq, Hq, D) fp32, lse (B, Hq, Sq) fp32 or None)."""
    torch = _torch()
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_u8(n, t)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or q.shape[3] != k.shape[3]:
        raise ValueError("q must be (B, Sq, Hq, D) and k, v (B, Sk, Hkv, D)")
    b, sq, hq, d = q.shape
    _, sk, hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((b, sq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    st = lib.attn_fwd_fp8_dense(_ptr(q), _ptr(k), _ptr(v), b, sq, sk, hq, hkv, d, float(scale),
                                float(q_scale), float(k_scale), float(v_scale), int(bool(causal)),
                                _ptr(out), _ptr(lse), _stream_ptr(q.device, stream))
    _lib.check("attn_fwd_fp8_dense", st)
    return out, lse


def attn_fwd_paged_fp8kv(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table,
                         max_seqlen_q: int, max_seqlen_k: int, scale: Optional[float] = None,
                         k_scale: float = 1.0, v_scale: float = 1.0, causal: bool = True,
                         out=None, lse=None, return_lse: bool = True, workspace=None,
                         stream=None):
    """attn_fwd_paged over E4M3 caches (num_pages, page_size, Hkv, D) bytes with
    per-tensor factors; q (Tq, Hq, D) bf16.  Returns (out fp32, lse or None)."""
    torch = _torch()
    lib = _lib.load()
    _check_bf16("q", q)
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _check_u8(n, t)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be (Tq, Hq, D) and the caches (num_pages, page_size, Hkv, D)")
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("seqlens_k", seqlens_k),
                 ("block_table", block_table)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 GPU tensor")
    tq, hq, d = q.shape
    num_pages, page_size, hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError("head_dim of q and the caches differ")
    nseq = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((tq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    ws_ptr, ws_bytes = _ws_args(workspace)
    st = lib.attn_fwd_paged_fp8kv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q),
                                  _ptr(seqlens_k), _ptr(block_table), nseq, tq, num_pages,
                                  page_size, block_table.shape[1], hq, hkv, d, int(max_seqlen_q),
                                  int(max_seqlen_k), float(scale), float(k_scale), float(v_scale),
                                  int(bool(causal)), _ptr(out), _ptr(lse), ws_ptr, ws_bytes,
                                  _stream_ptr(q.device, stream))
    _lib.check("attn_fwd_paged_fp8kv", st)
    return out, lse
