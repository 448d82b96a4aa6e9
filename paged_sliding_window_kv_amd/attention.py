"""paged_attention: marshals torch tensors into one paged_attn_fwd call."""
from __future__ import annotations

import ctypes as C
import math
from typing import Optional

from . import _lib as L


def _torch():
    import torch
    return torch


def _dtype_code(t, x) -> int:
    if x.dtype == t.bfloat16:
        return L.KVC_DTYPE_BF16
    if x.dtype == t.float32:
        return L.KVC_DTYPE_F32
    raise ValueError(f"unsupported dtype {x.dtype}")


def _ptr(x) -> Optional[int]:
    return None if x is None else x.data_ptr()


def make_args(q, k_pool, v_pool, page_ids, page_lens, qo_indptr, kv_indptr, out, lse, max_qo_len: int,
              max_kv_pages: int, sm_scale: Optional[float], num_splits: int,
              fp8_pages: Optional[tuple] = None) -> L.PagedAttnArgs:
    """fp8_pages = (num_pool_pages, page_size) when the pools are flat FP8 buffers (codes + exponents)."""
    t = _torch()
    total_q, num_heads, head_dim = q.shape
    a = L.PagedAttnArgs()
    a.dtype = L.KVC_DTYPE_FP8_E4M3 if fp8_pages is not None else _dtype_code(t, q)
    a.num_heads = num_heads
    a.head_dim = head_dim
    a.page_size = fp8_pages[1] if fp8_pages is not None else k_pool.shape[2]
    a.sm_scale = (1.0 / math.sqrt(head_dim)) if sm_scale is None else float(sm_scale)
    a.num_seqs = qo_indptr.shape[0] - 1
    a.total_q = total_q
    a.max_qo_len = int(max_qo_len)
    a.max_kv_pages = int(max_kv_pages)
    a.num_pool_pages = fp8_pages[0] if fp8_pages is not None else k_pool.shape[0]
    a.num_splits = int(num_splits)
    a.qo_indptr, a.kv_indptr = qo_indptr.data_ptr(), kv_indptr.data_ptr()
    a.page_ids, a.page_lens = _ptr(page_ids), _ptr(page_lens)
    a.q, a.k_pool, a.v_pool = q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr()
    a.o, a.lse = out.data_ptr(), _ptr(lse)
    return a


def workspace_bytes(args: L.PagedAttnArgs) -> int:
    n = C.c_size_t()
    L.check(L.lib().paged_attn_workspace_size(C.byref(args), C.byref(n)), "paged_attn_workspace_size")
    return n.value


def num_splits_for(args: L.PagedAttnArgs) -> int:
    n = C.c_int32()
    L.check(L.lib().paged_attn_num_splits(C.byref(args), C.byref(n)), "paged_attn_num_splits")
    return n.value


def paged_attention(q, k_pool, v_pool, page_ids, page_lens, qo_indptr, kv_indptr, max_qo_len: int,
                    max_kv_pages: int, out=None, lse=None, sm_scale: Optional[float] = None,
                    num_splits: int = 0, workspace=None, stream: Optional[int] = None,
                    fp8_pages: Optional[tuple] = None):
    """Softmax attention of each query sequence against its page-table entries.

    q [total_q, H, d]; k_pool [pages, H, P, d]; v_pool [pages, H, d, P];
    page_ids / page_lens / qo_indptr / kv_indptr: device int32.  Returns (out, lse).
    FP8 pools: flat uint8 buffers (codes then row exponents, layout in kvc.h)
    with fp8_pages = (num_pool_pages, page_size); q and out bf16.
    """
    t = _torch()
    for name, x in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        if not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    for name, x in (("page_ids", page_ids), ("page_lens", page_lens), ("qo_indptr", qo_indptr),
                    ("kv_indptr", kv_indptr)):
        if x.dtype != t.int32 or not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if fp8_pages is not None:
        if k_pool.dtype != t.uint8 or v_pool.dtype != t.uint8 or q.dtype != t.bfloat16:
            raise ValueError("FP8 pools are uint8 buffers and take bf16 q")
    elif k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise ValueError("q and pools must share a dtype")
    from .cache import on_stream
    with on_stream(stream, q.device):
        # outputs and workspace are allocated on the launch stream
        if out is None:
            out = t.empty_like(q)
        if lse is None:
            lse = t.empty(q.shape[:2], dtype=t.float32, device=q.device)
        a = make_args(q, k_pool, v_pool, page_ids, page_lens, qo_indptr, kv_indptr, out, lse, max_qo_len,
                      max_kv_pages, sm_scale, num_splits, fp8_pages)
        need = workspace_bytes(a)
        if need:
            if workspace is None or workspace.numel() * workspace.element_size() < need:
                workspace = t.empty(need, dtype=t.uint8, device=q.device)
            a.workspace = workspace.data_ptr()
            a.workspace_bytes = workspace.numel() * workspace.element_size()
        L.check(L.lib().paged_attn_fwd(C.byref(a), t.cuda.current_stream(q.device).cuda_stream), "paged_attn_fwd")
    return out, lse


def merge_partials(partial_o, partial_lse, out, lse=None, stream: Optional[int] = None):
    """LSE-weighted merge of split partials: partial_o [parts, rows, H, d] fp32, partial_lse [parts, rows, H]."""
    t = _torch()
    parts, rows, heads, d = partial_o.shape
    dt = _dtype_code(t, out)
    s = t.cuda.current_stream(out.device).cuda_stream if stream is None else stream  # allocates nothing
    L.check(L.lib().paged_attn_merge(dt, parts, rows, heads, d, partial_o.data_ptr(), partial_lse.data_ptr(),
                                     out.data_ptr(), _ptr(lse), s), "paged_attn_merge")
    return out, lse
