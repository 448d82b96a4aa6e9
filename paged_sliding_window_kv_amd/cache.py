"""Python handle over one layer's paged KV cache (libkvc.so).

Marshalling only: page planning, the visible table and rollback run in the
library's C++ host code, the K/V scatter and the attention in its HIP
kernels.  PyTorch provides the device memory (the two pools) and the stream.
"""
from __future__ import annotations

import contextlib
import ctypes as C
from typing import Optional, Tuple

import numpy as np

from . import _lib as L

_DTYPES = {"bf16": L.KVC_DTYPE_BF16, "f32": L.KVC_DTYPE_F32, "fp8": L.KVC_DTYPE_FP8_E4M3}
_PACKING = {"frame_aligned": L.KVC_SPECIAL_FRAME_ALIGNED, "contiguous": L.KVC_SPECIAL_CONTIGUOUS}


def _torch():
    import torch
    return torch


def torch_dtype(dtype: str):
    """Activation dtype (K/V appended, q, o) of a cache dtype; FP8 caches take and give bf16."""
    t = _torch()
    return {"bf16": t.bfloat16, "f32": t.float32, "fp8": t.bfloat16}[dtype]


def current_stream_ptr(device=None) -> int:
    t = _torch()
    return t.cuda.current_stream(device).cuda_stream


def on_stream(stream: Optional[int], device):
    """Context that makes `stream` (a raw stream pointer) torch's current stream.

    Tensors allocated and copies made inside it are ordered on that stream, the
    one the library launches on, so the caching allocator does not hand their
    memory out again while the stream still reads it.  None (or the current
    stream) changes nothing.
    """
    t = _torch()
    if stream is None or stream == t.cuda.current_stream(device).cuda_stream:
        return contextlib.nullcontext()
    return t.cuda.stream(t.cuda.ExternalStream(stream, device=device))


class KvCache:
    """One layer's cache.

    device=None gives a host-only handle: appends take no data and only the
    page metadata moves (useful to check tables without a GPU).  Otherwise the
    K pool [num_pages, H, P, d] and the V pool [num_pages, H, d, P] are
    allocated on `device` and appends scatter device K/V into them.
    dtype "fp8": the pools are flat uint8 buffers of OCP E4M3 codes, both
    slot-major [num_pages, H, P, d], followed by int8 row exponents
    [num_pages, H, P] (views: k_codes, k_exps, v_codes, v_exps); appends
    take bf16 K/V and quantise them, attention takes bf16 q.
    """

    def __init__(self, num_heads: int, head_dim: int = 64, page_size: int = 256, dtype: str = "bf16",
                 patch_tokens: int = 256, special_tokens: int = 6, num_scale_units: int = 8,
                 window_units: int = 64, special_packing: str = "frame_aligned", max_units: int = 1000,
                 num_pages: int = 0, device=None, pools=None):
        self.cfg = L.KvcConfig(num_heads, head_dim, page_size, _DTYPES[dtype], patch_tokens, special_tokens,
                               num_scale_units, window_units, _PACKING[special_packing], max_units, num_pages)
        self.dtype = dtype
        self.num_heads, self.head_dim, self.page_size = num_heads, head_dim, page_size
        self.patch_tokens, self.special_tokens = patch_tokens, special_tokens
        self.unit_tokens = patch_tokens + special_tokens
        lib = L.lib()
        n = C.c_int32(num_pages)
        if num_pages == 0:
            L.check(lib.kvc_required_pages(C.byref(self.cfg), C.byref(n)), "kvc_required_pages")
        self.num_pages = n.value
        self.device = device
        self.k_pool = self.v_pool = None
        if dtype == "fp8":
            if pools is not None:
                raise ValueError("FP8 caches allocate their own pools")
            if device is not None:
                t = _torch()
                nb = C.c_size_t()
                L.check(lib.kvc_pool_bytes(C.byref(self.cfg), C.byref(nb)), "kvc_pool_bytes")
                self.k_pool = t.empty(nb.value, dtype=t.uint8, device=device)
                self.v_pool = t.empty(nb.value, dtype=t.uint8, device=device)
        elif pools is not None:
            # caller-owned pool tensors (e.g. page slices of a pool shared by a batch)
            k_pool, v_pool = pools
            want_k = (self.num_pages, num_heads, page_size, head_dim)
            want_v = (self.num_pages, num_heads, head_dim, page_size)
            if tuple(k_pool.shape) != want_k or tuple(v_pool.shape) != want_v:
                raise ValueError(f"pools must have shapes {want_k} and {want_v}")
            if not (k_pool.is_contiguous() and v_pool.is_contiguous()):
                raise ValueError("pools must be contiguous")
            if k_pool.dtype != torch_dtype(dtype) or v_pool.dtype != torch_dtype(dtype):
                raise ValueError(f"pools must be {dtype}")
            self.k_pool, self.v_pool = k_pool, v_pool
            self.device = k_pool.device
        elif device is not None:
            t = _torch()
            td = torch_dtype(dtype)
            self.k_pool = t.empty((self.num_pages, num_heads, page_size, head_dim), dtype=td, device=device)
            self.v_pool = t.empty((self.num_pages, num_heads, head_dim, page_size), dtype=td, device=device)
        h = C.c_void_p()
        L.check(lib.kvc_create(C.byref(self.cfg), self._ptr(self.k_pool), self._ptr(self.v_pool), C.byref(h)),
                "kvc_create")
        if dtype == "fp8" and self.k_pool is not None:
            ncode = self.num_pages * num_heads * page_size * head_dim
            shp = (self.num_pages, num_heads, page_size, head_dim)
            t = _torch()
            self.k_codes = self.k_pool[:ncode].view(shp)
            self.v_codes = self.v_pool[:ncode].view(shp)
            self.k_exps = self.k_pool[ncode:].view(t.int8).view(shp[:3])
            self.v_exps = self.v_pool[ncode:].view(t.int8).view(shp[:3])
        self._h = h
        self._ids = np.zeros(self.num_pages, np.int32)
        self._lens = np.zeros(self.num_pages, np.int32)

    @staticmethod
    def _ptr(t) -> Optional[int]:
        return None if t is None else t.data_ptr()

    @property
    def handle(self) -> C.c_void_p:
        return self._h

    def close(self) -> None:
        if getattr(self, "_h", None):
            L.lib().kvc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- stream operations ------------------------------------------------------
    def append(self, k=None, v=None, stream: Optional[int] = None) -> None:
        """Append one unit.  k, v: [patch + special, H, d] device tensors in the cache dtype."""
        if self.device is None:
            if k is not None or v is not None:
                raise ValueError("host-only cache takes no K/V")
            L.check(L.lib().kvc_append_frame(self._h, None, None, None), "kvc_append_frame")
            return
        self._check_unit(k, "k")
        self._check_unit(v, "v")
        s = current_stream_ptr(k.device) if stream is None else stream
        L.check(L.lib().kvc_append_frame(self._h, k.data_ptr(), v.data_ptr(), s), "kvc_append_frame")

    def _check_unit(self, x, name):
        t = _torch()
        want = (self.unit_tokens, self.num_heads, self.head_dim)
        if not isinstance(x, t.Tensor) or tuple(x.shape) != want:
            raise ValueError(f"{name} must be a tensor of shape {want}")
        if x.dtype != torch_dtype(self.dtype) or not x.is_contiguous() or x.device != self.k_pool.device:
            raise ValueError(f"{name} must be a contiguous {self.dtype} tensor on {self.k_pool.device}")

    def rollback(self) -> None:
        L.check(L.lib().kvc_rollback_last_frame(self._h), "kvc_rollback_last_frame")

    def reset(self) -> None:
        L.check(L.lib().kvc_reset(self._h), "kvc_reset")

    # -- metadata -----------------------------------------------------------------
    def visible_table(self) -> Tuple[np.ndarray, np.ndarray]:
        n = C.c_int32()
        last = C.c_int32()
        ip = self._ids.ctypes.data_as(C.POINTER(C.c_int32))
        lp = self._lens.ctypes.data_as(C.POINTER(C.c_int32))
        L.check(L.lib().kvc_build_visible_table(self._h, ip, lp, self.num_pages, C.byref(n), C.byref(last)),
                "kvc_build_visible_table")
        return self._ids[:n.value].copy(), self._lens[:n.value].copy()

    def subset_table(self, keep_ratio: float, seed: int, keep_first: int = 0,
                     keep_last: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Page-subset of the visible table (kvc_build_subset_table)."""
        n = C.c_int32()
        ip = self._ids.ctypes.data_as(C.POINTER(C.c_int32))
        lp = self._lens.ctypes.data_as(C.POINTER(C.c_int32))
        L.check(L.lib().kvc_build_subset_table(self._h, float(keep_ratio), int(seed) & (2**64 - 1), keep_first,
                                               keep_last, ip, lp, self.num_pages, C.byref(n)),
                "kvc_build_subset_table")
        return self._ids[:n.value].copy(), self._lens[:n.value].copy()

    def state(self) -> dict:
        cap = self.num_pages
        bufs = [np.zeros(cap, np.int32) for _ in range(4)]
        st = L.KvcState()
        st.capacity = cap
        st.free_pages, st.scale_pages, st.window_pages, st.special_pages = (
            b.ctypes.data_as(C.POINTER(C.c_int32)) for b in bufs)
        L.check(L.lib().kvc_get_state(self._h, C.byref(st)), "kvc_get_state")
        return {
            "free": bufs[0][:st.num_free].tolist(),
            "scale_pages": bufs[1][:st.num_scale_pages].tolist(),
            "window_pages": bufs[2][:st.num_window_pages].tolist(),
            "window_units": st.num_window_units,
            "special_pages": bufs[3][:st.num_special_pages].tolist(),
            "special_fill": st.special_fill,
            "num_units": st.num_units,
            "has_undo": bool(st.has_undo),
        }

    # -- attention ------------------------------------------------------------------
    def workspace_bytes(self, num_q: int) -> int:
        n = C.c_size_t()
        L.check(L.lib().kvc_attend_workspace_size(self._h, num_q, C.byref(n)), "kvc_attend_workspace_size")
        return n.value

    def num_splits(self, num_q: int) -> int:
        """Key splits an attention call of num_q queries over the current visible table gets (paged_attn_num_splits)."""
        n = C.c_int32()
        L.check(L.lib().kvc_build_visible_table(self._h, None, None, 0, C.byref(n), None), "kvc_build_visible_table")
        a = L.PagedAttnArgs()
        a.dtype, a.num_heads, a.head_dim, a.page_size = self.cfg.dtype, self.num_heads, self.head_dim, self.page_size
        a.sm_scale = 1.0
        a.num_seqs, a.total_q, a.max_qo_len = 1, num_q, num_q
        a.max_kv_pages, a.num_pool_pages = n.value, self.num_pages
        out = C.c_int32()
        L.check(L.lib().paged_attn_num_splits(C.byref(a), C.byref(out)), "paged_attn_num_splits")
        return out.value

    def _check_q(self, q):
        dev = self.k_pool.device
        if tuple(q.shape) != (q.shape[0], self.num_heads, self.head_dim) or not q.is_contiguous():
            raise ValueError("q must be a contiguous [Lq, H, d] tensor")
        if q.dtype != torch_dtype(self.dtype) or q.device != dev:
            raise ValueError(f"q must be {self.dtype} on {dev}")

    def _outputs(self, q, out, lse, workspace):
        """out, lse and a workspace of kvc_attend_workspace_size bytes, allocated where missing."""
        t = _torch()
        dev = self.k_pool.device
        if out is None:
            out = t.empty_like(q)
        if lse is None:
            lse = t.empty(q.shape[:2], dtype=t.float32, device=dev)
        need = self.workspace_bytes(q.shape[0])
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = t.empty(need, dtype=t.uint8, device=dev)
        wp = workspace.data_ptr() if need else None
        wb = workspace.numel() * workspace.element_size() if need else 0
        return out, lse, wp, wb

    def attend_subset(self, q, keep_ratio: float, seed: int, keep_first: int = 0, keep_last: int = 0, out=None,
                      lse=None, sm_scale: Optional[float] = None, workspace=None, stream: Optional[int] = None):
        """Attention of q [Lq, H, d] against a page subset of the visible table (kvc_attend_subset)."""
        self._check_q(q)
        dev = self.k_pool.device
        with on_stream(stream, dev):
            out, lse, wp, wb = self._outputs(q, out, lse, workspace)
            scale = 0.0 if sm_scale is None else float(sm_scale)
            L.check(L.lib().kvc_attend_subset(self._h, float(keep_ratio), int(seed) & (2**64 - 1), keep_first,
                                              keep_last, q.data_ptr(), q.shape[0], scale, out.data_ptr(),
                                              lse.data_ptr(), wp, wb, current_stream_ptr(dev)), "kvc_attend_subset")
        return out, lse

    def attend(self, q, out=None, lse=None, sm_scale: Optional[float] = None, num_splits: int = 0,
               workspace=None, stream: Optional[int] = None):
        """Attention of q [Lq, H, d] against the visible table (one sequence).

        kvc_attend builds the table in the library (in the launch arguments up
        to 640 pages, else staged into the workspace).  num_splits != 0 forces
        that split count through paged_attn_fwd with a device copy of the
        table.  Everything is allocated and enqueued on `stream` (default: the
        current stream).  Returns (out, lse).
        """
        self._check_q(q)
        dev = self.k_pool.device
        with on_stream(stream, dev):
            if num_splits == 0:
                out, lse, wp, wb = self._outputs(q, out, lse, workspace)
                scale = 0.0 if sm_scale is None else float(sm_scale)
                L.check(L.lib().kvc_attend(self._h, q.data_ptr(), q.shape[0], scale, out.data_ptr(),
                                           lse.data_ptr(), wp, wb, current_stream_ptr(dev)), "kvc_attend")
                return out, lse
            from .attention import paged_attention
            t = _torch()
            ids, lens = self.visible_table()
            page_ids = t.from_numpy(ids).to(dev)
            page_lens = t.from_numpy(lens).to(dev)
            qo = t.tensor([0, q.shape[0]], dtype=t.int32, device=dev)
            kv = t.tensor([0, len(ids)], dtype=t.int32, device=dev)
            fp8 = (self.num_pages, self.page_size) if self.dtype == "fp8" else None
            return paged_attention(q, self.k_pool, self.v_pool, page_ids, page_lens, qo, kv,
                                   max_qo_len=q.shape[0], max_kv_pages=len(ids), out=out, lse=lse,
                                   sm_scale=sm_scale, num_splits=num_splits, fp8_pages=fp8)


def shared_pool_caches(count: int, device, **cfg) -> list:
    """`count` caches with one config whose pools are page slices of one shared K and one shared V tensor.

    Such caches can attend together in one launch (attend_batch).  Keyword
    arguments are KvCache's; num_pages per cache is derived from the config
    unless given.
    """
    t = _torch()
    probe = KvCache(**cfg)  # host-only: page count and shapes
    n, H, P, d = probe.num_pages, probe.num_heads, probe.page_size, probe.head_dim
    td = torch_dtype(probe.dtype)
    probe.close()
    k_all = t.empty((count * n, H, P, d), dtype=td, device=device)
    v_all = t.empty((count * n, H, d, P), dtype=td, device=device)
    caches = []
    for i in range(count):
        c = dict(cfg)
        c["num_pages"] = n
        caches.append(KvCache(pools=(k_all[i * n:(i + 1) * n], v_all[i * n:(i + 1) * n]), **c))
    return caches


def attend_batch_workspace_bytes(caches, qo_indptr) -> int:
    hs = (C.c_void_p * len(caches))(*[c.handle.value for c in caches])
    qo = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    n = C.c_size_t()
    L.check(L.lib().kvc_attend_batch_workspace_size(hs, len(caches), qo.ctypes.data_as(C.POINTER(C.c_int32)),
                                                    C.byref(n)), "kvc_attend_batch_workspace_size")
    return n.value


def attend_batch(caches, q, qo_indptr, out=None, lse=None, sm_scale: Optional[float] = None, workspace=None,
                 stream: Optional[int] = None):
    """One launch of attention for several caches (kvc_attend_batch).

    q: [total, H, d] device tensor; rows qo_indptr[i] .. qo_indptr[i+1]-1 belong
    to caches[i].  The caches must share pools (shared_pool_caches).  Returns
    (out, lse).
    """
    t = _torch()
    c0 = caches[0]
    dev = c0.k_pool.device
    qo = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    if len(qo) != len(caches) + 1 or int(qo[-1]) != q.shape[0]:
        raise ValueError("qo_indptr must have len(caches) + 1 entries ending at q.shape[0]")
    if tuple(q.shape[1:]) != (c0.num_heads, c0.head_dim) or not q.is_contiguous():
        raise ValueError("q must be a contiguous [total, H, d] tensor")
    if q.dtype != torch_dtype(c0.dtype) or q.device != dev:
        raise ValueError(f"q must be {c0.dtype} on {dev}")
    with on_stream(stream, dev):
        if out is None:
            out = t.empty_like(q)
        if lse is None:
            lse = t.empty(q.shape[:2], dtype=t.float32, device=dev)
        need = attend_batch_workspace_bytes(caches, qo)
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = t.empty(need, dtype=t.uint8, device=dev)
        wp = workspace.data_ptr() if need else None
        wb = workspace.numel() * workspace.element_size() if need else 0
        hs = (C.c_void_p * len(caches))(*[c.handle.value for c in caches])
        scale = 0.0 if sm_scale is None else float(sm_scale)
        L.check(L.lib().kvc_attend_batch(hs, len(caches), q.data_ptr(), qo.ctypes.data_as(C.POINTER(C.c_int32)),
                                         scale, out.data_ptr(), lse.data_ptr(), wp, wb, current_stream_ptr(dev)),
                "kvc_attend_batch")
    return out, lse
