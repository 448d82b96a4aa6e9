"""ctypes view of libkvc.so (the C ABI in include/kvc.h).

Argument marshalling only.  The library is loaded on first use; if it is
missing the call raises, there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvc.so")

KVC_OK = 0
KVC_ERR_INVALID_ARGUMENT = -1
KVC_ERR_OUT_OF_PAGES = -2
KVC_ERR_NO_UNDO = -3
KVC_ERR_BUFFER_TOO_SMALL = -4
KVC_ERR_UNSUPPORTED = -5
KVC_ERR_DEVICE = -6
KVC_ERR_HOST_MEMORY = -7
KVC_ERR_INTERNAL = -8

KVC_DTYPE_BF16 = 0
KVC_DTYPE_F32 = 1
KVC_DTYPE_FP8_E4M3 = 2
KVC_SPECIAL_FRAME_ALIGNED = 0
KVC_SPECIAL_CONTIGUOUS = 1

EXPORTED = (
    "kvc_required_pages", "kvc_pool_bytes", "kvc_create", "kvc_destroy", "kvc_append_frame",
    "kvc_rollback_last_frame", "kvc_reset", "kvc_build_visible_table", "kvc_get_state",
    "paged_attn_workspace_size", "paged_attn_num_splits", "paged_attn_fwd", "paged_attn_merge",
    "kvc_attend", "kvc_attend_workspace_size", "kvc_attend_batch", "kvc_attend_batch_workspace_size",
    "kvc_build_subset_table", "kvc_attend_subset", "kvc_attend_noalloc",
    "kvc_windowed_ring_bytes", "kvc_windowed_create", "kvc_windowed_destroy", "kvc_windowed_append",
    "kvc_windowed_keep", "kvc_windowed_drop", "kvc_windowed_get_state",
    "kvc_strerror", "kvc_last_error", "kvc_version", "kvc_set_kernel_events",
    # include/kvc_probe.h
    "kvc_probe_scratch_bytes", "kvc_probe_mfma_bf16", "kvc_probe_tile_mix", "kvc_probe_hbm",
)
MAX_INLINE_PAGES = 640
NOALLOC_SCRATCH_BYTES = 32 << 20
MAX_BATCH_CACHES = 16


class KvcConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "num_heads", "head_dim", "page_size", "dtype", "patch_tokens", "special_tokens",
        "num_scale_units", "window_units", "special_packing", "max_units", "num_pages")]


class KvcState(C.Structure):
    _fields_ = [
        ("capacity", C.c_int32),
        ("free_pages", C.POINTER(C.c_int32)),
        ("scale_pages", C.POINTER(C.c_int32)),
        ("window_pages", C.POINTER(C.c_int32)),
        ("special_pages", C.POINTER(C.c_int32)),
        ("num_free", C.c_int32),
        ("num_scale_pages", C.c_int32),
        ("num_window_pages", C.c_int32),
        ("num_window_units", C.c_int32),
        ("num_special_pages", C.c_int32),
        ("special_fill", C.c_int32),
        ("num_units", C.c_int32),
        ("has_undo", C.c_int32),
        ("num_pages", C.c_int32),
    ]


class KvcWindowedState(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("slots", "windows", "ring_units", "pending")]


class PagedAttnArgs(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32),
        ("num_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("page_size", C.c_int32),
        ("sm_scale", C.c_float),
        ("num_seqs", C.c_int32),
        ("total_q", C.c_int32),
        ("max_qo_len", C.c_int32),
        ("max_kv_pages", C.c_int32),
        ("num_pool_pages", C.c_int32),
        ("num_splits", C.c_int32),
        ("qo_indptr", C.c_void_p),
        ("kv_indptr", C.c_void_p),
        ("page_ids", C.c_void_p),
        ("page_lens", C.c_void_p),
        ("q", C.c_void_p),
        ("k_pool", C.c_void_p),
        ("v_pool", C.c_void_p),
        ("o", C.c_void_p),
        ("lse", C.c_void_p),
        ("workspace", C.c_void_p),
        ("workspace_bytes", C.c_size_t),
    ]


class KvcError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


class OutOfPages(KvcError):
    pass


class NoUndo(KvcError):
    pass


_lib = None
_lock = threading.Lock()


def _declare(lib):
    i32, vp, i32p = C.c_int32, C.c_void_p, C.POINTER(C.c_int32)
    sig = {
        "kvc_required_pages": (C.c_int, [C.POINTER(KvcConfig), i32p]),
        "kvc_pool_bytes": (C.c_int, [C.POINTER(KvcConfig), C.POINTER(C.c_size_t)]),
        "kvc_create": (C.c_int, [C.POINTER(KvcConfig), vp, vp, C.POINTER(vp)]),
        "kvc_destroy": (C.c_int, [vp]),
        "kvc_append_frame": (C.c_int, [vp, vp, vp, vp]),
        "kvc_rollback_last_frame": (C.c_int, [vp]),
        "kvc_reset": (C.c_int, [vp]),
        "kvc_build_visible_table": (C.c_int, [vp, i32p, i32p, i32, i32p, i32p]),
        "kvc_get_state": (C.c_int, [vp, C.POINTER(KvcState)]),
        "paged_attn_workspace_size": (C.c_int, [C.POINTER(PagedAttnArgs), C.POINTER(C.c_size_t)]),
        "paged_attn_num_splits": (C.c_int, [C.POINTER(PagedAttnArgs), i32p]),
        "paged_attn_fwd": (C.c_int, [C.POINTER(PagedAttnArgs), vp]),
        "paged_attn_merge": (C.c_int, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]),
        "kvc_attend": (C.c_int, [vp, vp, i32, C.c_float, vp, vp, vp, C.c_size_t, vp]),
        "kvc_attend_workspace_size": (C.c_int, [vp, i32, C.POINTER(C.c_size_t)]),
        "kvc_build_subset_table": (C.c_int, [vp, C.c_float, C.c_uint64, i32, i32, i32p, i32p, i32, i32p]),
        "kvc_attend_subset": (C.c_int, [vp, C.c_float, C.c_uint64, i32, i32, vp, i32, C.c_float, vp, vp, vp,
                                        C.c_size_t, vp]),
        "kvc_attend_batch": (C.c_int, [C.POINTER(vp), i32, vp, i32p, C.c_float, vp, vp, vp, C.c_size_t, vp]),
        "kvc_attend_batch_workspace_size": (C.c_int, [C.POINTER(vp), i32, i32p, C.POINTER(C.c_size_t)]),
        "kvc_attend_noalloc": (C.c_int, [vp, vp, i32, C.c_float, vp, vp, vp]),
        "kvc_windowed_ring_bytes": (C.c_int, [vp, i32, C.POINTER(C.c_size_t)]),
        "kvc_windowed_create": (C.c_int, [vp, i32, i32, vp, vp, C.POINTER(vp)]),
        "kvc_windowed_destroy": (C.c_int, [vp]),
        "kvc_windowed_append": (C.c_int, [vp, vp, vp, vp, i32p]),
        "kvc_windowed_keep": (C.c_int, [vp, vp]),
        "kvc_windowed_drop": (C.c_int, [vp]),
        "kvc_windowed_get_state": (C.c_int, [vp, C.POINTER(KvcWindowedState)]),
        "kvc_set_kernel_events": (C.c_int, [vp, vp]),
        "kvc_probe_scratch_bytes": (C.c_size_t, []),
        "kvc_probe_mfma_bf16": (C.c_int, [vp, C.c_size_t, vp, C.POINTER(C.c_double)]),
        "kvc_probe_tile_mix": (C.c_int, [vp, C.c_size_t, vp, C.POINTER(C.c_double)]),
        "kvc_probe_hbm": (C.c_int, [vp, vp, C.c_size_t, vp, C.c_size_t, vp, C.POINTER(C.c_double),
                                    C.POINTER(C.c_double)]),
        "kvc_strerror": (C.c_char_p, [C.c_int]),
        "kvc_last_error": (C.c_char_p, []),
        "kvc_version": (C.c_int, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with `python -m paged_sliding_window_kv_amd.build`")
                l = C.CDLL(LIB_PATH)
                _declare(l)
                _lib = l
    return _lib


def check(status: int, where: str) -> None:
    if status == KVC_OK:
        return
    msg = lib().kvc_last_error().decode(errors="replace")
    cls = {KVC_ERR_OUT_OF_PAGES: OutOfPages, KVC_ERR_NO_UNDO: NoUndo}.get(status, KvcError)
    raise cls(status, where, msg or lib().kvc_strerror(status).decode())
