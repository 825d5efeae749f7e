"""Python binding of libqsa: query-sparse NVFP4 decode / verify attention on gfx950.

Argument marshalling only. Every step of the path runs in the HIP kernels of
`libqsa.so`, reached through the C ABI in `include/qsa.h`. The functions have the
same names and argument order as the C entry points. They take torch tensors
(for device memory) and a stream, pass raw pointers, and raise QsaError on a
non-OK status. There is no CPU fallback: if the library is missing or cannot be
loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "QsaError", "Shape", "Paged", "lib", "qsa_abi_version", "qsa_status_string",
    "qsa_index_scores", "qsa_select_topk", "qsa_workspace_bytes", "qsa_sparse_decode",
    "qsa_select_sparse_decode", "qsa_kv_store", "qsa_nvfp4_dequant_pages", "LIB_PATH", "EXPORTED",
    "Plane", "qsa_rollback_stash_bytes", "qsa_rollback_gather", "qsa_rollback_restore", "qsa_step_slots",
    "QSA_DEVERR_SLOT",
    "QSA_DEVERR_PAGE_ID", "QSA_DEVERR_SEQ_LEN", "QSA_DEVERR_ROWS", "QSA_DEVERR_Q_RANGE",
    "QSA_DEVERR_SELECTED", "DecodePlan", "qsa_plan_decode", "qsa_select_sparse_decode_static",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

QSA_OK, QSA_ERR_INVALID_ARG, QSA_ERR_UNSUPPORTED, QSA_ERR_WORKSPACE_TOO_SMALL, QSA_ERR_HIP = range(5)
QSA_DEVERR_PAGE_ID = 0x1
QSA_DEVERR_SEQ_LEN = 0x2
QSA_DEVERR_ROWS = 0x4
QSA_DEVERR_Q_RANGE = 0x8
QSA_DEVERR_SELECTED = 0x10
QSA_DEVERR_SLOT = 0x20
QSA_KV_NVFP4, QSA_KV_FP8 = 0, 1
QSA_MAX_PLANES = 16

# every symbol that include/qsa.h declares
EXPORTED = (
    "qsa_index_scores", "qsa_select_topk", "qsa_workspace_bytes", "qsa_sparse_decode", "qsa_select_sparse_decode",
    "qsa_kv_store", "qsa_rollback_stash_bytes", "qsa_step_slots", "qsa_rollback_gather", "qsa_rollback_restore",
    "qsa_nvfp4_dequant_pages", "qsa_status_string", "qsa_abi_version", "qsa_plan_decode",
    "qsa_select_sparse_decode_static",
)


class QsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = qsa_status_string(status) if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})")


class Shape(ctypes.Structure):
    """Mirror of `qsa_shape`."""
    _fields_ = [
        ("num_requests", ctypes.c_int32),
        ("num_rows", ctypes.c_int32),
        ("max_rows_per_request", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int64),
        ("topk", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("kv_format", ctypes.c_int32),
    ]


class Paged(ctypes.Structure):
    """Mirror of `qsa_paged` (device pointers as integers)."""
    _fields_ = [
        ("page_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("row_offsets", ctypes.c_void_p),
        ("k_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("index_keys", ctypes.c_void_p),
        ("k_global", ctypes.c_float),
        ("v_global", ctypes.c_float),
        ("error_word", ctypes.c_void_p),
    ]


class DecodePlan(ctypes.Structure):
    """Mirror of `qsa_decode_plan`: the launch the attention calls make for a shape."""
    _fields_ = [
        ("tile_cols", ctypes.c_int32),
        ("rows_per_tile", ctypes.c_int32),
        ("col_tiles", ctypes.c_int32),
        ("splits", ctypes.c_int32),
        ("select_cols", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("workgroups", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class Plane(ctypes.Structure):
    """Mirror of `qsa_plane`: one plane of the rollback (a device byte array and the strides
    that address row r of it: base + pages[r] * page_stride + within[r] * slot_stride +
    s * seg_stride, s < nseg)."""
    _fields_ = [
        ("base", ctypes.c_void_p),
        ("plane_bytes", ctypes.c_int64),
        ("page_stride", ctypes.c_int64),
        ("slot_stride", ctypes.c_int64),
        ("seg_stride", ctypes.c_int64),
        ("seg_bytes", ctypes.c_int32),
        ("nseg", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("num_slots", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqsa.so (built in-tree by `block_sparse_decode_amd.build`). Raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it first (python -m block_sparse_decode_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sp, pp = ctypes.POINTER(Shape), ctypes.POINTER(Paged)
        L.qsa_index_scores.argtypes = [sp, pp, P, P, P]
        L.qsa_select_topk.argtypes = [sp, pp, P, P, P]
        L.qsa_workspace_bytes.argtypes = [sp, I32]
        L.qsa_workspace_bytes.restype = SZ
        L.qsa_plan_decode.argtypes = [sp, I32, I32, ctypes.POINTER(DecodePlan)]
        L.qsa_sparse_decode.argtypes = [sp, pp, P, P, P, P, P, I32, P, SZ, P]
        L.qsa_select_sparse_decode.argtypes = [sp, pp, P, P, P, P, P, P, I32, P, SZ, P]
        L.qsa_select_sparse_decode_static.argtypes = [sp, pp, P, P, P, P, P, P, I32, P]
        L.qsa_kv_store.argtypes = [sp, pp, P, P, P]
        L.qsa_nvfp4_dequant_pages.argtypes = [sp, P, P, ctypes.c_float, P, I32, P, P]
        plp = ctypes.POINTER(Plane)
        L.qsa_rollback_stash_bytes.argtypes = [plp, I32, I32]
        L.qsa_rollback_stash_bytes.restype = SZ
        L.qsa_rollback_gather.argtypes = [plp, I32, P, P, I32, P, SZ, P, P]
        L.qsa_rollback_restore.argtypes = [plp, I32, P, P, P, I32, P, SZ, P, P]
        L.qsa_step_slots.argtypes = [sp, pp, P, P, P]
        L.qsa_status_string.argtypes = [ctypes.c_int]
        L.qsa_status_string.restype = ctypes.c_char_p
        L.qsa_abi_version.restype = I32
        for name in ("qsa_index_scores", "qsa_select_topk", "qsa_sparse_decode", "qsa_select_sparse_decode",
                     "qsa_kv_store", "qsa_nvfp4_dequant_pages", "qsa_rollback_gather", "qsa_rollback_restore",
                     "qsa_step_slots", "qsa_plan_decode", "qsa_select_sparse_decode_static"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != QSA_OK:
        raise QsaError(status, where)


def qsa_abi_version() -> int:
    return int(lib().qsa_abi_version())


def qsa_status_string(status: int) -> str:
    return lib().qsa_status_string(int(status)).decode()


def qsa_index_scores(shape: Shape, paged: Paged, q, scores, stream=None) -> None:
    _check(lib().qsa_index_scores(ctypes.byref(shape), ctypes.byref(paged), _ptr(q), _ptr(scores),
                                  _stream(stream)), "qsa_index_scores")


def qsa_select_topk(shape: Shape, paged: Paged, scores, selected, stream=None) -> None:
    _check(lib().qsa_select_topk(ctypes.byref(shape), ctypes.byref(paged), _ptr(scores), _ptr(selected),
                                 _stream(stream)), "qsa_select_topk")


def qsa_workspace_bytes(shape: Shape, num_splits: int = 0) -> int:
    return int(lib().qsa_workspace_bytes(ctypes.byref(shape), int(num_splits)))


def qsa_plan_decode(shape: Shape, num_splits: int = 0, fused: bool = True) -> DecodePlan:
    plan = DecodePlan()
    _check(lib().qsa_plan_decode(ctypes.byref(shape), int(num_splits), int(bool(fused)), ctypes.byref(plan)),
           "qsa_plan_decode")
    return plan


def qsa_sparse_decode(shape: Shape, paged: Paged, q, selected, out, lse=None, num_splits: int = 0,
                      workspace=None, workspace_bytes: Optional[int] = None, stream=None, gate=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qsa_sparse_decode(ctypes.byref(shape), ctypes.byref(paged), _ptr(q), _ptr(selected), _ptr(out),
                                   _ptr(lse), _ptr(gate), int(num_splits), _ptr(workspace), int(workspace_bytes),
                                   _stream(stream)), "qsa_sparse_decode")


def qsa_select_sparse_decode(shape: Shape, paged: Paged, q, scores, selected, out, lse=None, num_splits: int = 0,
                             workspace=None, workspace_bytes: Optional[int] = None, stream=None, gate=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qsa_select_sparse_decode(ctypes.byref(shape), ctypes.byref(paged), _ptr(q), _ptr(scores),
                                          _ptr(selected), _ptr(out), _ptr(lse), _ptr(gate), int(num_splits),
                                          _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "qsa_select_sparse_decode")


def qsa_select_sparse_decode_static(shape: Shape, paged: Paged, q, scores, selected, out, lse=None,
                                    num_splits: int = 0, stream=None, gate=None) -> None:
    _check(lib().qsa_select_sparse_decode_static(ctypes.byref(shape), ctypes.byref(paged), _ptr(q), _ptr(scores),
                                                 _ptr(selected), _ptr(out), _ptr(lse), _ptr(gate), int(num_splits),
                                                 _stream(stream)), "qsa_select_sparse_decode_static")


def qsa_kv_store(shape: Shape, paged: Paged, new_k, new_v, stream=None) -> None:
    _check(lib().qsa_kv_store(ctypes.byref(shape), ctypes.byref(paged), _ptr(new_k), _ptr(new_v), _stream(stream)),
           "qsa_kv_store")


def qsa_nvfp4_dequant_pages(shape: Shape, codes, scales, global_scale: float, pages, num_pages: int, out,
                            stream=None) -> None:
    _check(lib().qsa_nvfp4_dequant_pages(ctypes.byref(shape), _ptr(codes), _ptr(scales), float(global_scale),
                                         _ptr(pages), int(num_pages), _ptr(out), _stream(stream)),
           "qsa_nvfp4_dequant_pages")


def _planes(planes):
    arr = (Plane * len(planes))(*planes)
    return arr, len(planes)


def qsa_rollback_stash_bytes(planes, num_rows: int) -> int:
    arr, n = _planes(planes)
    return int(lib().qsa_rollback_stash_bytes(arr, n, int(num_rows)))


def qsa_step_slots(shape: Shape, paged: Paged, pages, within, stream=None) -> None:
    _check(lib().qsa_step_slots(ctypes.byref(shape), ctypes.byref(paged), _ptr(pages), _ptr(within),
                                _stream(stream)), "qsa_step_slots")


def qsa_rollback_gather(planes, pages, within, num_rows: int, stash, stash_bytes: Optional[int] = None,
                        error_word=None, stream=None) -> None:
    arr, n = _planes(planes)
    if stash_bytes is None:
        stash_bytes = stash.numel() * stash.element_size()
    _check(lib().qsa_rollback_gather(arr, n, _ptr(pages), _ptr(within), int(num_rows), _ptr(stash),
                                     int(stash_bytes), _ptr(error_word), _stream(stream)), "qsa_rollback_gather")


def qsa_rollback_restore(planes, pages, within, rejected, num_rows: int, stash, stash_bytes: Optional[int] = None,
                         error_word=None, stream=None) -> None:
    arr, n = _planes(planes)
    if stash_bytes is None:
        stash_bytes = stash.numel() * stash.element_size()
    _check(lib().qsa_rollback_restore(arr, n, _ptr(pages), _ptr(within), _ptr(rejected), int(num_rows), _ptr(stash),
                                      int(stash_bytes), _ptr(error_word), _stream(stream)), "qsa_rollback_restore")
