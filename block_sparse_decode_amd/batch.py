"""Device-side batch: the paged NVFP4 cache and the query rows as torch tensors on a GPU.

torch only allocates device memory and supplies the stream. This module copies
host arrays (numpy, in the layouts of include/qsa.h) to the device and builds the
`Shape` / `Paged` argument blocks of the C ABI. It also sizes the outputs of
the three calls and runs one whole step.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import (Paged, Shape, qsa_index_scores, qsa_select_sparse_decode, qsa_select_topk, qsa_sparse_decode,
               qsa_workspace_bytes)


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


@dataclasses.dataclass
class DeviceBatch:
    page_table: torch.Tensor
    seq_lens: torch.Tensor
    row_offsets: torch.Tensor
    q: torch.Tensor                 # int16 view of bf16 bits
    k_codes: torch.Tensor
    k_scales: torch.Tensor
    v_codes: torch.Tensor
    v_scales: torch.Tensor
    index_keys: torch.Tensor        # int16 view of bf16 bits
    error_word: torch.Tensor        # int32 [1]
    num_requests: int
    num_rows: int
    max_rows: int
    q_heads: int
    kv_heads: int
    head_dim: int
    page_size: int
    max_pages: int
    num_phys_pages: int
    topk: int
    window: int
    sm_scale: float
    k_global: float = 1.0
    v_global: float = 1.0
    kv_format: int = 0              # QSA_KV_NVFP4 or QSA_KV_FP8

    @staticmethod
    def upload(w, device="cuda") -> "DeviceBatch":
        """`w`: a host workload (numpy arrays in the C-ABI layouts plus its config)."""
        c = w.cfg
        return DeviceBatch(
            page_table=_dev(w.page_table, device), seq_lens=_dev(w.seq_lens, device),
            row_offsets=_dev(w.row_offsets, device), q=_dev(w.q, device),
            k_codes=_dev(w.k_codes, device), k_scales=_dev(w.k_scales, device),
            v_codes=_dev(w.v_codes, device), v_scales=_dev(w.v_scales, device),
            index_keys=_dev(w.index_keys, device),
            error_word=torch.zeros(4, dtype=torch.int32, device=device),
            num_requests=int(w.B), num_rows=int(w.N), max_rows=max(1, int(w.max_rows)),
            q_heads=c.q_heads, kv_heads=c.kv_heads, head_dim=c.head_dim, page_size=c.page_size,
            max_pages=int(w.MP), num_phys_pages=int(w.NP), topk=c.topk, window=c.window,
            sm_scale=float(w.sm_scale), k_global=float(c.k_global), v_global=float(c.v_global),
            kv_format=1 if getattr(c, "kv_format", "nvfp4") == "fp8" else 0)

    @property
    def kw(self) -> int:
        return self.topk + self.window

    def shape(self) -> Shape:
        return Shape(self.num_requests, self.num_rows, self.max_rows, self.q_heads, self.kv_heads,
                     self.head_dim, self.page_size, self.max_pages, self.num_phys_pages, self.topk,
                     self.window, self.sm_scale, self.kv_format)

    def paged(self, error_word: bool = True) -> Paged:
        return Paged(self.page_table.data_ptr(), self.seq_lens.data_ptr(), self.row_offsets.data_ptr(),
                     self.k_codes.data_ptr(), self.k_scales.data_ptr(), self.v_codes.data_ptr(),
                     self.v_scales.data_ptr(), self.index_keys.data_ptr(), self.k_global, self.v_global,
                     self.error_word.data_ptr() if error_word else None)

    def rollback_planes(self):
        """The cache's planes as rollback planes: k_codes, k_scales, v_codes, v_scales (a row
        is one token slot across the KV heads) and index_keys (a row is one page)."""
        from . import Plane
        out = []
        for t in (self.k_codes, self.k_scales, self.v_codes, self.v_scales):
            NP, Hkv, P, nb = t.shape
            if nb == 0:
                continue                      # the FP8 cache has no scale planes
            out.append(Plane(t.data_ptr(), t.numel(), Hkv * P * nb, nb, P * nb, nb, Hkv, NP, P, 0))
        NP, Hkv, d = self.index_keys.shape
        out.append(Plane(self.index_keys.data_ptr(), self.index_keys.numel() * 2, Hkv * d * 2, 0, d * 2, d * 2, Hkv,
                         NP, self.page_size, 0))
        return out

    # output buffers ----------------------------------------------------------------
    def new_scores(self) -> torch.Tensor:
        return torch.empty((self.num_rows, self.max_pages), dtype=torch.float32, device=self.q.device)

    def new_selected(self) -> torch.Tensor:
        return torch.empty((self.num_rows, max(1, self.kw)), dtype=torch.int32, device=self.q.device)

    def new_out(self) -> torch.Tensor:
        return torch.empty((self.num_rows, self.q_heads, self.head_dim), dtype=torch.int16, device=self.q.device)

    def new_lse(self) -> torch.Tensor:
        return torch.empty((self.num_rows, self.q_heads), dtype=torch.float32, device=self.q.device)

    def new_workspace(self, num_splits: int = 0) -> Optional[torch.Tensor]:
        """Zero-filled, as qsa_sparse_decode requires of a workspace on its first use."""
        n = qsa_workspace_bytes(self.shape(), num_splits)
        return torch.zeros(max(n, 16), dtype=torch.uint8, device=self.q.device)


class Step:
    """One decode / verify step of one attention layer: scores -> selection -> attention.

    fused=True (the default) runs the selection inside the attention launch
    (qsa_select_sparse_decode); fused=False runs qsa_select_topk, then qsa_sparse_decode.
    Both give the same selection rows and outputs.

    The argument blocks and outputs are built once, so a call only launches kernels.
    """

    def __init__(self, batch: DeviceBatch, num_splits: int = 0, with_lse: bool = True, fused: bool = True,
                 gate=None):
        self.b = batch
        self.gate = gate
        self.fused = fused
        self.num_splits = num_splits
        self.shape_ = batch.shape()
        self.paged_ = batch.paged()
        self.scores = batch.new_scores()
        self.selected = batch.new_selected()
        self.out = batch.new_out()
        self.lse = batch.new_lse() if with_lse else None
        self.ws = batch.new_workspace(num_splits)

        # the raw argument lists of the two calls of a step, built once (pointers of the
        # tensors above); a step then costs two foreign calls
        import ctypes
        from . import QsaError, lib
        self._L = lib()
        self._QsaError = QsaError
        sh, pg = ctypes.byref(self.shape_), ctypes.byref(self.paged_)
        ws = self.ws
        self._a_scores = (sh, pg, self.b.q.data_ptr(), self.scores.data_ptr())
        self._a_fused = (sh, pg, self.b.q.data_ptr(), self.scores.data_ptr(), self.selected.data_ptr(),
                         self.out.data_ptr(), None if self.lse is None else self.lse.data_ptr(),
                         None if gate is None else gate.data_ptr(), int(num_splits), ws.data_ptr(), ws.numel())

    def _raw(self, fn, args, stream, name):
        import torch
        st = (torch.cuda.current_stream() if stream is None else stream).cuda_stream
        status = fn(*args, st)
        if status != 0:
            raise self._QsaError(status, name)

    def scores_call(self, stream=None):
        self._raw(self._L.qsa_index_scores, self._a_scores, stream, "qsa_index_scores")

    def select_call(self, stream=None):
        qsa_select_topk(self.shape_, self.paged_, self.scores, self.selected, stream)

    def decode_call(self, stream=None, selected=None):
        qsa_sparse_decode(self.shape_, self.paged_, self.b.q, self.selected if selected is None else selected,
                          self.out, self.lse, self.num_splits, self.ws, None, stream, gate=self.gate)

    def select_decode_call(self, stream=None):
        self._raw(self._L.qsa_select_sparse_decode, self._a_fused, stream, "qsa_select_sparse_decode")

    def __call__(self, stream=None):
        self.scores_call(stream)
        if self.fused:
            self.select_decode_call(stream)
        else:
            self.select_call(stream)
            self.decode_call(stream)
        return self.out
