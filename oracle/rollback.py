"""CPU oracle of the index-plane rollback: gather and restore of plane rows.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path never calls it.

Method: TensorRT-LLM PR #20937, Description > What changes > Rollback and PLE (the index
planes' writes of rejected rows undone in one batch) and its file list (a gather/restore operation
whose test restores the rejected rows and leaves the kept rows as the step wrote them).
The pages give the operation, not its addressing. The reading taken here:

  * a plane is a byte array; row r of it (for a verify row r of the step) is the bytes at
        pages[r] * page_stride + within[r] * slot_stride + s * seg_stride + [0, seg_bytes)
    for segments s = 0 .. nseg - 1 (slot_stride 0: one row per page);
  * gather copies every addressed row into the stash, plane by plane, before the step;
  * restore copies the stashed bytes back for each row with rejected[r] != 0;
  * a row with pages[r] == -1 is skipped; a page outside [-1, num_pages) or a slot outside
    [0, num_slots) is skipped and reported.

Plain numpy byte copies, one row and one segment at a time, in row order. Parity pinned
(tests/test_oracle_rollback.py) against numpy fancy indexing of the KV-cache layouts.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence

import numpy as np

ERR_PAGE_ID = 0x1
ERR_SLOT = 0x20


@dataclasses.dataclass
class Plane:
    buf: np.ndarray          # the plane's bytes (flat uint8, modified in place by restore)
    page_stride: int
    slot_stride: int
    seg_stride: int
    seg_bytes: int
    nseg: int
    num_pages: int
    num_slots: int

    @property
    def row_bytes(self) -> int:
        return self.nseg * self.seg_bytes


def _offsets(pl: Plane, page: int, slot: int):
    base = page * pl.page_stride + slot * pl.slot_stride
    return [base + s * pl.seg_stride for s in range(pl.nseg)]


def _valid(pl: Plane, page: int, slot: int):
    """(use the row, error bits) for one row of one plane."""
    if page == -1:
        return False, 0
    if page < -1 or page >= pl.num_pages:
        return False, ERR_PAGE_ID
    if slot < 0 or slot >= pl.num_slots:
        return False, ERR_SLOT
    return True, 0


def gather(planes: Sequence[Plane], pages, within, stash: List[np.ndarray]) -> int:
    """Copy row r of every plane into stash[k][r] (uint8 [nrows][row_bytes]); rows that are
    skipped leave their stash bytes as they were. Returns the error bits."""
    err = 0
    for k, pl in enumerate(planes):
        flat = pl.buf.reshape(-1)
        for r in range(len(pages)):
            ok, e = _valid(pl, int(pages[r]), int(within[r]))
            err |= e
            if not ok:
                continue
            for s, off in enumerate(_offsets(pl, int(pages[r]), int(within[r]))):
                stash[k][r, s * pl.seg_bytes:(s + 1) * pl.seg_bytes] = flat[off:off + pl.seg_bytes]
    return err


def restore(planes: Sequence[Plane], pages, within, rejected, stash: Sequence[np.ndarray]) -> int:
    """Copy stash[k][r] back into row r of every plane for each rejected row. Returns the
    error bits (of every row, rejected or not)."""
    err = 0
    for k, pl in enumerate(planes):
        flat = pl.buf.reshape(-1)
        for r in range(len(pages)):
            ok, e = _valid(pl, int(pages[r]), int(within[r]))
            err |= e
            if not ok or int(rejected[r]) == 0:
                continue
            for s, off in enumerate(_offsets(pl, int(pages[r]), int(within[r]))):
                flat[off:off + pl.seg_bytes] = stash[k][r, s * pl.seg_bytes:(s + 1) * pl.seg_bytes]
    return err


def kv_planes(k_codes, k_scales, v_codes, v_scales, index_keys) -> List[Plane]:
    """The five planes of the paged NVFP4 cache as rollback planes: the four per-slot planes
    [NP][Hkv][P][bytes] (a row is the slot's bytes for every KV head, one segment per head)
    and the per-page index keys [NP][Hkv][d] bf16 (one row per page: slot_stride 0, the slot
    only validated). Restoring a page's key for a rejected row returns it to its value before
    the step, which is the page's key again when every row the step put in that page is
    rejected."""
    out = []
    for a in (k_codes, k_scales, v_codes, v_scales):
        NP, Hkv, P, nb = a.shape
        out.append(Plane(a.view(np.uint8), Hkv * P * nb, nb, P * nb, nb, Hkv, NP, P))
    NP, Hkv, d = index_keys.shape
    P = k_codes.shape[2]
    out.append(Plane(index_keys.view(np.uint8), Hkv * d * 2, 0, d * 2, d * 2, Hkv, NP, P))
    return out
