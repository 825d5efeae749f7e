"""C-ABI checks that need no GPU: the library loads, exports every function that
include/qsa.h declares, and its struct layouts match the ctypes mirrors. Host-side
argument validation rejects bad calls before any launch (these calls never reach HIP).
"""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_decode_amd as q
from block_sparse_decode_amd import Paged, Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = q.lib()
    declared = _declared_functions()
    assert declared == sorted(q.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True, check=True)
    syms = set(l.split()[-1] for l in out.stdout.splitlines() if l.strip())
    for name in declared:
        assert name in syms, name
        assert hasattr(L, name)


def test_abi_version_and_status_strings():
    assert q.qsa_abi_version() == 2
    for st, text in [(0, "ok"), (1, "invalid argument"), (2, "unsupported configuration"),
                     (3, "workspace too small"), (4, "HIP launch error"), (99, "unknown status")]:
        assert q.qsa_status_string(st) == text


def test_struct_layout_matches_header(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "qsa.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu\n", sizeof(qsa_shape), offsetof(qsa_shape, num_phys_pages),
         offsetof(qsa_shape, topk), offsetof(qsa_shape, sm_scale), sizeof(qsa_paged));
  printf("%zu %zu %zu %zu\n", offsetof(qsa_paged, index_keys), offsetof(qsa_paged, k_global),
         offsetof(qsa_paged, v_global), offsetof(qsa_paged, error_word));
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)], check=True)
    a, b = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")[:2]
    want_a = [ctypes.sizeof(Shape), Shape.num_phys_pages.offset, Shape.topk.offset, Shape.sm_scale.offset,
              ctypes.sizeof(Paged)]
    want_b = [Paged.index_keys.offset, Paged.k_global.offset, Paged.v_global.offset, Paged.error_word.offset]
    assert list(map(int, a.split())) == want_a
    assert list(map(int, b.split())) == want_b


def _shape(**kw):
    base = dict(num_requests=2, num_rows=8, max_rows_per_request=4, num_q_heads=32, num_kv_heads=4,
                head_dim=128, page_size=64, max_pages=512, num_phys_pages=1024, topk=32, window=2,
                sm_scale=0.088388)
    base.update(kw)
    return Shape(**base)


FAKE = 0x1000     # a 16-byte aligned, never dereferenced address: every call below fails validation first


def _paged(**kw):
    base = dict(page_table=FAKE, seq_lens=FAKE, row_offsets=FAKE, k_codes=FAKE, k_scales=FAKE, v_codes=FAKE,
                v_scales=FAKE, index_keys=FAKE, k_global=1.0, v_global=1.0, error_word=None)
    base.update(kw)
    return Paged(**base)


def _raw(name, *args):
    return getattr(q.lib(), name)(*args)


def _rawd(name, *args):
    """The attention calls without a gate: None goes in the gate position (after lse)."""
    args = list(args)
    args.insert(6 if name == "qsa_sparse_decode" else 7, None)
    return _raw(name, *args)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 2), (dict(head_dim=256), 2), (dict(page_size=32), 2), (dict(max_pages=4097), 2),
    (dict(topk=250, window=7), 2), (dict(max_rows_per_request=1025), 2),
    (dict(num_q_heads=30), 1), (dict(num_kv_heads=0), 1), (dict(num_requests=-1), 1), (dict(topk=-1), 1),
    (dict(max_pages=0), 1), (dict(num_rows=9), 1), (dict(sm_scale=float("inf")), 1),
])
def test_shape_validation(kw, status):
    sh = _shape(**kw)
    pg = _paged()
    assert _raw("qsa_index_scores", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE, None) == status
    assert _raw("qsa_select_topk", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE, None) == status
    assert _rawd("qsa_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE, FAKE, None, 0, FAKE,
                1 << 30, None) == status
    assert q.qsa_workspace_bytes(sh, 0) == 0


def test_pointer_validation():
    sh, pg = _shape(), _paged()
    # NULL shape / paged / required tensors
    assert _raw("qsa_index_scores", None, ctypes.byref(pg), FAKE, FAKE, None) == 1
    assert _raw("qsa_index_scores", ctypes.byref(sh), None, FAKE, FAKE, None) == 1
    assert _raw("qsa_index_scores", ctypes.byref(sh), ctypes.byref(pg), None, FAKE, None) == 1
    assert _raw("qsa_select_topk", ctypes.byref(sh), ctypes.byref(pg), FAKE, None, None) == 1
    assert _rawd("qsa_sparse_decode", ctypes.byref(sh), ctypes.byref(_paged(v_codes=None)), FAKE, FAKE, FAKE,
                None, 0, FAKE, 1 << 30, None) == 1
    # misaligned tensors
    assert _raw("qsa_index_scores", ctypes.byref(sh), ctypes.byref(pg), FAKE + 2, FAKE, None) == 1
    assert _rawd("qsa_sparse_decode", ctypes.byref(sh), ctypes.byref(_paged(k_codes=FAKE + 8)), FAKE, FAKE, FAKE,
                None, 0, FAKE, 1 << 30, None) == 1
    # negative split count, non-finite global scale
    assert _rawd("qsa_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE, FAKE, None, -1, FAKE,
                1 << 30, None) == 1
    assert _rawd("qsa_sparse_decode", ctypes.byref(sh), ctypes.byref(_paged(k_global=float("nan"))), FAKE, FAKE,
                FAKE, None, 0, FAKE, 1 << 30, None) == 1
    # the logit scale sm_scale * k_global must be positive
    for bad_sh, bad_pg in ((_shape(sm_scale=0.0), pg), (_shape(sm_scale=-0.1), pg), (sh, _paged(k_global=-1.0)),
                           (sh, _paged(k_global=0.0))):
        assert _rawd("qsa_sparse_decode", ctypes.byref(bad_sh), ctypes.byref(bad_pg), FAKE, FAKE, FAKE, None, 0,
                    FAKE, 1 << 30, None) == 1
        assert _rawd("qsa_select_sparse_decode", ctypes.byref(bad_sh), ctypes.byref(bad_pg), FAKE, FAKE, FAKE,
                    FAKE, None, 0, FAKE, 1 << 30, None) == 1
    # the KV store takes at most 4 rows per request (a context step's rows are stored elsewhere)
    assert _raw("qsa_kv_store", ctypes.byref(_shape(max_rows_per_request=16, num_rows=16)), ctypes.byref(pg), FAKE,
                FAKE, None) == 2


def test_kv_format_and_gate_validation():
    pg = _paged()
    # an unknown format is refused by every call that takes a shape
    bad = _shape(kv_format=2)
    assert _raw("qsa_index_scores", ctypes.byref(bad), ctypes.byref(pg), FAKE, FAKE, None) == 1
    assert _rawd("qsa_sparse_decode", ctypes.byref(bad), ctypes.byref(pg), FAKE, FAKE, FAKE, None, 0, FAKE,
                 1 << 30, None) == 1
    # FP8 pools: the scale planes are not needed; the store does not take FP8 pools
    fp8 = _shape(kv_format=1)
    no_scales = _paged(k_scales=None, v_scales=None)
    assert _raw("qsa_kv_store", ctypes.byref(fp8), ctypes.byref(pg), FAKE, FAKE, None) == 2
    assert _rawd("qsa_sparse_decode", ctypes.byref(_shape()), ctypes.byref(no_scales), FAKE, FAKE, FAKE, None, 0,
                 FAKE, 1 << 30, None) == 1                       # NVFP4 needs them
    assert _rawd("qsa_sparse_decode", ctypes.byref(fp8), ctypes.byref(no_scales), FAKE, FAKE, FAKE, None, -1,
                 FAKE, 1 << 30, None) == 1                       # (refused later, on the split count)
    # a gate must be 16-byte aligned
    sh = _shape()
    assert _raw("qsa_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE, FAKE, None, FAKE + 2, 0, FAKE,
                1 << 30, None) == 1
    assert _raw("qsa_select_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE, FAKE, FAKE, None,
                FAKE + 8, 0, FAKE, 1 << 30, None) == 1


def test_fused_select_decode_validation():
    sh, pg = _shape(), _paged()
    # the selection needs the scores and somewhere to write the rows
    assert _rawd("qsa_select_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), FAKE, None, FAKE, FAKE, None, 0,
                FAKE, 1 << 30, None) == 1
    assert _rawd("qsa_select_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE, None, FAKE, None, 0,
                FAKE, 1 << 30, None) == 1
    assert _rawd("qsa_select_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE + 4, FAKE, FAKE, None,
                0, FAKE, 1 << 30, None) == 1
    # the checks of qsa_sparse_decode apply
    assert _rawd("qsa_select_sparse_decode", ctypes.byref(_shape(head_dim=96)), ctypes.byref(pg), FAKE, FAKE, FAKE,
                FAKE, None, 0, FAKE, 1 << 30, None) == 2
    assert _rawd("qsa_select_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE, FAKE, FAKE, None, 4,
                FAKE, q.qsa_workspace_bytes(sh, 4) - 1, None) == 3


def test_kv_store_validation():
    sh, pg = _shape(), _paged()
    args = lambda s, p, k=FAKE, v=FAKE: (ctypes.byref(s), ctypes.byref(p), k, v, None)
    # the new tokens and every plane the store writes are required, 16-byte aligned
    assert _raw("qsa_kv_store", *args(sh, pg, k=None)) == 1
    assert _raw("qsa_kv_store", *args(sh, pg, v=None)) == 1
    assert _raw("qsa_kv_store", *args(sh, pg, k=FAKE + 2)) == 1
    for plane in ("page_table", "k_codes", "k_scales", "v_codes", "v_scales", "index_keys"):
        assert _raw("qsa_kv_store", *args(sh, _paged(**{plane: None}))) == 1, plane
        assert _raw("qsa_kv_store", *args(sh, _paged(**{plane: FAKE + 8}))) == 1, plane
    # global scales: positive and finite
    for g in (0.0, -1.0, float("nan"), float("inf")):
        assert _raw("qsa_kv_store", *args(sh, _paged(k_global=g))) == 1
        assert _raw("qsa_kv_store", *args(sh, _paged(v_global=g))) == 1
    # the shape checks apply
    assert _raw("qsa_kv_store", *args(_shape(head_dim=96), pg)) == 2
    assert _raw("qsa_kv_store", *args(_shape(max_rows_per_request=5), pg)) == 2
    assert _raw("qsa_kv_store", *args(_shape(num_rows=9), pg)) == 1
    assert _raw("qsa_kv_store", None, ctypes.byref(pg), FAKE, FAKE, None) == 1
    assert _raw("qsa_kv_store", ctypes.byref(sh), None, FAKE, FAKE, None) == 1
    # an empty batch is a no-op, whatever the pointers
    assert _raw("qsa_kv_store", ctypes.byref(_shape(num_requests=0, num_rows=0)), ctypes.byref(pg), None, None,
                None) == 0


def test_plane_struct_layout(tmp_path):
    prog = tmp_path / "plane.c"
    prog.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "qsa.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(qsa_plane), offsetof(qsa_plane, plane_bytes),
         offsetof(qsa_plane, seg_bytes), offsetof(qsa_plane, nseg), offsetof(qsa_plane, num_pages),
         offsetof(qsa_plane, num_slots));
  return 0;
}
''')
    exe = tmp_path / "plane"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)], check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()))
    P = q.Plane
    assert got == [ctypes.sizeof(P), P.plane_bytes.offset, P.seg_bytes.offset, P.nseg.offset, P.num_pages.offset,
                   P.num_slots.offset]


def _plane(**kw):
    base = dict(base=FAKE, plane_bytes=4 * 3 * 64 * 64, page_stride=3 * 64 * 64, slot_stride=64, seg_stride=64 * 64,
                seg_bytes=64, nseg=3, num_pages=4, num_slots=64, reserved=0)
    base.update(kw)
    return q.Plane(**base)


def test_rollback_stash_bytes():
    # plane k's rows at a 16-byte aligned offset after the earlier planes' rows
    a, b = _plane(), _plane(seg_bytes=4, slot_stride=4, seg_stride=4 * 64, page_stride=3 * 64 * 4,
                            plane_bytes=4 * 3 * 64 * 4)
    assert q.qsa_rollback_stash_bytes([a], 5) == 5 * 192
    assert q.qsa_rollback_stash_bytes([b, a], 5) == 64 + 5 * 192          # 5 * 12 = 60 -> 64
    assert q.qsa_rollback_stash_bytes([a, b], 0) == 0
    # invalid descriptors give 0
    for bad in (dict(base=None), dict(base=FAKE + 2), dict(seg_bytes=6), dict(seg_bytes=0), dict(nseg=0),
                dict(num_slots=0), dict(page_stride=-64), dict(slot_stride=66), dict(plane_bytes=4 * 3 * 64 * 64 - 1),
                dict(num_pages=-1)):
        assert q.qsa_rollback_stash_bytes([_plane(**bad)], 5) == 0, bad
    assert q.qsa_rollback_stash_bytes([a] * 17, 5) == 0
    assert q.qsa_rollback_stash_bytes([a], -1) == 0
    assert q.qsa_rollback_stash_bytes([], 5) == 0


def test_rollback_validation():
    arr = (q.Plane * 2)(_plane(), _plane())
    g = lambda planes, n, pages, within, rows, stash, sb: _raw("qsa_rollback_gather", planes, n, pages, within, rows,
                                                               stash, sb, None, None)
    r = lambda planes, n, pages, within, rej, rows, stash, sb: _raw("qsa_rollback_restore", planes, n, pages, within,
                                                                    rej, rows, stash, sb, None, None)
    need = q.qsa_rollback_stash_bytes(list(arr), 8)
    assert g(arr, 2, None, None, 0, None, 0) == 0                       # no rows: no-op
    assert g(arr, 2, None, FAKE, 8, FAKE, need) == 1
    assert g(arr, 2, FAKE, FAKE + 2, 8, FAKE, need) == 1
    assert g(arr, 2, FAKE, FAKE, 8, None, need) == 1
    assert g(arr, 2, FAKE, FAKE, 8, FAKE + 8, need) == 1                # stash 16-byte aligned
    assert g(arr, 2, FAKE, FAKE, 8, FAKE, need - 1) == 3
    assert g(arr, 0, FAKE, FAKE, 8, FAKE, need) == 1
    assert g(None, 2, FAKE, FAKE, 8, FAKE, need) == 1
    bad = (q.Plane * 1)(_plane(seg_bytes=6))
    assert g(bad, 1, FAKE, FAKE, 8, FAKE, need) == 1
    assert r(arr, 2, FAKE, FAKE, None, 8, FAKE, need) == 1              # rejected flags required
    assert r(arr, 2, FAKE, FAKE, FAKE, 8, FAKE, need - 1) == 3
    assert r(arr, 2, None, None, None, 0, None, 0) == 0
    assert _raw("qsa_rollback_gather", arr, 2, FAKE, FAKE, 8, FAKE, need, FAKE + 2, None) == 1   # error word
    # step slots: the shape checks apply; outputs required
    sh, pg = _shape(), _paged()
    assert _raw("qsa_step_slots", ctypes.byref(_shape(head_dim=96)), ctypes.byref(pg), FAKE, FAKE, None) == 2
    assert _raw("qsa_step_slots", ctypes.byref(sh), ctypes.byref(pg), None, FAKE, None) == 1
    assert _raw("qsa_step_slots", ctypes.byref(sh), ctypes.byref(_paged(page_table=None)), FAKE, FAKE, None) == 1
    assert _raw("qsa_step_slots", ctypes.byref(_shape(num_requests=0, num_rows=0)), ctypes.byref(pg), None, None,
                None) == 0


def test_workspace_sizing():
    sh = _shape()
    assert q.qsa_workspace_bytes(sh, 1) == 0
    # 2 requests x 4 KV heads x 4 tiles: 4 rows x 8 q heads per KV head, one row per tile
    # (grouping rows would leave fewer tiles than CUs); a fixed 32 KiB counter region, then
    # per (tile, split) 9 accumulator tiles (8 of d 128 + the denominator) of 64 lanes x 4
    # floats, plus 64 column maxima
    tiles = 2 * 4 * 4
    part = tiles * 4 * (9 * 64 * 4 + 64) * 4
    assert q.qsa_workspace_bytes(sh, 4) == 32768 + part
    assert q.qsa_workspace_bytes(sh, 1000) == q.qsa_workspace_bytes(sh, 64)
    # the counter region does not grow with the batch: only the partials do
    big = _shape(num_requests=200, num_rows=800)
    tiles_big = 200 * 4 * 2                     # enough tiles for two rows per tile
    assert q.qsa_workspace_bytes(big, 2) == 32768 + tiles_big * 2 * (9 * 64 * 4 + 64) * 4
    # past 8192 tiles a split is not possible (no counter for it): one split, no workspace
    huge = _shape(num_requests=1100, num_rows=4400)
    assert 1100 * 4 * 2 > 8192 and q.qsa_workspace_bytes(huge, 4) == 0
    # a too-small workspace is refused before any launch
    pg = _paged()
    assert _rawd("qsa_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE, FAKE, None, 4, FAKE,
                q.qsa_workspace_bytes(sh, 4) - 1, None) == 3
    assert _rawd("qsa_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), FAKE, FAKE, FAKE, None, 4, None,
                1 << 30, None) == 3


def test_plan_struct_layout(tmp_path):
    prog = tmp_path / "plan.c"
    prog.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "qsa.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(qsa_decode_plan), offsetof(qsa_decode_plan, select_cols),
         offsetof(qsa_decode_plan, workgroups), offsetof(qsa_decode_plan, workspace_bytes));
  return 0;
}
''')
    exe = tmp_path / "plan"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)], check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()))
    D = q.DecodePlan
    assert got == [ctypes.sizeof(D), D.select_cols.offset, D.workgroups.offset, D.workspace_bytes.offset]


@pytest.mark.parametrize("B,R,Hq,Hkv,MP,rows,cols,ctiles,waves", [
    (16, 4, 32, 4, 512, 1, 8, 4, 8),      # the 32K verify workload: 256 one-row tiles
    (32, 4, 32, 4, 64, 2, 16, 2, 8),      # 2 rows x 8 q heads: 256 tiles
    (64, 4, 16, 4, 64, 4, 16, 1, 8),      # 4 rows x 4 q heads: 256 tiles
    (64, 3, 20, 4, 64, 3, 15, 1, 8),      # 3 rows x 5 q heads
    (8, 4, 16, 4, 64, 1, 4, 4, 8),        # few tiles: rows halved down to one
    (8, 2, 48, 2, 64, 0, 16, 3, 8),       # 24 q heads per KV head: tiles cut rows
    # verify rows over 1024-page tables share few pages: 768 one-row tiles beat 384 two-row
    # ones (2 rounds of tiles with twice the union); 768 one-row tiles take 4-wave workgroups
    (48, 4, 32, 4, 1024, 1, 8, 4, 4),
    (16, 2, 64, 4, 256, 1, 16, 2, 8),     # 16-column tiles of 16-head rows: one row each, 128
    (64, 4, 64, 4, 256, 1, 16, 4, 4),     # the same over 1024 tiles
    # a context step's neighbouring rows over 128 pages share most of theirs: two rows per tile
    (4, 256, 32, 4, 128, 2, 16, 128, 8),
])
def test_plan_tile_heights(B, R, Hq, Hkv, MP, rows, cols, ctiles, waves):
    sh = _shape(num_requests=B, num_rows=B * R, max_rows_per_request=R, num_q_heads=Hq, num_kv_heads=Hkv,
                max_pages=MP)
    p = q.qsa_plan_decode(sh, 0, True)
    assert (p.rows_per_tile, p.tile_cols, p.col_tiles) == (rows, cols, ctiles)
    assert p.waves == waves
    # forced splits count too: more than two work items per CU take 4-wave one-row workgroups
    p3 = q.qsa_plan_decode(sh, 3, True)
    one_row = rows == 1 or (rows == 0 and Hq // Hkv % 16 == 0)
    assert p3.waves == (4 if one_row and B * Hkv * ctiles * 3 > 512 else 8)
    assert p.workspace_bytes == q.qsa_workspace_bytes(sh, 0)
    assert p.workgroups % 8 == 0 and p.workgroups >= B * Hkv * ctiles * p.splits
    assert p.select_cols == (2 if MP <= 128 else 4 if MP <= 256 else 8 if MP <= 512 else 16)
    assert q.qsa_plan_decode(sh, 0, False).select_cols == 0
    assert q.qsa_plan_decode(sh, 3, True).splits == 3


def test_plan_select_cols_and_validation():
    for MP, c in ((16, 2), (128, 2), (129, 4), (256, 4), (512, 8), (1024, 16), (1025, 0), (4096, 0)):
        assert q.qsa_plan_decode(_shape(max_pages=MP), 0, True).select_cols == c, MP
    assert q.qsa_plan_decode(_shape(topk=0, window=0), 0, True).select_cols == 0
    plan = q.DecodePlan()
    assert _raw("qsa_plan_decode", ctypes.byref(_shape()), 0, 1, None) == 1
    assert _raw("qsa_plan_decode", ctypes.byref(_shape()), -1, 1, ctypes.byref(plan)) == 1
    assert _raw("qsa_plan_decode", ctypes.byref(_shape(head_dim=96)), 0, 1, ctypes.byref(plan)) == 2
    assert _raw("qsa_plan_decode", None, 0, 1, ctypes.byref(plan)) == 1


def test_empty_batches_are_no_ops():
    sh = _shape(num_requests=0, num_rows=0)
    pg = _paged()
    assert _raw("qsa_index_scores", ctypes.byref(sh), ctypes.byref(pg), None, None, None) == 0
    assert _raw("qsa_select_topk", ctypes.byref(sh), ctypes.byref(pg), None, None, None) == 0
    assert _rawd("qsa_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), None, None, None, None, 0, None, 0,
                None) == 0
    assert _rawd("qsa_select_sparse_decode", ctypes.byref(sh), ctypes.byref(pg), None, None, None, None, None, 0,
                None, 0, None) == 0
    dq = _shape()
    assert _raw("qsa_nvfp4_dequant_pages", ctypes.byref(dq), None, None, ctypes.c_float(1.0), None, 0, None,
                None) == 0
