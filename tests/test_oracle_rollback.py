"""Pins of the rollback oracle (gather / restore of plane rows for rejected draft rows):
its byte arithmetic against numpy fancy indexing of the cache layouts, the restore
invariants (rejected rows back to their pre-step bytes, kept rows and every other byte as
the step left them), the round trip, skipped and reported rows, and duplicate rows.
"""
import numpy as np
import pytest

from oracle import rollback as rb


def _cache(rng, NP=6, Hkv=3, P=64, d=64):
    k_codes = rng.integers(0, 256, (NP, Hkv, P, d // 2), dtype=np.uint8)
    k_scales = rng.integers(0, 127, (NP, Hkv, P, d // 16), dtype=np.uint8)
    v_codes = rng.integers(0, 256, (NP, Hkv, P, d // 2), dtype=np.uint8)
    v_scales = rng.integers(0, 127, (NP, Hkv, P, d // 16), dtype=np.uint8)
    keys = rng.integers(0, 1 << 16, (NP, Hkv, d), dtype=np.uint16)
    return [k_codes, k_scales, v_codes, v_scales, keys]


def _rows_by_indexing(arrs, pages, within):
    """The addressed rows by plain array indexing (an independent formulation)."""
    out = []
    for a in arrs[:4]:
        out.append(np.stack([a[p, :, w, :].reshape(-1) for p, w in zip(pages, within)]))
    out.append(np.stack([arrs[4][p].view(np.uint8).reshape(-1) for p in pages]))
    return out


def _stash(planes, n, fill=0xA5):
    return [np.full((n, pl.row_bytes), fill, np.uint8) for pl in planes]


def test_gather_equals_array_indexing():
    rng = np.random.default_rng(1)
    arrs = _cache(rng)
    pages = np.array([3, 0, 5, 3, 1], np.int32)
    within = np.array([63, 0, 17, 62, 40], np.int32)
    planes = rb.kv_planes(*arrs)
    st = _stash(planes, len(pages))
    assert rb.gather(planes, pages, within, st) == 0
    for got, want in zip(st, _rows_by_indexing(arrs, pages, within)):
        assert np.array_equal(got, want)


@pytest.mark.parametrize("rows", [4, 512])
def test_restore_rejected_rows_only(rows):
    rng = np.random.default_rng(rows)
    arrs = _cache(rng, NP=8 if rows == 4 else 64, P=64)
    NP, P = arrs[0].shape[0], arrs[0].shape[2]
    # distinct (page, slot) per row, as the rows of a step occupy distinct slots
    flat = rng.choice(NP * P, size=rows, replace=False)
    pages, within = (flat // P).astype(np.int32), (flat % P).astype(np.int32)
    before = [a.copy() for a in arrs]
    planes = rb.kv_planes(*arrs)
    st = _stash(planes, rows)
    rb.gather(planes, pages, within, st)
    # the step writes new bytes into every addressed row
    for a in arrs[:4]:
        a[pages, :, within, :] = rng.integers(0, 256, a[pages, :, within, :].shape, dtype=np.uint8)
    after = [a.copy() for a in arrs]
    # exactly half the rows rejected, interleaved
    rejected = (np.random.default_rng(rows).permutation(rows) < rows // 2).astype(np.int32)
    assert 0 < rejected.sum() < rows
    assert rb.restore(planes, pages, within, rejected, st) == 0
    for a, b0, a1 in zip(arrs[:4], before[:4], after[:4]):
        want = a1.copy()
        rj = rejected.astype(bool)
        want[pages[rj], :, within[rj], :] = b0[pages[rj], :, within[rj], :]
        assert np.array_equal(a, want)
    # the keys plane was not written by the step, so restoring it is a no-op on its bytes
    assert np.array_equal(arrs[4], before[4])


def test_round_trip_restores_everything():
    rng = np.random.default_rng(3)
    arrs = _cache(rng)
    before = [a.copy() for a in arrs]
    pages = np.array([2, 2, 4, 0], np.int32)          # two rows in one page: same key row
    within = np.array([10, 11, 0, 63], np.int32)
    planes = rb.kv_planes(*arrs)
    st = _stash(planes, 4)
    rb.gather(planes, pages, within, st)
    for a in arrs:
        a.view(np.uint8)[...] = rng.integers(0, 256, a.view(np.uint8).shape, dtype=np.uint8)
    rb.restore(planes, pages, within, np.ones(4, np.int32), st)
    for a, b in zip(arrs[:4], before[:4]):
        assert np.array_equal(a[pages, :, within, :], b[pages, :, within, :])
    assert np.array_equal(arrs[4][pages], before[4][pages])


def test_skipped_and_reported_rows():
    rng = np.random.default_rng(4)
    arrs = _cache(rng, NP=4)
    before = [a.copy() for a in arrs]
    planes = rb.kv_planes(*arrs)
    pages = np.array([-1, 4, 1, 2], np.int32)          # skip, out of range, bad slot, good
    within = np.array([0, 0, 64, 5], np.int32)
    st = _stash(planes, 4, fill=0x5A)
    err = rb.gather(planes, pages, within, st)
    assert err == rb.ERR_PAGE_ID | rb.ERR_SLOT
    for s in st:
        assert np.all(s[:3] == 0x5A)                    # skipped rows leave the stash alone
    want = _rows_by_indexing(arrs, pages[3:], within[3:])
    for s, w in zip(st, want):
        assert np.array_equal(s[3:], w)
    for s in st:
        s[...] = 0
    err = rb.restore(planes, pages, within, np.ones(4, np.int32), st)
    assert err == rb.ERR_PAGE_ID | rb.ERR_SLOT
    for a, b in zip(arrs[:4], before[:4]):
        a2 = a.copy()
        a2[2, :, 5, :] = b[2, :, 5, :]                  # only the good row was rewritten (to 0)
        assert np.array_equal(a2, b)
        assert not a[2, :, 5, :].any()
