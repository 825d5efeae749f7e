"""GPU parity of the index-plane rollback (qsa_step_slots, qsa_rollback_gather,
qsa_rollback_restore) against the oracle, bit for bit: the step rows' slots, the stash, and
every plane after a store and a restore of the rejected rows.
"""
import numpy as np
import pytest
import torch

import block_sparse_decode_amd as q
import synth
from block_sparse_decode_amd.batch import DeviceBatch
from oracle import rollback as rb

pytestmark = pytest.mark.gpu

PLANES = ("k_codes", "k_scales", "v_codes", "v_scales", "index_keys")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    yield


def _host_planes(b):
    arrs = []
    for name in PLANES:
        t = getattr(b, name).cpu().numpy()
        arrs.append(t.view(np.uint16) if name == "index_keys" else t)
    return arrs


def _slots_on_host(w):
    """Row j of request b sits at position L - R + j (the store's placement)."""
    P = w.cfg.page_size
    pages = np.full(w.N, -1, np.int32)
    within = np.zeros(w.N, np.int32)
    for b in range(w.B):
        r0, r1 = int(w.row_offsets[b]), int(w.row_offsets[b + 1])
        L = int(w.seq_lens[b])
        for j in range(r1 - r0):
            pos = L - (r1 - r0) + j
            if pos < 0 or pos // P >= w.MP:
                continue
            ph = int(w.page_table[b, pos // P])
            if 0 <= ph < w.NP:
                pages[r0 + j], within[r0 + j] = ph, pos % P
    return pages, within


def _stash_regions(stash, planes_np, nrows):
    out, off = [], 0
    for pl in planes_np:
        n = nrows * pl.row_bytes
        out.append(stash[off:off + n].reshape(nrows, pl.row_bytes))
        off += (n + 15) // 16 * 16
    return out


def _tokens(w, rng):
    x = rng.standard_normal((w.N, w.cfg.kv_heads, w.cfg.head_dim)).astype(np.float32)
    return torch.from_numpy(synth.bf16_bits_from_f32(x).view(np.int16)).cuda()


CASES = [
    synth.Config("rb_d128", 4, 4, 16, 2, 128, 64, (70, 3000), 6, 2, seed=601),
    synth.Config("rb_d64_p128", 3, 2, 8, 4, 64, 128, (130, 5000), 4, 1, seed=602, invalid_frac=0.1),
    synth.Config("rb_r1", 6, 1, 32, 4, 128, 64, (1, 900), 8, 2, seed=603),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_store_then_restore_rejected_rows(cfg):
    print(f"[rollback] {cfg.name}", flush=True)
    w = synth.generate(cfg)
    b = DeviceBatch.upload(w)
    n = w.N
    # the step's slots, on the device and on the host
    pages_d = torch.empty(n, dtype=torch.int32, device="cuda")
    within_d = torch.empty(n, dtype=torch.int32, device="cuda")
    q.qsa_step_slots(b.shape(), b.paged(), pages_d, within_d)
    pages, within = _slots_on_host(w)
    assert np.array_equal(pages_d.cpu().numpy(), pages)
    assert np.array_equal(within_d.cpu().numpy(), within)
    # gather
    planes = b.rollback_planes()
    sb = q.qsa_rollback_stash_bytes(planes, n)
    stash = torch.full((sb,), 0xA5, dtype=torch.uint8, device="cuda")
    q.qsa_rollback_gather(planes, pages_d, within_d, n, stash, error_word=b.error_word)
    before = _host_planes(b)
    planes_np = rb.kv_planes(*[a.copy() for a in before])
    st_ref = [np.full((n, pl.row_bytes), 0xA5, np.uint8) for pl in planes_np]
    assert rb.gather(planes_np, pages, within, st_ref) == 0
    torch.cuda.synchronize()
    for got, want in zip(_stash_regions(stash.cpu().numpy(), planes_np, n), st_ref):
        assert np.array_equal(got, want)
    # the step's store, then a restore of exactly half the rows (interleaved)
    rng = np.random.default_rng(cfg.seed)
    q.qsa_kv_store(b.shape(), b.paged(), _tokens(w, rng), _tokens(w, rng))
    torch.cuda.synchronize()
    after = _host_planes(b)
    rejected = (np.random.default_rng(n).permutation(n) < max(1, n // 2)).astype(np.int32)
    q.qsa_rollback_restore(planes, pages_d, within_d, torch.from_numpy(rejected).cuda(), n, stash,
                           error_word=b.error_word)
    torch.cuda.synchronize()
    planes_after = rb.kv_planes(*[a.copy() for a in after])
    assert rb.restore(planes_after, pages, within, rejected, st_ref) == 0
    for got, pl in zip(_host_planes(b), planes_after):
        assert np.array_equal(got.view(np.uint8).reshape(-1), pl.buf.reshape(-1))
    assert int(b.error_word[0].item()) == 0


def test_full_size_round_trip():
    """Gather, store and restore every row at the 32K verify workload: the cache is as before."""
    w = synth.generate("mtp_verify_32k")
    b = DeviceBatch.upload(w)
    n = w.N
    print("[rollback] mtp_verify_32k", flush=True)
    pages_d = torch.empty(n, dtype=torch.int32, device="cuda")
    within_d = torch.empty(n, dtype=torch.int32, device="cuda")
    q.qsa_step_slots(b.shape(), b.paged(), pages_d, within_d)
    planes = b.rollback_planes()
    stash = torch.zeros(q.qsa_rollback_stash_bytes(planes, n), dtype=torch.uint8, device="cuda")
    q.qsa_rollback_gather(planes, pages_d, within_d, n, stash)
    rng = np.random.default_rng(5)
    q.qsa_kv_store(b.shape(), b.paged(), _tokens(w, rng), _tokens(w, rng))
    q.qsa_rollback_restore(planes, pages_d, within_d, torch.ones(n, dtype=torch.int32, device="cuda"), n, stash)
    torch.cuda.synchronize()
    for name, got in zip(PLANES, _host_planes(b)):
        want = getattr(w, name)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), name
    assert int(b.error_word[0].item()) == 0


def test_skipped_and_reported_rows():
    cfg = synth.Config("rb_bad", 2, 2, 8, 2, 64, 64, (200, 400), 4, 1, seed=604)
    w = synth.generate(cfg)
    b = DeviceBatch.upload(w)
    pages = np.array([-1, w.NP, 1, 2], np.int32)            # skip, out of range, bad slot, good
    within = np.array([0, 0, 64, 5], np.int32)
    planes = b.rollback_planes()
    sb = q.qsa_rollback_stash_bytes(planes, 4)
    stash = torch.full((sb,), 0x5A, dtype=torch.uint8, device="cuda")
    pd, wd = torch.from_numpy(pages).cuda(), torch.from_numpy(within).cuda()
    q.qsa_rollback_gather(planes, pd, wd, 4, stash, error_word=b.error_word)
    torch.cuda.synchronize()
    assert int(b.error_word[0].item()) == q.QSA_DEVERR_PAGE_ID | q.QSA_DEVERR_SLOT
    planes_np = rb.kv_planes(*_host_planes(b))
    st_ref = [np.full((4, pl.row_bytes), 0x5A, np.uint8) for pl in planes_np]
    rb.gather(planes_np, pages, within, st_ref)
    for got, want in zip(_stash_regions(stash.cpu().numpy(), planes_np, 4), st_ref):
        assert np.array_equal(got, want)
