"""GPU parity of attention launches with more work items than two per CU, against the oracle on
every output.

Such a launch of one-row tiles runs 4-wave workgroups (three fit a CU) instead of 8-wave ones
(two fit), so that its items run in fewer rounds (TensorRT-LLM PR #20937, Description > What
changes > MTP > Verify: the last wave of a ragged verify batch is what the scheduling has to
fill). In that form each wave streams every fourth sub-chunk of its tile and finishes two of
the eight d/16 output tiles, so the wave merge, the split hand-off and the output write all
run their multi-tile forms. Each case asserts the wave count the launch takes
(qsa_plan_decode), then compares every (row, head) of `out` and `lse` with the oracle, for the
fused and the composed calls, one split and two.

Cases: decode rows of 8 q heads per KV head (640 and 516 tiles: just past the threshold),
verify rows of 16 q heads (one 16-column tile per row), d = 64, pages of 128, FP8 pools,
tables of up to 1024 pages, -1 page-table entries, copied index keys, and the gated epilogue.
Bars: attention |gpu - ref| <= 2e-3 + 1e-2 |ref| per element, lse within 2e-3, selection
rows bit for bit.
"""
import numpy as np
import pytest
import torch

import block_sparse_decode_amd as q
import oracle
import synth
from block_sparse_decode_amd.batch import DeviceBatch, Step

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 2e-3, 1e-2, 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    yield


def _check(out_t, lse_t, ref_out, ref_lse, where):
    out = synth.f32_from_bf16_bits(out_t.cpu().numpy().view(np.uint16)).astype(np.float64)
    err = np.abs(out - ref_out) - (ATOL + RTOL * np.abs(ref_out))
    assert err.max(initial=-1) <= 0, f"{where}: out beyond tolerance by {err.max()}"
    lse = lse_t.cpu().numpy()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)), where
    if fin.any():
        assert np.abs(lse[fin] - ref_lse[fin]).max() <= LSE_TOL, where


# (sizes kept small where the oracle's cost grows: rows x q heads x selected pages x P)
CASES = [
    synth.Config("wg_r1_g8", 130, 1, 32, 4, 128, 64, (200, 3000), 3, 1, seed=951, invalid_frac=0.1),
    synth.Config("wg_r1_b129", 129, 1, 8, 4, 128, 64, (64, 2000), 3, 1, seed=952, dup_key_frac=0.2),
    synth.Config("wg_r4_g16", 33, 4, 64, 4, 128, 64, (64, 1000), 2, 1, seed=953, invalid_frac=0.05),
    synth.Config("wg_r1_d64", 130, 1, 16, 4, 64, 64, (200, 3000), 4, 1, seed=954),
    synth.Config("wg_r1_p128", 130, 1, 8, 4, 128, 128, (300, 6000), 3, 1, seed=955, dup_key_frac=0.2),
    synth.Config("wg_r1_fp8", 130, 1, 16, 4, 128, 64, (100, 3000), 3, 1, seed=956, kv_format="fp8"),
    # page tables 512 and 1024 entries wide (8 and 16 score columns per lane in the fused
    # selection), over requests of up to 94 and 125 pages
    synth.Config("wg_r1_mp512", 130, 1, 8, 4, 128, 64, (2000, 6000), 8, 1, seed=957, invalid_frac=0.02,
                 max_pages=512),
    synth.Config("wg_r1_mp1024", 130, 1, 8, 4, 128, 64, (3000, 8000), 8, 1, seed=958, dup_key_frac=0.05,
                 max_pages=1024),
]

_cache = {}


def _case(cfg):
    """The workload, its scores and selection rows, and the oracle's attention, once per case."""
    if cfg.name not in _cache:
        w = synth.generate(cfg)
        s = oracle.index_scores(w)
        sel = oracle.select_w(w, s)
        _cache[cfg.name] = (w, s, sel, oracle.attention(w, sel))
    return _cache[cfg.name]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("splits", [0, 2])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_wide_grid_vs_oracle(cfg, splits, fused):
    w, ref_s, ref_sel, (ref_out, ref_lse) = _case(cfg)
    b = DeviceBatch.upload(w)
    plan = q.qsa_plan_decode(b.shape(), splits, fused)
    print(f"[wide grid] {cfg.name} tiles={b.shape().num_requests * cfg.kv_heads * plan.col_tiles} "
          f"splits={plan.splits} waves={plan.waves} fused={fused}", flush=True)
    assert plan.rows_per_tile == 1 and plan.waves == 4
    assert plan.splits == (splits if splits else 1)
    st = Step(b, num_splits=splits, fused=fused)
    st()
    torch.cuda.synchronize()
    assert np.array_equal(st.scores.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(st.selected.cpu().numpy(), ref_sel)
    _check(st.out, st.lse, ref_out, ref_lse, f"{cfg.name} splits={splits} fused={fused}")
    assert int(b.error_word[0].item()) == 0


def test_wide_grid_threshold():
    """512 one-row tiles (two per CU) keep 8-wave workgroups, 516 take 4-wave ones; both match
    the oracle."""
    cfg = CASES[1]
    w, _, _, _ = _case(cfg)
    nb = 128
    rows = int(w.row_offsets[nb])
    w128 = synth.Workload(w.cfg, w.page_table[:nb], w.seq_lens[:nb], w.row_offsets[:nb + 1], w.q[:rows],
                          w.k_codes, w.k_scales, w.v_codes, w.v_scales, w.index_keys)
    for ww, waves in ((w128, 8), (w, 4)):
        b = DeviceBatch.upload(ww)
        assert q.qsa_plan_decode(b.shape(), 0, True).waves == waves
        st = Step(b)
        st()
        torch.cuda.synchronize()
        sel = st.selected.cpu().numpy()
        assert np.array_equal(sel, oracle.select_w(ww, oracle.index_scores(ww)))
        ref_out, ref_lse = oracle.attention(ww, sel)
        _check(st.out, st.lse, ref_out, ref_lse, f"B={ww.B} waves={waves}")


_gated = {}


@pytest.mark.parametrize("splits", [0, 2])
def test_wide_grid_gated(splits):
    cfg = CASES[0]
    w, _, sel_ref, _ = _case(cfg)
    g = np.random.default_rng(17).standard_normal(w.q.shape).astype(np.float32) * 3.0
    gbits = synth.bf16_bits_from_f32(g)
    if not _gated:
        _gated["ref"] = oracle.attention(w, sel_ref, gate=gbits)
    ref_out, ref_lse = _gated["ref"]
    b = DeviceBatch.upload(w)
    assert q.qsa_plan_decode(b.shape(), splits, True).waves == 4
    st = Step(b, num_splits=splits, gate=torch.from_numpy(gbits.view(np.int16)).cuda())
    st()
    torch.cuda.synchronize()
    assert np.array_equal(st.selected.cpu().numpy(), sel_ref)
    _check(st.out, st.lse, ref_out, ref_lse, f"gated splits={splits}")


@pytest.mark.parametrize("splits", [0, 2])
@pytest.mark.parametrize("idx", [0, 6])
def test_wide_grid_fused_equals_composed_and_repeats(idx, splits):
    """With 4-wave workgroups the fused call (selection in the prologue, union placed by every
    thread) and the composed one (selection given, union built by one wave) list the same union
    entries, a selected page without a valid physical page included, so their waves stream the
    same sub-chunks in the same order: out and lse agree bit for bit. Repeated launches of each
    call give the same bits."""
    cfg = CASES[idx]
    w, ref_s, ref_sel, _ = _case(cfg)
    b = DeviceBatch.upload(w)
    assert q.qsa_plan_decode(b.shape(), splits, True).waves == 4
    ref = Step(b, num_splits=splits, fused=False)
    fus = Step(b, num_splits=splits, fused=True)
    for st in (ref, fus):
        st.scores.copy_(torch.from_numpy(ref_s).cuda())
    ref.select_call()
    ref.decode_call()
    fus.select_decode_call()
    torch.cuda.synchronize()
    assert np.array_equal(fus.selected.cpu().numpy(), ref_sel)
    assert torch.equal(fus.out, ref.out) and torch.equal(fus.lse, ref.lse)
    first_out, first_lse = fus.out.clone(), fus.lse.clone()
    for _ in range(5):
        fus.select_decode_call()
        ref.decode_call()
    torch.cuda.synchronize()
    assert torch.equal(fus.out, first_out) and torch.equal(fus.lse, first_lse)
    assert torch.equal(ref.out, first_out) and torch.equal(ref.lse, first_lse)


@pytest.mark.parametrize("fused", [True, False])
def test_wide_grid_short_long_and_bad_ids(fused):
    """4-wave launches (which load the request length before the score row and copy only the
    row's visible columns) on requests whose length is 0 (the row sees nothing), longer than the
    page table covers (rows clipped, flagged), and a page-table entry past the pool in a row's
    window (treated as -1, flagged): scores, selection rows and every output against the oracle."""
    import dataclasses
    cfg = CASES[0]
    w0, _, _, _ = _case(cfg)
    w = dataclasses.replace(w0)
    w.seq_lens = w0.seq_lens.copy()
    w.page_table = w0.page_table.copy()
    P = cfg.page_size
    w.seq_lens[3] = 0
    w.seq_lens[7] = w.MP * P + 5
    n9 = -(-int(w.seq_lens[9]) // P)
    w.page_table[9, n9 - 1] = w.NP + 3
    b = DeviceBatch.upload(w)
    assert q.qsa_plan_decode(b.shape(), 0, fused).waves == 4
    st = Step(b, fused=fused)
    st()
    torch.cuda.synchronize()
    ref_s = oracle.index_scores(w)
    assert np.array_equal(st.scores.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    sel = st.selected.cpu().numpy()
    assert np.array_equal(sel, oracle.select_w(w, ref_s))
    ref_out, ref_lse = oracle.attention(w, sel)
    _check(st.out, st.lse, ref_out, ref_lse, f"short/long/bad fused={fused}")
    err = int(b.error_word[0].item())
    assert err & q.QSA_DEVERR_PAGE_ID and err & q.QSA_DEVERR_SEQ_LEN
