"""GPU parity of attention tiles that hold several rows, against the oracle on every output.

A tile is a run of at most 16 of a request's query columns (rows x the q heads of one KV
head); the pages any of its rows selected are read once for the whole tile (TensorRT-LLM
PR #20276, Performance > What runs on the fast paths: rows of a request share their K/V
page reads). The launch groups rows only when the batch still gives at least one tile per CU,
so these shapes are large batches of short requests: 2, 3 and 4 rows per tile, and tiles
that cut rows (24 q heads per KV head). Each case asserts the tile height the launch takes
(qsa_plan_decode), then compares every (row, head) of `out` and `lse` with the oracle, for
the fused and the composed calls at 1, 2 and 3 splits.

Cases the row grouping has to get right:
  * rows of a request that select disjoint pages (scores injected), so each page of the
    union is visible to one row of the tile only;
  * requests whose length ends one to three tokens into a page, so the tile's rows end in
    different pages and the last page is visible to some rows of the tile and not others;
  * -1 page-table entries inside the union.
Bars: attention |gpu - ref| <= 2e-3 + 1e-2 |ref| per element, lse within 2e-3, selection
rows bit for bit.
"""
import dataclasses

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


def _check(out_bits, lse, ref_out, ref_lse, where):
    out = synth.f32_from_bf16_bits(out_bits).astype(np.float64)
    err = np.abs(out - ref_out) - (ATOL + RTOL * np.abs(ref_out))
    assert err.max(initial=-1) <= 0, f"{where}: out beyond tolerance by {err.max()}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)), where
    if fin.any():
        assert np.abs(lse[fin] - ref_lse[fin]).max() <= LSE_TOL, where


def _ragged_ends(w, every=3):
    """Every `every`-th request ends 1..3 tokens into its last page (the rest keep their length),
    so that the causal rows of one request end in different pages."""
    w = dataclasses.replace(w)
    seq = w.seq_lens.copy()
    P = w.cfg.page_size
    for b in range(0, w.B, every):
        t = 1 + (b // every) % 3
        new = (int(seq[b]) // P) * P + t
        R = int(w.row_offsets[b + 1] - w.row_offsets[b])
        if R <= new <= int(seq[b]):
            seq[b] = new
    w.seq_lens = seq
    return w


# (config, rows per tile the launch must take, or 0: tiles cut rows)
CASES = [
    (synth.Config("gt_g4_r4", 64, 4, 16, 4, 128, 64, (200, 3000), 6, 2, seed=901, invalid_frac=0.1), 4),
    (synth.Config("gt_g8_r4", 32, 4, 32, 4, 128, 64, (200, 3000), 6, 2, seed=902, invalid_frac=0.1), 2),
    (synth.Config("gt_g5_r3_d64", 64, 3, 20, 4, 64, 64, (200, 3000), 5, 1, seed=903, invalid_frac=0.1), 3),
    (synth.Config("gt_g4_p128", 64, 4, 16, 4, 128, 128, (300, 6000), 4, 1, seed=904, dup_key_frac=0.2), 4),
    (synth.Config("gt_g24_r2", 8, 2, 48, 2, 128, 64, (200, 3000), 6, 2, seed=905, invalid_frac=0.1), 0),
]

_cache = {}
_refs = {}


def _oracle_attention(w, sel):
    """oracle.attention, computed once per (workload, selection): the split and fused variants
    of a case share their selection rows."""
    key = (w.cfg.name, sel.tobytes())
    if key not in _refs:
        _refs[key] = oracle.attention(w, sel)
    return _refs[key]


def _workload(cfg):
    if cfg.name not in _cache:
        _cache[cfg.name] = _ragged_ends(synth.generate(cfg))
    return _cache[cfg.name]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("splits", [1, 2, 3])
@pytest.mark.parametrize("cfg,rows", CASES, ids=lambda v: v.name if isinstance(v, synth.Config) else str(v))
def test_grouped_tiles_vs_oracle(cfg, rows, splits, fused):
    w = _workload(cfg)
    b = DeviceBatch.upload(w)
    plan = q.qsa_plan_decode(b.shape(), splits, fused)
    print(f"[grouped] {cfg.name} N={w.N} rows/tile={plan.rows_per_tile} cols={plan.tile_cols} "
          f"splits={plan.splits} fused={fused}", flush=True)
    assert plan.rows_per_tile == rows and plan.splits == splits
    st = Step(b, num_splits=splits, fused=fused)
    st()
    torch.cuda.synchronize()
    ref_s = oracle.index_scores(w)
    assert np.array_equal(st.scores.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    sel = st.selected.cpu().numpy()
    assert np.array_equal(sel, oracle.select_w(w, ref_s))
    ref_out, ref_lse = _oracle_attention(w, sel)
    _check(st.out.cpu().numpy().view(np.uint16), st.lse.cpu().numpy(), ref_out, ref_lse, cfg.name)
    assert int(b.error_word[0].item()) == 0


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("cfg,rows", CASES[:3] + CASES[4:], ids=lambda v: v.name if isinstance(v, synth.Config) else str(v))
def test_grouped_tiles_disjoint_rows(cfg, rows, splits):
    """Injected scores make the rows of each request select disjoint candidate pages (row j of
    R prefers pages p with p mod R = j), so every union page is visible to one row of its tile;
    the fused launch selects them itself, the composed one from qsa_select_topk."""
    # long enough that every row has k candidates of its own residue
    w = _workload(cfg.with_(name=cfg.name + "_long", context=(2600, 3200)))
    b = DeviceBatch.upload(w)
    assert q.qsa_plan_decode(b.shape(), splits, True).rows_per_tile == rows
    rng = np.random.default_rng(cfg.seed)
    scores = oracle.index_scores(w).copy()
    for bb in range(w.B):
        r0, r1 = int(w.row_offsets[bb]), int(w.row_offsets[bb + 1])
        R = r1 - r0
        for j in range(R):
            row = scores[r0 + j]
            cand = np.isfinite(row)
            p = np.arange(w.MP)
            boost = np.where(p % R == j, 50.0, 0.0).astype(np.float32)
            row[cand] = (boost[cand] + rng.random(int(cand.sum()), dtype=np.float32)).astype(np.float32)
    ref_sel = oracle.select_w(w, scores)
    # the injected scores do what they are for: candidates of different rows of a request differ
    for bb in range(w.B):
        r0, r1 = int(w.row_offsets[bb]), int(w.row_offsets[bb + 1])
        tops = [set(int(p) for p in ref_sel[r] if p >= 0) for r in range(r0, r1)]
        n = -(-int(w.seq_lens[bb]) // w.cfg.page_size)
        win = set(range(max(0, n - w.cfg.window - (r1 - r0)), n))
        for i in range(len(tops)):
            for j in range(i + 1, len(tops)):
                assert not ((tops[i] & tops[j]) - win)
    ref_out, ref_lse = _oracle_attention(w, ref_sel)
    for fused in (True, False):
        st = Step(b, num_splits=splits, fused=fused)
        st.scores.copy_(torch.from_numpy(scores).cuda())
        st.selected.fill_(-7)
        if fused:
            st.select_decode_call()
        else:
            st.select_call()
            st.decode_call()
        torch.cuda.synchronize()
        assert np.array_equal(st.selected.cpu().numpy(), ref_sel)
        _check(st.out.cpu().numpy().view(np.uint16), st.lse.cpu().numpy(), ref_out, ref_lse,
               f"{cfg.name} disjoint fused={fused} splits={splits}")


def test_workspace_reused_by_a_larger_batch():
    """One zero-filled workspace serves a small batch and then a larger one (more tiles, so the
    second call's counters would reach past the first call's if their place followed the tile
    count), then the small one again: each call matches the oracle and leaves the counters zero."""
    small = _workload(CASES[1][0])
    # the first 6 requests of the same workload
    nb = 6
    rows = int(small.row_offsets[nb])
    w_small = synth.Workload(small.cfg, small.page_table[:nb], small.seq_lens[:nb], small.row_offsets[:nb + 1],
                             small.q[:rows], small.k_codes, small.k_scales, small.v_codes, small.v_scales,
                             small.index_keys)
    big = small
    runs = []
    for w, sp in ((w_small, 3), (big, 2), (w_small, 5)):
        b = DeviceBatch.upload(w)
        runs.append((w, b, sp))
    need = max(q.qsa_workspace_bytes(b.shape(), sp) for _, b, sp in runs)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for w, b, sp in runs:
        st = Step(b, num_splits=sp, fused=False)
        st.scores_call()
        st.select_call()
        st.out.fill_(0x1234)
        q.qsa_sparse_decode(st.shape_, st.paged_, b.q, st.selected, st.out, st.lse, sp, ws, None, None)
        torch.cuda.synchronize()
        sel = st.selected.cpu().numpy()
        ref_out, ref_lse = oracle.attention(w, sel)
        _check(st.out.cpu().numpy().view(np.uint16), st.lse.cpu().numpy(), ref_out, ref_lse,
               f"B={w.B} splits={sp}")
        assert int(ws[:32768].count_nonzero().item()) == 0, "counters left non-zero"


@pytest.mark.parametrize("spread", [1, 16])
def test_grouped_tiles_clustered_scores(spread):
    """4-row tiles whose rows' k-th place falls in a cluster of nearly equal scores (at most
    `spread` ulps apart, repeats included): each of the tile's selecting waves runs a long bit
    search through the re-derivation of its interval's common bits. Selection rows and every
    output against the oracle, fused and composed."""
    cfg, rows = CASES[0]
    w = _workload(cfg)
    b = DeviceBatch.upload(w)
    assert q.qsa_plan_decode(b.shape(), 1, True).rows_per_tile == rows
    rng = np.random.default_rng(40 + spread)
    k = w.cfg.topk
    scores = oracle.index_scores(w).copy()
    for r in range(w.N):
        cand = np.flatnonzero(np.isfinite(scores[r]))
        if len(cand) <= k:
            continue
        vals = (rng.standard_normal(len(cand)) - 3.0).astype(np.float32)
        order = rng.permutation(len(cand))
        nb = int(rng.integers(k // 2, k))
        vals[order[:nb]] = 10.0 + rng.random(nb).astype(np.float32)
        nc = min(int(rng.integers(k - nb + 1, k - nb + 6)), len(cand) - nb)
        x0 = np.float32(rng.uniform(0.5, 4.0))
        m = rng.integers(0, spread, size=nc)
        vals[order[nb:nb + nc]] = (x0.view(np.int32) + m).astype(np.int32).view(np.float32)
        scores[r, cand] = vals
    ref_sel = oracle.select_w(w, scores)
    ref_out, ref_lse = _oracle_attention(w, ref_sel)
    for fused in (True, False):
        st = Step(b, num_splits=1, fused=fused)
        st.scores.copy_(torch.from_numpy(scores).cuda())
        st.selected.fill_(-7)
        if fused:
            st.select_decode_call()
        else:
            st.select_call()
            st.decode_call()
        torch.cuda.synchronize()
        assert np.array_equal(st.selected.cpu().numpy(), ref_sel)
        _check(st.out.cpu().numpy().view(np.uint16), st.lse.cpu().numpy(), ref_out, ref_lse,
               f"{cfg.name} clustered spread={spread} fused={fused}")
