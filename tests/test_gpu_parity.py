"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bars: dequantised values, index scores and selected pages bit-exact; attention output
within |gpu - ref| <= 2e-3 + 1e-2 |ref| (elementwise, against the fp64 oracle); lse within
2e-3 absolute. Full-size workloads are checked on all scores and selections and on
sampled attention outputs (the oracle evaluates those one (row, head) at a time), in the
launch configuration the benchmark uses.
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


_cache = {}


def workload(name_or_cfg):
    key = name_or_cfg if isinstance(name_or_cfg, str) else repr(name_or_cfg)
    if key not in _cache:
        _cache[key] = synth.generate(name_or_cfg)
    return _cache[key]


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


def _bf16_to_f64(bits):
    return synth.f32_from_bf16_bits(bits).astype(np.float64)


def _check_attention(out_bits, lse, ref_out, ref_lse, where=""):
    out = _bf16_to_f64(out_bits)
    err = np.abs(out - ref_out) - (ATOL + RTOL * np.abs(ref_out))
    assert err.max(initial=-1) <= 0, f"{where}: out beyond tolerance by {err.max()}"
    if lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(lse)), where
        if fin.any():
            assert np.abs(lse[fin] - ref_lse[fin]).max() <= LSE_TOL, where


def _run(w, num_splits=0, sel_override=None):
    b = DeviceBatch.upload(w)
    st = Step(b, num_splits=num_splits)
    st.scores_call()
    st.select_call()
    if sel_override is not None:
        st.selected.copy_(torch.from_numpy(sel_override).cuda())
    st.decode_call()
    torch.cuda.synchronize()
    return b, st


# ------------------------------------------------------------------------ dequant --

@pytest.mark.parametrize("d,P,Hkv", [(128, 64, 1), (64, 128, 2)])
@pytest.mark.parametrize("g", [1.0, 0.5, 3.0])
def test_dequant_every_code_and_scale_bitwise(d, P, Hkv, g):
    """Every (code byte, scale byte) pair, through the attention kernel's decode function."""
    NP = 256
    codes = ((np.arange(NP * Hkv * P * d // 2) * 7 + 3) % 256).astype(np.uint8).reshape(NP, Hkv, P, d // 2)
    scales = np.broadcast_to(np.arange(NP, dtype=np.uint8)[:, None, None, None], (NP, Hkv, P, d // 16)).copy()
    pages = np.arange(NP, dtype=np.int32)
    sh = q.Shape(1, 1, 1, Hkv, Hkv, d, P, 1, NP, 0, 1, 1.0)
    out = torch.empty((NP, Hkv, P, d), dtype=torch.float32, device="cuda")
    q.qsa_nvfp4_dequant_pages(sh, torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), g,
                              torch.from_numpy(pages).cuda(), NP, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.dequant_pages(codes, scales, g, pages).astype(np.float32)   # exact products -> one rounding
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ------------------------------------------------------------ scores and selection --

SMALL = [
    synth.Config("s_d64_g4", 2, 1, 4, 1, 64, 64, 1000, 4, 1, seed=101),
    synth.Config("s_verify_ragged", 5, 4, 16, 2, 128, 64, (60, 3000), 6, 2, seed=102, invalid_frac=0.1),
    synth.Config("s_hkv8_p128", 3, 2, 16, 8, 128, 128, (500, 9000), 8, 1, seed=103, max_pages=77),
    synth.Config("s_g1_d64", 2, 3, 4, 4, 64, 128, (129, 700), 3, 3, seed=104, dup_key_frac=0.3),
    # more than 8 q heads per KV head: several head groups per KV head, the last one partial
    # at 12, and at 8 KV heads on a small grid the eight-wave launch
    synth.Config("s_g16_d128", 2, 4, 32, 2, 128, 64, 9000, 6, 2, seed=105),
    synth.Config("s_g12_d64", 2, 2, 24, 2, 64, 64, (100, 3000), 5, 1, seed=106, dup_key_frac=0.2),
    synth.Config("s_hkv8_g12", 2, 1, 96, 8, 128, 64, (200, 2000), 4, 1, seed=107, invalid_frac=0.05),
    # a large grid (6400 waves) with an odd number of rows per request
    synth.Config("s_rows5_large", 64, 5, 16, 2, 64, 64, (3000, 20000), 8, 1, seed=108, invalid_frac=0.05),
    # rows of 16 and 24 page tiles (two and three aligned groups of 8), whose index launch starts
    # the tile groups one after another: batches that are not a multiple of 8, and short
    # requests whose later groups hold no page; one pass per KV head and (12 q heads per KV
    # head) two head groups
    synth.Config("s_ord_16tiles", 5, 3, 16, 4, 128, 64, (200, 60000), 6, 2, seed=111, invalid_frac=0.05,
                 max_pages=1024),
    synth.Config("s_ord_24tiles_g12", 3, 2, 24, 2, 64, 64, (100, 95000), 5, 1, seed=112, max_pages=1536),
]
CONFIG_NAMES = list(synth.CONFIGS)


@pytest.mark.parametrize("cfg", SMALL + CONFIG_NAMES, ids=lambda c: c if isinstance(c, str) else c.name)
def test_scores_and_selection_bitwise(cfg):
    w = workload(cfg)
    print(f"[scores/select] {w.cfg.name} N={w.N} MP={w.MP} NP={w.NP}", flush=True)
    b = DeviceBatch.upload(w)
    st = Step(b)
    st.scores_call()
    st.select_call()
    torch.cuda.synchronize()
    ref_s = oracle.index_scores(w)
    got_s = st.scores.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), ref_s.view(np.uint32))
    ref_sel = oracle.select_w(w, ref_s)
    assert np.array_equal(st.selected.cpu().numpy(), ref_sel)
    assert int(b.error_word[0].item()) == 0


@pytest.mark.parametrize("seed,MP,k,W,R", [(1, 64, 4, 1, 1), (2, 300, 16, 2, 4), (3, 1000, 32, 2, 3),
                                           (4, 4096, 200, 7, 2), (5, 17, 40, 3, 4), (6, 513, 0, 2, 1)])
def test_selection_on_injected_tie_heavy_scores(seed, MP, k, W, R):
    """Scores from a 5-value set (both zero signs, NaN and -inf mixed in): the tie rule decides."""
    rng = np.random.default_rng(seed)
    B, P = 6, 64
    seq = np.maximum(rng.integers(1, MP * P + 1, size=B), R).astype(np.int32)
    ro = (np.arange(B + 1) * R).astype(np.int32)
    N = B * R
    vals = np.array([1.5, 0.0, -0.0, -2.0, 7.25], np.float32)
    scores = vals[rng.integers(0, 5, size=(N, MP))]
    holes = rng.random((N, MP))
    scores[holes < 0.05] = np.nan
    scores[(holes >= 0.05) & (holes < 0.1)] = -np.inf
    ref = oracle.select(seq, ro, P, MP, k, W, scores)
    sh = q.Shape(B, N, R, 1, 1, 64, P, MP, 1, k, W, 1.0)
    seq_d, ro_d, sc_d = (torch.from_numpy(a).cuda() for a in (seq, ro, scores))
    pg = q.Paged(None, seq_d.data_ptr(), ro_d.data_ptr(), None, None, None, None, None, 1.0, 1.0, None)
    sel = torch.empty((N, k + W), dtype=torch.int32, device="cuda")
    q.qsa_select_topk(sh, pg, sc_d, sel)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), ref)


@pytest.mark.parametrize("rows,context,k,W,splits", [(1, (64, 4000), 4, 1, 1), (1, (64, 4000), 0, 2, 1),
                                                      (1, (100, 40000), 40, 3, 1), (2, (64, 9000), 6, 2, 2),
                                                      (1, (3000, 60000), 200, 2, 2)])
def test_fused_selection_on_injected_tie_heavy_scores(rows, context, k, W, splits):
    """The selection fused into the attention launch (one-row tiles write their union from the
    selecting wave) on scores from a 5-value set with NaN and -inf mixed in, k = 0 and k above
    the candidates: the oracle's rows, and bit for bit the composed calls' outputs."""
    cfg = synth.Config("fused_ties", 5, rows, 8, 2, 64, 64, context, k, W, seed=311 + k, invalid_frac=0.05)
    w = workload(cfg)
    b = DeviceBatch.upload(w)
    rng = np.random.default_rng(17 + k)
    vals = np.array([1.5, 0.0, -0.0, -2.0, 7.25], np.float32)
    scores = vals[rng.integers(0, 5, size=(w.N, w.MP))]
    holes = rng.random((w.N, w.MP))
    scores[holes < 0.05] = np.nan
    scores[(holes >= 0.05) & (holes < 0.1)] = -np.inf
    print(f"[fused ties] rows={rows} MP={w.MP} k={k} W={W} splits={splits}", flush=True)
    ref = Step(b, num_splits=splits, fused=False)
    fus = Step(b, num_splits=splits, fused=True)
    for st in (ref, fus):
        st.scores.copy_(torch.from_numpy(scores).cuda())
    ref.select_call()
    ref.decode_call()
    fus.selected.fill_(-7)
    fus.select_decode_call()
    torch.cuda.synchronize()
    ref_sel = oracle.select_w(w, scores)
    assert np.array_equal(ref.selected.cpu().numpy(), ref_sel)
    assert np.array_equal(fus.selected.cpu().numpy(), ref_sel)
    assert torch.equal(fus.out, ref.out) and torch.equal(fus.lse, ref.lse)
    ref_out, ref_lse = oracle.attention(w, ref_sel)
    _check_attention(_u16(fus.out), fus.lse.cpu().numpy(), ref_out, ref_lse, "fused ties")


def _cluster_scores(rng, N, MP, k, spread):
    """Rows whose k-th place falls in a cluster of values at most `spread` ulps apart (repeats
    included), above a spread of lower values and below fewer than k clearly larger ones: the
    bit search runs past its re-derivation step, where the interval's keys are all equal
    (spread 1) or still differ in their low bits (the search then restarts below them)."""
    s = (rng.standard_normal((N, MP)) - 3.0).astype(np.float32)
    for r in range(N):
        nb = int(rng.integers(k // 2, k))
        cols = rng.permutation(MP)
        s[r, cols[:nb]] = 10.0 + rng.random(nb).astype(np.float32)
        nc = int(rng.integers(k - nb + 1, k - nb + 12))
        x0 = np.float32(rng.uniform(0.5, 4.0))
        m = rng.integers(0, spread, size=nc)
        s[r, cols[nb:nb + nc]] = (x0.view(np.int32) + m).astype(np.int32).view(np.float32)
    return s


@pytest.mark.parametrize("spread", [1, 4, 64, 4096])
def test_selection_on_clustered_scores(spread):
    """The k-th place inside a cluster of nearly equal scores: long bit searches, through the
    re-derivation of the interval's common bits, against the oracle row by row."""
    rng = np.random.default_rng(100 + spread)
    B, R, P, MP, k, W = 40, 4, 64, 1000, 32, 2
    seq = np.full(B, MP * P, np.int32)
    ro = (np.arange(B + 1) * R).astype(np.int32)
    N = B * R
    scores = _cluster_scores(rng, N, MP, k, spread)
    ref = oracle.select(seq, ro, P, MP, k, W, scores)
    sh = q.Shape(B, N, R, 1, 1, 64, P, MP, 1, k, W, 1.0)
    seq_d, ro_d, sc_d = (torch.from_numpy(a).cuda() for a in (seq, ro, scores))
    pg = q.Paged(None, seq_d.data_ptr(), ro_d.data_ptr(), None, None, None, None, None, 1.0, 1.0, None)
    sel = torch.empty((N, k + W), dtype=torch.int32, device="cuda")
    q.qsa_select_topk(sh, pg, sc_d, sel)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), ref)


@pytest.mark.parametrize("spread", [1, 16])
def test_fused_selection_on_clustered_scores(spread):
    """The same score tables through the selection fused into the attention launch: the
    oracle's rows, and bit for bit the composed calls' outputs."""
    cfg = synth.Config("fused_cluster", 6, 4, 8, 2, 64, 64, (40000, 60000), 32, 2, seed=331 + spread)
    w = workload(cfg)
    b = DeviceBatch.upload(w)
    scores = _cluster_scores(np.random.default_rng(7 + spread), w.N, w.MP, 32, spread)
    print(f"[fused cluster] MP={w.MP} spread={spread}", flush=True)
    ref = Step(b, fused=False)
    fus = Step(b, fused=True)
    for st in (ref, fus):
        st.scores.copy_(torch.from_numpy(scores).cuda())
    ref.select_call()
    ref.decode_call()
    fus.selected.fill_(-7)
    fus.select_decode_call()
    torch.cuda.synchronize()
    ref_sel = oracle.select_w(w, scores)
    assert np.array_equal(ref.selected.cpu().numpy(), ref_sel)
    assert np.array_equal(fus.selected.cpu().numpy(), ref_sel)
    assert torch.equal(fus.out, ref.out) and torch.equal(fus.lse, ref.lse)


def test_selection_repeated_launch_determinism():
    """The same rows launched 50 times select identical sets in identical order."""
    w = workload("mtp_verify_32k")
    b = DeviceBatch.upload(w)
    st = Step(b)
    st.scores_call()
    first = None
    for _ in range(50):
        st.select_call()
        cur = st.selected.clone()
        if first is None:
            first = cur
        else:
            assert torch.equal(cur, first)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------- attention --

ATT_SMALL = [
    synth.Config("a_tiny", 1, 1, 4, 1, 64, 64, 1024, 4, 1, seed=0, shuffled=False),
    synth.Config("a_decode", 4, 1, 16, 2, 128, 64, (100, 5000), 8, 2, seed=201),
    synth.Config("a_verify", 5, 4, 16, 2, 128, 64, (60, 6000), 6, 2, seed=202, invalid_frac=0.1),
    synth.Config("a_p128", 3, 2, 16, 2, 128, 128, (129, 9000), 5, 1, seed=203, outlier_frac=0.01),
    synth.Config("a_d64_g16", 2, 4, 32, 2, 64, 64, (300, 4000), 6, 2, seed=204),
    synth.Config("a_g2", 3, 3, 8, 4, 128, 64, (70, 2000), 5, 3, seed=205, dup_key_frac=0.2),
]


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7])
@pytest.mark.parametrize("cfg", ATT_SMALL, ids=lambda c: c.name)
def test_attention_small_vs_oracle(cfg, splits):
    w = workload(cfg)
    print(f"[attention] {cfg.name} splits={splits}", flush=True)
    b, st = _run(w, num_splits=splits)
    sel = st.selected.cpu().numpy()
    assert np.array_equal(sel, oracle.select_w(w, oracle.index_scores(w)))
    ref_out, ref_lse = oracle.attention(w, sel)
    _check_attention(_u16(st.out), st.lse.cpu().numpy(), ref_out, ref_lse, cfg.name)
    assert int(b.error_word[0].item()) == 0


def test_attention_split_invariance_bitwise_per_split_count():
    """Fixed split count -> bitwise reproducible; all split counts agree within tolerance."""
    w = workload(ATT_SMALL[2])
    outs = []
    for splits in (1, 2, 4, 64):
        b, st = _run(w, num_splits=splits)
        a = _u16(st.out).copy()
        st.decode_call()
        torch.cuda.synchronize()
        assert np.array_equal(a, _u16(st.out))
        outs.append(_bf16_to_f64(a))
    for o in outs[1:]:
        assert np.all(np.abs(o - outs[0]) <= ATOL + RTOL * np.abs(outs[0]))


def test_workspace_reused_across_split_counts():
    """One zero-filled workspace serves calls with different split counts: every call
    leaves the per-tile completion counters (the first bytes) zero and matches the oracle."""
    w = workload(ATT_SMALL[3])
    b = DeviceBatch.upload(w)
    st = Step(b, num_splits=7)
    st.scores_call()
    st.select_call()
    torch.cuda.synchronize()
    sel = st.selected.cpu().numpy()
    ref_out, ref_lse = oracle.attention(w, sel)
    sh = b.shape()
    # the counters come first: workspace(S) = counter bytes + tiles * S * per-split partial
    part = ((w.cfg.head_dim // 16 + 1) * 64 * 4 + 64) * 4
    tiles = (q.qsa_workspace_bytes(sh, 3) - q.qsa_workspace_bytes(sh, 2)) // part
    assert tiles > 0
    ws = torch.zeros(max(q.qsa_workspace_bytes(sh, sp) for sp in (7, 2, 5, 3)), dtype=torch.uint8, device="cuda")
    for sp in (7, 2, 5, 3, 7):
        st.out.fill_(0x1234)
        q.qsa_sparse_decode(sh, st.paged_, b.q, st.selected, st.out, st.lse, sp, ws, None, None)
        torch.cuda.synchronize()
        _check_attention(_u16(st.out), st.lse.cpu().numpy(), ref_out, ref_lse, f"ws reuse splits={sp}")
        assert int(ws[:tiles * 4].count_nonzero().item()) == 0, f"counters left non-zero after splits={sp}"


FUSED_CASES = [(c, sp) for c in ATT_SMALL[:4] for sp in (0, 1, 3)] + [(n, 0) for n in CONFIG_NAMES] + [
    (synth.Config("f_wide_table", 3, 2, 16, 2, 128, 64, (300, 5000), 6, 2, seed=401, max_pages=1500), 0),
    (synth.Config("f_mp1024", 2, 4, 32, 4, 64, 64, (900, 60000), 8, 1, seed=402, invalid_frac=0.1), 2),
]


@pytest.mark.parametrize("cfg,splits", FUSED_CASES,
                         ids=lambda v: v if isinstance(v, (str, int)) else v.name)
def test_fused_select_decode_equals_composed(cfg, splits):
    """qsa_select_sparse_decode (selection in the attention launch; two launches past 1024
    table columns) writes the oracle's rows and, bit for bit, the composed calls' outputs."""
    w = workload(cfg)
    print(f"[fused select+decode] {w.cfg.name} MP={w.MP} splits={splits}", flush=True)
    b = DeviceBatch.upload(w)
    ref = Step(b, num_splits=splits, fused=False)
    ref()
    fus = Step(b, num_splits=splits, fused=True)
    fus.selected.fill_(-7)
    fus.out.fill_(0x1234)
    fus()
    torch.cuda.synchronize()
    ref_sel = oracle.select_w(w, oracle.index_scores(w))
    assert np.array_equal(ref.selected.cpu().numpy(), ref_sel)
    assert np.array_equal(fus.selected.cpu().numpy(), ref_sel)
    assert torch.equal(fus.out, ref.out)
    assert torch.equal(fus.lse, ref.lse)
    assert int(b.error_word[0].item()) == 0
    if not isinstance(cfg, str):
        # the small and wide-table cases are also compared with the oracle on every output
        # (the full-size workloads on sampled outputs, in test_attention_full_size_sampled)
        ref_out, ref_lse = oracle.attention(w, ref_sel)
        _check_attention(_u16(fus.out), fus.lse.cpu().numpy(), ref_out, ref_lse, w.cfg.name)


SAMPLES = 24


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_attention_full_size_sampled(name):
    w = workload(name)
    print(f"[attention full] {name} N={w.N}", flush=True)
    b, st = _run(w)
    sel = st.selected.cpu().numpy()
    out = _u16(st.out)
    lse = st.lse.cpu().numpy()
    assert int(b.error_word[0].item()) == 0
    assert np.all(np.isfinite(_bf16_to_f64(out)))
    rng = np.random.default_rng(7)
    Hq = w.cfg.q_heads
    pairs = {(0, 0), (w.N - 1, Hq - 1)} | {(int(r), int(h)) for r, h in
                                            zip(rng.integers(0, w.N, SAMPLES), rng.integers(0, Hq, SAMPLES))}
    for r, h in sorted(pairs):
        ref_o, ref_l = oracle.attention_one(w, sel, r, h)
        _check_attention(out[r, h][None], np.array([lse[r, h]]), ref_o[None], np.array([ref_l]), f"{name} r{r} h{h}")


# --------------------------------------------------------------------- edge cases --

@pytest.mark.parametrize("splits", [1, 3])
def test_attention_edge_selections(splits):
    """Empty rows, pages past a row's length, duplicates, invalid pages, out-of-range ids.
    With one split, rows that leave out a page of their window take the path without
    early window units."""
    cfg = synth.Config("edge", 4, 4, 16, 2, 128, 64, (10, 700), 4, 2, seed=301, invalid_frac=0.2)
    w = workload(cfg)
    base = oracle.select_w(w, oracle.index_scores(w))
    sel = base.copy()
    sel[0] = -1                                    # empty row
    sel[1, :3] = [0, 0, 0]                          # duplicates count once
    sel[2, -1] = w.MP - 1                           # a page at/after the row's end
    sel[3, -2:] = -1                                # the window left out
    b, st = _run(w, num_splits=splits, sel_override=sel)
    ref_out, ref_lse = oracle.attention(w, sel)
    _check_attention(_u16(st.out), st.lse.cpu().numpy(), ref_out, ref_lse, "edge")
    out0 = _u16(st.out)[0]
    assert np.all(out0 == 0) and np.all(np.isneginf(st.lse.cpu().numpy()[0]))
    # an out-of-range id is ignored and reported
    sel2 = base.copy()
    sel2[3, 0] = w.MP + 5
    b.error_word.zero_()
    st.selected.copy_(torch.from_numpy(sel2).cuda())
    st.decode_call()
    torch.cuda.synchronize()
    assert int(b.error_word[0].item()) & q.QSA_DEVERR_SELECTED
    sel2[3, 0] = -1
    ref_out, ref_lse = oracle.attention(w, sel2)
    _check_attention(_u16(st.out), st.lse.cpu().numpy(), ref_out, ref_lse, "edge-oor")


@pytest.mark.parametrize("splits", [1, 2])
def test_short_request_and_bad_page_ids(splits):
    """A request shorter than its rows, and a page-table entry >= NP (treated as -1, flagged),
    with one split inside the pages every row's window holds."""
    cfg = synth.Config("short", 3, 4, 8, 2, 64, 64, (1, 300), 3, 1, seed=302)
    w = workload(cfg)
    w = dataclasses.replace(w)
    w.seq_lens = w.seq_lens.copy()
    w.seq_lens[1] = 2                               # 4 rows, 2 tokens: the first two rows see nothing
    w.page_table = w.page_table.copy()
    n0 = -(-int(w.seq_lens[0]) // 64)
    w.page_table[0, n0 - 1] = w.NP + 3              # out-of-range physical id in row 0's window
    b, st = _run(w, num_splits=splits)
    ref_s = oracle.index_scores(w)
    assert np.array_equal(st.scores.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    sel = st.selected.cpu().numpy()
    assert np.array_equal(sel, oracle.select_w(w, ref_s))
    ref_out, ref_lse = oracle.attention(w, sel)
    _check_attention(_u16(st.out), st.lse.cpu().numpy(), ref_out, ref_lse, "short")
    err = int(b.error_word[0].item())
    assert err & q.QSA_DEVERR_PAGE_ID and err & q.QSA_DEVERR_SEQ_LEN


@pytest.mark.parametrize("splits", [1, 2])
def test_fused_bad_page_ids(splits):
    """The selection fused into the attention launch (one-row tiles: the selecting wave builds the
    union itself) with -1 entries and a page-table entry >= NP inside a row's window: the same
    selection rows and outputs as the composed calls, the oracle's attention, and the PAGE_ID bit."""
    cfg = synth.Config("fused_bad", 3, 1, 8, 2, 64, 64, (300, 2000), 4, 2, seed=303, invalid_frac=0.15)
    w = dataclasses.replace(workload(cfg))
    w.page_table = w.page_table.copy()
    n1 = -(-int(w.seq_lens[1]) // 64)
    w.page_table[1, n1 - 1] = w.NP + 7              # out-of-range physical id in request 1's window
    b = DeviceBatch.upload(w)
    ref = Step(b, num_splits=splits, fused=False)
    ref()
    torch.cuda.synchronize()
    err_ref = int(b.error_word[0].item())
    b.error_word.zero_()
    fus = Step(b, num_splits=splits, fused=True)
    fus.selected.fill_(-7)
    fus()
    torch.cuda.synchronize()
    err = int(b.error_word[0].item())
    ref_s = oracle.index_scores(w)
    ref_sel = oracle.select_w(w, ref_s)
    assert np.array_equal(fus.selected.cpu().numpy(), ref_sel)
    assert torch.equal(fus.out, ref.out) and torch.equal(fus.lse, ref.lse)
    ref_out, ref_lse = oracle.attention(w, ref_sel)
    _check_attention(_u16(fus.out), fus.lse.cpu().numpy(), ref_out, ref_lse, "fused bad pages")
    assert err & q.QSA_DEVERR_PAGE_ID and err_ref & q.QSA_DEVERR_PAGE_ID


def test_graph_capture_replay():
    """The three calls captured in one graph: every replay equals the eager step bitwise."""
    w = workload(ATT_SMALL[2])
    b = DeviceBatch.upload(w)
    st = Step(b, num_splits=3)
    st()
    torch.cuda.synchronize()
    eager = (st.scores.clone(), st.selected.clone(), st.out.clone(), st.lse.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st(stream=torch.cuda.current_stream())
    for i in range(4):
        st.out.fill_(0x1234)
        st.scores.fill_(1.0)
        st.selected.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.scores, eager[0]) and torch.equal(st.selected, eager[1])
        assert torch.equal(st.out, eager[2]) and torch.equal(st.lse, eager[3]), f"replay {i}"


def test_uniform_rows_offsets_checked():
    """When num_rows is B * max_rows, the kernels take request b's rows as [b * R, (b + 1) * R)
    without waiting for row_offsets, and compare the offsets with that afterwards: offsets that
    say otherwise set the ROWS bit, in the index scores and in both attention calls."""
    cfg = synth.Config("uni_rows", 3, 4, 8, 2, 64, 64, (300, 2000), 4, 1, seed=309)
    w = workload(cfg)
    b = DeviceBatch.upload(w)
    st = Step(b, num_splits=1)
    st()
    torch.cuda.synchronize()
    assert int(b.error_word[0].item()) == 0
    # the same total, split 3 + 5 + 4: still N == B * R, but request 0 has 3 rows
    b.row_offsets.copy_(torch.tensor([0, 3, 8, 12], dtype=torch.int32))
    for call in (st.scores_call, st.select_decode_call, st.decode_call):
        b.error_word.zero_()
        call()
        torch.cuda.synchronize()
        assert int(b.error_word[0].item()) & q.QSA_DEVERR_ROWS, call.__name__


@pytest.mark.parametrize("a", [100, 60, -20])
def test_q_scaled_by_a_power_of_two(a):
    """q * 2^a with sm_scale * 2^-a has the same logits: q far beyond f16's range (a = 100, 60)
    and q in f16's subnormal range (a = -20) give the same scores, selections, outputs and lse,
    bit for bit, as unscaled q, and the oracle's attention (each query column's q operand is
    scaled into range by a power of two that its logit scale takes back)."""
    cfg = synth.Config("q_pow2", 3, 4, 16, 2, 128, 64, (300, 3000), 5, 2, seed=310, invalid_frac=0.1)
    w = workload(cfg)
    ref_b = DeviceBatch.upload(w)
    ref = Step(ref_b, num_splits=2)
    ref()
    w2 = dataclasses.replace(w)
    w2.q = synth.bf16_bits_from_f32(synth.f32_from_bf16_bits(w.q) * np.float32(2.0 ** a))
    assert np.array_equal(synth.f32_from_bf16_bits(w2.q), synth.f32_from_bf16_bits(w.q) * np.float32(2.0 ** a))
    b2 = DeviceBatch.upload(w2)
    b2.sm_scale = float(np.float32(w.sm_scale) * np.float32(2.0 ** -a))
    for fused in (True, False):
        st = Step(b2, num_splits=2, fused=fused)
        st()
        torch.cuda.synchronize()
        assert torch.equal(st.scores, ref.scores) and torch.equal(st.selected, ref.selected), fused
        assert torch.equal(st.out, ref.out) and torch.equal(st.lse, ref.lse), fused
    assert int(b2.error_word[0].item()) == 0
    sel = st.selected.cpu().numpy()
    ref_out, ref_lse = oracle.attention(w2, sel, sm_scale=b2.sm_scale)
    _check_attention(_u16(st.out), st.lse.cpu().numpy(), ref_out, ref_lse, f"q * 2^{a}")


def test_non_finite_q_is_flagged():
    """A q element that is not finite sets the Q_RANGE bit (the other rows are unaffected)."""
    cfg = synth.Config("q_inf", 2, 2, 8, 2, 64, 64, (300, 2000), 4, 1, seed=311)
    w = dataclasses.replace(workload(cfg))
    w.q = w.q.copy()
    w.q[1, 3, 5] = 0x7F80                          # +inf in bf16
    b, st = _run(w, num_splits=1)
    assert int(b.error_word[0].item()) & q.QSA_DEVERR_Q_RANGE
    good = [r for r in range(w.N) if r != 1]
    ref_out, ref_lse = oracle.attention(w, st.selected.cpu().numpy())
    _check_attention(_u16(st.out)[good], st.lse.cpu().numpy()[good], ref_out[good], ref_lse[good], "q inf")
