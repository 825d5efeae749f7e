"""Pins for the oracle's row bookkeeping, index scores and canonical selection (CPU only).

Row geometry: closed forms. Scores: integer-exact inputs (every fp32 sum exact),
a hand-worked order example (tests/golden/score_sum_order.txt), an fp64 error
bound, and a GQA-mapping probe. Selection: brute force over every tie pattern on
tiny rows, plus the invariants of the canonical rule (TensorRT-LLM PR #20276,
Features, "Canonical QSA selection" row): candidates scoring above the k-th
largest value are kept, and equal scores rank by descending page index.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


# ------------------------------------------------------------------ rows --

def test_rows_closed_form_small():
    # one request, 4 causal verify rows at the end of 65 tokens, 64-token pages
    rq, rl, rn = oracle.rows(np.array([65]), np.array([0, 4]), 64, 4)
    assert list(rl) == [62, 63, 64, 65]
    assert list(rn) == [1, 1, 1, 2]
    assert list(rq) == [0, 0, 0, 0]
    # request with fewer tokens than rows: the early rows see nothing
    rq, rl, rn = oracle.rows(np.array([2, 10]), np.array([0, 4, 5]), 8, 4)
    assert list(rl) == [0, 0, 1, 2, 10]
    assert list(rn) == [0, 0, 1, 1, 2]
    assert list(rq) == [0, 0, 0, 0, 1]


def test_rows_context_step():
    """A context step: R rows at the end of L tokens; row j sees L - (R - 1 - j) of them
    (the causal prefix), in requests of different row counts."""
    seq = np.array([300, 40, 7], np.int32)
    ro = np.array([0, 128, 168, 175], np.int32)               # 128, 40 and 7 rows
    rq, rl, rn = oracle.rows(seq, ro, 64, 8)
    assert list(rl[:128]) == list(range(300 - 127, 301))
    assert list(rl[128:168]) == list(range(1, 41))
    assert list(rl[168:]) == list(range(1, 8))
    assert list(rn[:128]) == [-(-L // 64) for L in range(173, 301)]
    assert list(rq) == [0] * 128 + [1] * 40 + [2] * 7


def test_rows_configs():
    w = synth.generate("mtp_verify_32k")
    rq, rl, rn = oracle.rows(w.seq_lens, w.row_offsets, 64, w.MP)
    assert set(rl.tolist()) == {32765, 32766, 32767, 32768}
    assert set(rn.tolist()) == {512}                         # no page straddle at 32K
    c5 = synth.CONFIGS["wide_mixed"]
    seq = np.array([1024, 1025, 64 * 300 + 2, 65536], np.int32)
    rq, rl, rn = oracle.rows(seq, np.arange(5, dtype=np.int32) * 4, 64, 1024)
    assert list(rn[4:8]) == [16, 16, 16, 17]                  # L = 1022..1025: only the last row reaches page 16
    assert list(rn[8:12]) == [300, 300, 301, 301]
    assert list(rn[12:16]) == [1024] * 4


# ---------------------------------------------------------------- scores --

def _bf16(x):
    return synth.bf16_bits_from_f32(np.asarray(x, np.float32))


def _score_case(q, keys, page_table, seq, ro, P, W, sm_scale, Hkv):
    """Wrap raw arrays into a minimal workload object for oracle.index_scores."""
    cfg = synth.Config("t", len(seq), 1, q.shape[1], Hkv, q.shape[2], P, 0, 0, W, seed=0)
    w = synth.Workload(cfg, np.asarray(page_table, np.int32), np.asarray(seq, np.int32),
                       np.asarray(ro, np.int32), q, None, None, None, None, keys)
    return oracle.index_scores(w, sm_scale=sm_scale, q=q, keys=keys, page_table=page_table)


def test_scores_integer_exact_and_max_over_heads():
    rng = np.random.default_rng(3)
    N, Hq, Hkv, d, MP, P = 3, 6, 3, 32, 9, 4
    qi = rng.integers(-8, 9, size=(N, Hq, d))
    ki = rng.integers(-8, 9, size=(MP + 2, Hkv, d))
    q, keys = _bf16(qi), _bf16(ki)
    pt = np.array([[5, 2, 7, 0, 1, 3, -1, 4, 6]], np.int32)
    seq = [MP * P]
    ro = [0, N]
    sm = np.float32(0.125)
    s = _score_case(q, keys, pt, seq, ro, P, 2, sm, Hkv)
    rq, rl, rn = oracle.rows(np.array(seq), np.array(ro), P, MP)
    G = Hq // Hkv
    for r in range(N):
        for p in range(MP):
            phys = pt[0, p]
            if p >= rn[r] - 2 or phys < 0:
                assert s[r, p] == -np.inf
                continue
            dots = [int(np.dot(qi[r, h], ki[phys, h // G])) for h in range(Hq)]
            want = np.float32(sm * np.float32(max(dots)))
            assert s[r, p] == want, (r, p)


def test_scores_sequential_sum_worked_example():
    for row in read_golden("score_sum_order.txt"):
        vals = list(map(float, row))
        qv, kv, want = vals[:4], vals[4:8], vals[8]
        d = 16
        q = np.zeros((1, 1, d), np.float32)
        k = np.zeros((2, 1, d), np.float32)
        q[0, 0, :4] = qv
        k[0, 0, :4] = kv
        s = _score_case(_bf16(q), _bf16(k), np.array([[0, 1]]), [2], [0, 1], 1, 1, np.float32(1.0), 1)
        assert s[0, 0] == want
        assert s[0, 1] == -np.inf                      # the window page is never scored


def test_scores_fp64_error_bound():
    w = synth.generate(synth.CONFIGS["decode_8k"].with_(batch=2, context=1024))
    s = oracle.index_scores(w)
    q = synth.f32_from_bf16_bits(w.q).astype(np.float64)
    k = synth.f32_from_bf16_bits(w.index_keys).astype(np.float64)
    Hq, Hkv, d = w.cfg.q_heads, w.cfg.kv_heads, w.cfg.head_dim
    G = Hq // Hkv
    u = 2.0 ** -24
    rq, rl, rn = oracle.rows(w.seq_lens, w.row_offsets, w.cfg.page_size, w.MP)
    for r in range(w.N):
        for p in range(w.MP):
            phys = w.page_table[rq[r], p]
            if p >= rn[r] - w.cfg.window:
                assert s[r, p] == -np.inf
                continue
            prods = q[r] * k[phys][np.arange(Hq) // G]              # [Hq][d]
            exact = prods.sum(axis=1)
            bound = (d * u / (1 - d * u)) * np.abs(prods).sum(axis=1)
            hi = np.max(exact + bound)
            lo = np.max(exact - bound)
            sm = w.sm_scale
            assert lo * sm * (1 - u) - 1e-30 <= s[r, p] <= hi * sm * (1 + u) + 1e-30


def test_scores_gqa_mapping():
    """Only KV head h // G feeds q head h: a transposed or wrong head map fails."""
    N, Hq, Hkv, d = 1, 8, 4, 16
    G = Hq // Hkv
    for g_hot in range(Hkv):
        for h_hot in range(Hq):
            q = np.zeros((N, Hq, d), np.float32)
            q[0, h_hot, 0] = 1.0
            k = np.zeros((2, Hkv, d), np.float32)
            k[0, g_hot, 0] = 2.0
            s = _score_case(_bf16(q), _bf16(k), np.array([[0, 1]]), [2], [0, 1], 1, 1,
                            np.float32(1.0), Hkv)
            assert s[0, 0] == (2.0 if h_hot // G == g_hot else 0.0)


# ------------------------------------------------------------- selection --

def _brute(scores_row, n, k, W):
    wlo = max(0, n - W)
    cand = [p for p in range(wlo) if not (math.isnan(scores_row[p]) or scores_row[p] == -math.inf)]
    ranked = sorted(cand, key=lambda p: (-scores_row[p], -p))[:k]
    sel = sorted(set(ranked) | set(range(wlo, n)))
    return sel


def test_select_brute_force_all_tie_patterns():
    """Every score pattern over {0, 1, 2} on up to 6 candidates, every k, W in 0..2."""
    for n in range(0, 7):
        for pat in itertools.product([0.0, 1.0, 2.0], repeat=n):
            for W in range(0, 3):
                ntot = n + W
                scores = np.full((1, max(ntot, 1)), -np.inf, np.float32)
                scores[0, :n] = pat
                MP = scores.shape[1]
                seq = np.array([ntot], np.int32)          # P = 1: one token per page
                for k in range(0, n + 2):
                    got = oracle.select(seq, np.array([0, 1]), 1, MP, k, W, scores)[0]
                    want = _brute(scores[0].tolist(), ntot, k, W)
                    assert list(got[:len(want)]) == want and all(got[len(want):] == -1), \
                        (pat, k, W, got, want)


def test_select_signed_zero_ties_and_nonfinite():
    s = np.array([[0.0, -0.0, 0.0, -0.0, np.nan, -np.inf, 1.0, 0.0]], np.float32)
    got = oracle.select(np.array([8]), np.array([0, 1]), 1, 8, 3, 1, s)[0]
    # candidates 0..6 (window = page 7); 1.0 at 6 first; then the zeros tie: highest indices 3, 2
    assert list(got) == [2, 3, 6, 7]


def test_select_invariants_on_config():
    w = synth.generate("mtp_verify_32k")
    s = oracle.index_scores(w)
    sel = oracle.select_w(w, s)
    k, W = w.cfg.topk, w.cfg.window
    rq, rl, rn = oracle.rows(w.seq_lens, w.row_offsets, w.cfg.page_size, w.MP)
    decisive = 0
    for r in range(w.N):
        n = rn[r]
        row = [p for p in sel[r] if p >= 0]
        assert row == sorted(set(row))
        win = set(range(max(0, n - W), n))
        assert win <= set(row)
        ranked = [p for p in row if p not in win]
        cand = [p for p in range(max(0, n - W)) if np.isfinite(s[r, p])]
        assert len(ranked) == min(k, len(cand))
        unsel = [p for p in cand if p not in ranked]
        if ranked and unsel:
            thr = min(s[r, p] for p in ranked)
            assert all(s[r, p] <= thr for p in unsel)
            tied_out = [p for p in unsel if s[r, p] == thr]
            tied_in = [p for p in ranked if s[r, p] == thr]
            if tied_out:
                decisive += 1
                assert min(tied_in) > max(tied_out)
    # the copied index keys make the tie rule decide at least one row of this workload
    assert decisive >= 1


def test_select_ignores_physical_ids():
    """Permuting physical page ids (and their keys) leaves the selection unchanged."""
    w = synth.generate(synth.CONFIGS["decode_8k"].with_(batch=3, context=2048))
    s0 = oracle.index_scores(w)
    perm = np.random.default_rng(1).permutation(w.NP).astype(np.int32)
    pt = np.where(w.page_table >= 0, perm[np.maximum(w.page_table, 0)], -1).astype(np.int32)
    keys = np.empty_like(w.index_keys)
    keys[perm] = w.index_keys
    s1 = oracle.index_scores(w, keys=keys, page_table=pt)
    assert np.array_equal(s0, s1)
    assert np.array_equal(oracle.select_w(w, s0), oracle.select_w(w, s1))


def test_select_k_edges():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((1, 20)).astype(np.float32)
    seq, ro = np.array([20]), np.array([0, 1])
    allc = oracle.select(seq, ro, 1, 20, 50, 2, s)[0]
    assert list(allc[:20]) == list(range(20)) and all(allc[20:] == -1)
    none = oracle.select(seq, ro, 1, 20, 0, 2, s)[0]
    assert list(none) == [18, 19]
    # window wider than the row: clipped at page 0
    short = oracle.select(np.array([1]), ro, 1, 20, 3, 4, s)[0]
    assert list(short) == [0, -1, -1, -1, -1, -1, -1]
