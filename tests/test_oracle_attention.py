"""Pins for the oracle's sparse attention (CPU only).

* Brute-force dense softmax in numpy over the gathered token list (tiny inputs).
* When k + W covers every page, sparse attention is plain causal attention over
  each row's prefix: it must equal torch's scaled_dot_product_attention in fp64.
* Closed forms: one visible token gives out = V_t; equal keys give the mean of V;
  an empty token set gives out = 0 and lse = -inf.
* The split/merge identity that the GPU path relies on: attention over a union of
  disjoint token sets equals the LSE-weighted merge of the parts.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth


def _small(**kw):
    base = synth.Config("small", 3, 2, 4, 2, 32, 16, 100, 2, 1, seed=11, invalid_frac=0.0)
    return synth.generate(base.with_(**kw))


def _dense_reference(w, selected):
    """numpy fp64: gather every visible token of the selection, then softmax."""
    c = w.cfg
    Hq, Hkv, d, P = c.q_heads, c.kv_heads, c.head_dim, c.page_size
    G = Hq // Hkv
    K = oracle.dequant_pages(w.k_codes, w.k_scales, c.k_global, np.arange(w.NP, dtype=np.int32))
    V = oracle.dequant_pages(w.v_codes, w.v_scales, c.v_global, np.arange(w.NP, dtype=np.int32))
    q = synth.f32_from_bf16_bits(w.q).astype(np.float64)
    out = np.zeros((w.N, Hq, d))
    lse = np.full((w.N, Hq), -np.inf)
    for b in range(w.B):
        r0, r1 = w.row_offsets[b], w.row_offsets[b + 1]
        R = r1 - r0
        for j in range(R):
            r = r0 + j
            L = max(0, int(w.seq_lens[b]) - (R - 1 - j))
            toks = []
            for p in sorted(set(int(x) for x in selected[r] if 0 <= x < w.MP)):
                phys = w.page_table[b, p]
                if phys < 0 or phys >= w.NP:
                    continue
                for t in range(P):
                    if p * P + t < L:
                        toks.append((phys, t))
            if not toks:
                continue
            for h in range(Hq):
                g = h // G
                Kt = np.stack([K[ph, g, t] for ph, t in toks])
                Vt = np.stack([V[ph, g, t] for ph, t in toks])
                logits = w.sm_scale * (Kt @ q[r, h])
                lse[r, h] = scipy.special.logsumexp(logits)
                pr = np.exp(logits - lse[r, h])
                out[r, h] = pr @ Vt
    return out, lse


@pytest.mark.parametrize("kw", [dict(), dict(invalid_frac=0.2, seed=12), dict(rows=4, context=(40, 130), seed=13),
                                dict(rows=24, context=(40, 160), seed=19),                 # a context step
                                dict(rows=(1, 20), context=(10, 160), seed=20, invalid_frac=0.1)])   # mixed
def test_attention_matches_dense_bruteforce(kw):
    w = _small(**kw)
    sel = oracle.select_w(w, oracle.index_scores(w))
    out, lse = oracle.attention(w, sel)
    ref_out, ref_lse = _dense_reference(w, sel)
    assert np.allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], ref_lse[fin], rtol=1e-12, atol=1e-12)


def test_attention_full_window_is_causal_sdpa():
    """k + W >= pages: every row attends to its whole causal prefix."""
    w = _small(rows=4, topk=64, context=(20, 120), seed=21)
    sel = oracle.select_w(w, oracle.index_scores(w))
    out, lse = oracle.attention(w, sel)
    c = w.cfg
    G = c.q_heads // c.kv_heads
    K = oracle.dequant_pages(w.k_codes, w.k_scales, 1.0, np.arange(w.NP, dtype=np.int32))
    V = oracle.dequant_pages(w.v_codes, w.v_scales, 1.0, np.arange(w.NP, dtype=np.int32))
    q = synth.f32_from_bf16_bits(w.q).astype(np.float64)
    for b in range(w.B):
        L_b = int(w.seq_lens[b])
        n = -(-L_b // c.page_size)
        phys = w.page_table[b, :n]
        Kseq = K[phys].transpose(1, 0, 2, 3).reshape(c.kv_heads, n * c.page_size, c.head_dim)[:, :L_b]
        Vseq = V[phys].transpose(1, 0, 2, 3).reshape(c.kv_heads, n * c.page_size, c.head_dim)[:, :L_b]
        R = c.rows
        Q = torch.from_numpy(q[b * R:(b + 1) * R]).permute(1, 0, 2)           # [Hq][R][d]
        Kt = torch.from_numpy(Kseq).repeat_interleave(G, 0)                  # [Hq][L][d]
        Vt = torch.from_numpy(Vseq).repeat_interleave(G, 0)
        # row j sees tokens < L_b - (R-1-j): a causal mask aligned to the end
        mask = torch.ones(R, L_b, dtype=torch.bool).tril(diagonal=L_b - R)
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, Kt, Vt, attn_mask=mask, scale=w.sm_scale).permute(1, 0, 2).numpy()
        assert np.allclose(out[b * R:(b + 1) * R], ref, rtol=1e-10, atol=1e-12)


def test_attention_single_token_is_v():
    w = _small(batch=1, rows=1, context=1, seed=31)
    sel = oracle.select_w(w, oracle.index_scores(w))
    out, lse = oracle.attention(w, sel)
    V = oracle.dequant_pages(w.v_codes, w.v_scales, 1.0, np.array([w.page_table[0, 0]], np.int32))
    G = w.cfg.q_heads // w.cfg.kv_heads
    for h in range(w.cfg.q_heads):
        assert np.array_equal(out[0, h], V[0, h // G, 0])


def test_attention_equal_keys_give_mean_of_v():
    w = _small(batch=1, rows=1, context=40, seed=41)
    w.k_codes[:] = 0x22                       # every K element = 1.0 * scale
    w.k_scales[:] = 0x38
    sel = oracle.select_w(w, oracle.index_scores(w))
    out, lse = oracle.attention(w, sel)
    c = w.cfg
    V = oracle.dequant_pages(w.v_codes, w.v_scales, 1.0, np.arange(w.NP, dtype=np.int32))
    toks = [(w.page_table[0, p], t) for p in sel[0] if p >= 0 for t in range(c.page_size)
            if p * c.page_size + t < 40]
    G = c.q_heads // c.kv_heads
    for h in range(c.q_heads):
        mean = np.mean([V[ph, h // G, t] for ph, t in toks], axis=0)
        assert np.allclose(out[0, h], mean, rtol=1e-13, atol=1e-14)
        logit = w.sm_scale * float(synth.f32_from_bf16_bits(w.q[0, h]).astype(np.float64).sum())
        assert math.isclose(lse[0, h], logit + math.log(len(toks)), rel_tol=1e-13, abs_tol=1e-13)


def test_attention_empty_and_invalid():
    w = _small(batch=2, rows=1, seed=51)
    sel = np.full((w.N, 3), -1, np.int32)
    sel[1, 0] = 0
    w.page_table[1, 0] = -1                    # the only listed page is invalid
    out, lse = oracle.attention(w, sel)
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_attention_duplicate_listing_counts_once():
    w = _small(batch=1, rows=1, seed=61)
    sel = oracle.select_w(w, oracle.index_scores(w))
    dup = np.concatenate([sel, sel], axis=1)
    a, la = oracle.attention(w, sel)
    b, lb = oracle.attention(w, dup)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_lse_merge_of_disjoint_parts():
    """out over A u B == (e^{lse_A} out_A + e^{lse_B} out_B) / (e^{lse_A} + e^{lse_B})."""
    w = _small(batch=2, rows=2, topk=4, seed=71)
    sel = oracle.select_w(w, oracle.index_scores(w))
    A = np.where(np.arange(sel.shape[1]) % 2 == 0, sel, -1).astype(np.int32)
    Bp = np.where(np.arange(sel.shape[1]) % 2 == 1, sel, -1).astype(np.int32)
    o, l = oracle.attention(w, sel)
    oa, la = oracle.attention(w, A)
    ob, lb = oracle.attention(w, Bp)
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m)[..., None], np.exp(lb - m)[..., None]
    merged = (wa * oa + wb * ob) / (wa + wb)
    assert np.allclose(merged, o, rtol=1e-12, atol=1e-13)
    assert np.allclose(m + np.log(np.exp(la - m) + np.exp(lb - m)), l, rtol=1e-12, atol=1e-12)


def test_attention_one_matches_full():
    w = _small(rows=4, context=(40, 130), invalid_frac=0.1, seed=81)
    sel = oracle.select_w(w, oracle.index_scores(w))
    out, lse = oracle.attention(w, sel)
    for r in range(w.N):
        for h in (0, w.cfg.q_heads - 1):
            o1, l1 = oracle.attention_one(w, sel, r, h)
            assert np.array_equal(o1, out[r, h]) and l1 == lse[r, h]


# ---- FP8 KV cache (unit scales) and the gated epilogue ---------------------------------

_E4M3_TABLE = np.array([oracle.e4m3(b) for b in range(256)])


def _dense_fp8(w, selected):
    """As _dense_reference, with K and V decoded as one E4M3FN byte per element."""
    c = w.cfg
    K = _E4M3_TABLE[w.k_codes] * c.k_global
    V = _E4M3_TABLE[w.v_codes] * c.v_global
    Hq, Hkv, P = c.q_heads, c.kv_heads, c.page_size
    G = Hq // Hkv
    q = synth.f32_from_bf16_bits(w.q).astype(np.float64)
    out = np.zeros((w.N, Hq, c.head_dim))
    lse = np.full((w.N, Hq), -np.inf)
    for b in range(w.B):
        r0, r1 = w.row_offsets[b], w.row_offsets[b + 1]
        for j in range(r1 - r0):
            r = r0 + j
            L = max(0, int(w.seq_lens[b]) - (r1 - r0 - 1 - j))
            toks = [(w.page_table[b, p], t) for p in sorted(set(int(x) for x in selected[r] if 0 <= x < w.MP))
                    if 0 <= w.page_table[b, p] < w.NP for t in range(P) if p * P + t < L]
            for h in range(Hq if toks else 0):
                Kt = np.stack([K[ph, h // G, t] for ph, t in toks])
                Vt = np.stack([V[ph, h // G, t] for ph, t in toks])
                logits = w.sm_scale * (Kt @ q[r, h])
                lse[r, h] = scipy.special.logsumexp(logits)
                out[r, h] = np.exp(logits - lse[r, h]) @ Vt
    return out, lse


@pytest.mark.parametrize("kw", [dict(kv_format="fp8"), dict(kv_format="fp8", invalid_frac=0.2, seed=14, v_global=0.5),
                                dict(kv_format="fp8", rows=4, context=(40, 130), seed=15)])
def test_fp8_attention_matches_dense_bruteforce(kw):
    w = _small(**kw)
    assert w.k_codes.shape[-1] == w.cfg.head_dim and w.k_scales.shape[-1] == 0
    sel = oracle.select_w(w, oracle.index_scores(w))
    out, lse = oracle.attention(w, sel)
    ref_out, ref_lse = _dense_fp8(w, sel)
    assert np.allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)) and np.allclose(lse[fin], ref_lse[fin], rtol=1e-12, atol=1e-12)


def test_fp8_element_indexing():
    """oracle_fp8_elem reads byte [page][h][t][i] of the [NP][Hkv][P][d] plane."""
    w = _small(kv_format="fp8", seed=16)
    c = w.cfg
    rng = np.random.default_rng(0)
    codes = np.ascontiguousarray(w.k_codes)
    for _ in range(200):
        pg, h, t, i = (int(rng.integers(n)) for n in codes.shape)
        got = oracle.lib().oracle_fp8_elem(codes.ctypes.data_as(oracle._P), 2.0, c.kv_heads, c.page_size,
                                           c.head_dim, pg, h, t, i)
        assert got == 2.0 * _E4M3_TABLE[codes[pg, h, t, i]]


def test_fp8_encoder_is_nearest():
    """The generator's FP8 bytes decode to the nearest E4M3FN value (the recipe's stated rounding)."""
    x = np.random.default_rng(1).standard_normal(20000).astype(np.float32) * 3
    codes = synth.encode_fp8(x)
    dec = _E4M3_TABLE[codes]
    grid = np.concatenate([-synth.E4M3_POS_VALUES[::-1], synth.E4M3_POS_VALUES])
    best = np.abs(grid[None, :] - x[:, None].astype(np.float64)).min(axis=1)
    assert np.all(np.abs(dec - x) == best)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_gate_multiplies_by_sigmoid(fmt):
    w = _small(kv_format=fmt, rows=4, context=(40, 130), seed=17)
    sel = oracle.select_w(w, oracle.index_scores(w))
    out, lse = oracle.attention(w, sel)
    g = synth.bf16_bits_from_f32(np.random.default_rng(2).standard_normal(w.q.shape).astype(np.float32) * 3)
    gout, glse = oracle.attention(w, sel, gate=g)
    sig = scipy.special.expit(synth.f32_from_bf16_bits(g).astype(np.float64))
    assert np.allclose(gout, out * sig, rtol=1e-14, atol=0)
    assert np.array_equal(np.isfinite(glse), np.isfinite(lse))
    assert np.array_equal(glse[np.isfinite(lse)], lse[np.isfinite(lse)])
    # gate 0 halves the output exactly; a large gate leaves it unchanged
    half, _ = oracle.attention(w, sel, gate=np.zeros_like(g))
    assert np.array_equal(half, out * 0.5)
    big = synth.bf16_bits_from_f32(np.full(w.q.shape, 64.0, np.float32))
    same, _ = oracle.attention(w, sel, gate=big)
    assert np.array_equal(same, out)
    for r in range(w.N):
        o1, _ = oracle.attention_one(w, sel, r, 1, gate=g)
        assert np.array_equal(o1, gout[r, 1])
