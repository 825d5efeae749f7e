"""Pins of the oracle's KV store (the step before the decode path): the NVFP4 encoder and the
index-key recomputation, checked against torch's float8 conversion, the stated rounding
midpoints, exactly representable blocks and an fp64 mean of the stored page.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_encode_matches_torch_float8_rounding():
    """Nearest code, ties to even, for values up to the 448/480 midpoint (torch gives NaN above)."""
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        np.float32(2.0) ** rng.uniform(-12, 8.85, 20000).astype(np.float32),
        np.array([oracle.e4m3(c) for c in range(127)], np.float32),                     # grid points
        np.array([(oracle.e4m3(c) + oracle.e4m3(c + 1)) / 2 for c in range(126)], np.float32),  # midpoints
        np.array([0.0, 2.0 ** -10, 463.99, 447.9], np.float32),
    ]).astype(np.float32)
    vals = vals[vals < 464.0]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(v) for v in vals], np.uint8)
    assert np.array_equal(got, ref)
    assert oracle.e4m3_encode(464.0) == 0x7E and oracle.e4m3_encode(1e6) == 0x7E      # saturates


@pytest.mark.parametrize("y,code", [
    (0.0, 0), (0.25, 0), (0.2500001, 1), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
    (6.0, 7), (100.0, 7), (0.5, 1), (1.5, 3), (3.0, 5), (4.0, 6), (-0.75, 10), (-6.5, 15), (-0.1, 0)])
def test_e2m1_encode_midpoints(y, code):
    """The midpoints of the E2M1 grid go to the even code; beyond 6 saturates; tiny values give +0."""
    assert oracle.e2m1_encode(y) == code


def test_e2m1_encode_is_nearest():
    rng = np.random.default_rng(6)
    for y in rng.uniform(-8, 8, 4000).astype(np.float32):
        c = oracle.e2m1_encode(float(y))
        v = E2M1[c & 7] * (-1 if c & 8 else 1)
        a = min(abs(float(y)), 6.0)
        assert abs(abs(v) - a) <= min(abs(g - a) for g in E2M1) + 1e-12


def _dec_block(codes, sc, g=1.0):
    vals = []
    for byte in codes:
        for c in (byte & 0xF, byte >> 4):
            vals.append(oracle.e2m1(c) * oracle.e4m3(sc) * g)
    return np.array(vals)


def test_encode_block_exact_when_representable():
    """A block of E2M1 values times an E4M3-representable power of two with amax = 6 * scale is
    reproduced exactly."""
    rng = np.random.default_rng(7)
    for s in (1.0, 0.25, 8.0, 2.0 ** -6):
        x = np.array([E2M1[i] for i in rng.integers(0, 8, 16)]) * rng.choice([-1, 1], 16)
        x[3] = 6.0
        x = (x * s).astype(np.float32)
        codes, sc = oracle.nvfp4_encode_block(x)
        assert oracle.e4m3(sc) == s
        assert np.array_equal(_dec_block(codes, sc), x.astype(np.float64))


def test_encode_block_error_bound_and_zero_block():
    rng = np.random.default_rng(8)
    for g in (1.0, 0.5):
        for _ in range(300):
            x = (rng.standard_normal(16) * rng.uniform(0.01, 50)).astype(np.float32)
            codes, sc = oracle.nvfp4_encode_block(x, g)
            s = oracle.e4m3(sc) * g
            err = np.abs(_dec_block(codes, sc, g) - x)
            # each element is within half of the widest grid step (2 * s), or saturated at 6 s
            assert np.all((err <= s + 1e-6) | (np.abs(x) >= 6 * s))
    codes, sc = oracle.nvfp4_encode_block(np.zeros(16, np.float32))
    assert sc == 0 and not codes.any()


def _small(**kw):
    base = dict(name="kvs", batch=3, rows=3, q_heads=8, kv_heads=2, head_dim=64, page_size=64,
                context=(70, 900), topk=4, window=1, seed=91)
    base.update(kw)
    return synth.generate(synth.Config(**base))


def _new_tokens(w, rng, value=None):
    shape = (w.N, w.cfg.kv_heads, w.cfg.head_dim)
    x = np.full(shape, value, np.float32) if value is not None else rng.standard_normal(shape).astype(np.float32)
    return synth.bf16_bits_from_f32(x)


def test_kv_store_writes_the_new_tokens_in_place():
    """Row j of a request lands at position L - R + j; every other slot is unchanged."""
    w = _small()
    rng = np.random.default_rng(1)
    nk, nv = _new_tokens(w, rng), _new_tokens(w, rng)
    kc, ks, vc, vs, keys = oracle.kv_store(w, nk, nv)
    c = w.cfg
    P, Hkv, d = c.page_size, c.kv_heads, c.head_dim
    written = np.zeros((w.NP, Hkv, P), bool)
    for b in range(w.B):
        r0, R = int(w.row_offsets[b]), int(w.row_offsets[b + 1] - w.row_offsets[b])
        L = int(w.seq_lens[b])
        for j in range(R):
            pos = L - R + j
            phys = int(w.page_table[b, pos // P])
            for h in range(Hkv):
                for blk in range(d // 16):
                    x = synth.f32_from_bf16_bits(nk[r0 + j, h, blk * 16:(blk + 1) * 16])
                    codes, sc = oracle.nvfp4_encode_block(x)
                    assert np.array_equal(kc[phys, h, pos % P, blk * 8:(blk + 1) * 8], codes)
                    assert ks[phys, h, pos % P, blk] == sc
            written[phys, :, pos % P] = True
    assert np.array_equal(kc[~written], w.k_codes[~written])
    assert np.array_equal(vs[~written], w.v_scales[~written])


def test_kv_store_index_key_is_the_page_mean():
    """The recomputed key of a touched page is the bf16 mean of its stored K over its valid
    tokens (checked against an fp64 mean of the dequantised page); other keys are unchanged."""
    w = _small(seed=92)
    rng = np.random.default_rng(2)
    nk, nv = _new_tokens(w, rng), _new_tokens(w, rng)
    kc, ks, vc, vs, keys = oracle.kv_store(w, nk, nv)
    c = w.cfg
    P = c.page_size
    touched = set()
    for b in range(w.B):
        R = int(w.row_offsets[b + 1] - w.row_offsets[b])
        L = int(w.seq_lens[b])
        for j in range(R):
            page = (L - R + j) // P
            phys = int(w.page_table[b, page])
            if phys in touched:
                continue
            touched.add(phys)
            n = min(P, L - page * P)
            dq = oracle.dequant_pages(kc, ks, 1.0, np.array([phys]))[0]        # [Hkv][P][d]
            mean = dq[:, :n, :].mean(axis=1)
            got = synth.f32_from_bf16_bits(keys[phys]).astype(np.float64)
            # bf16 rounding (2^-9 relative) plus an fp32 sum of n terms
            assert np.all(np.abs(got - mean) <= 2.0 ** -8 * np.abs(mean) + n * 2.0 ** -23 * np.abs(dq).max() + 1e-30)
    others = np.array([p for p in range(w.NP) if p not in touched])
    assert np.array_equal(keys[others], w.index_keys[others])


def test_kv_store_constant_tokens_and_invalid_pages():
    """Tokens of all 6.0 store exactly (scale 1, code 6), and a page whose tokens are all new
    and equal gets that value as its key; a token whose page entry is -1 is not stored."""
    w = _small(seed=93, rows=1, context=(64, 64))       # one new token per request, at slot 63
    w.page_table = w.page_table.copy()
    w.page_table[1, 0] = -1
    nk = _new_tokens(w, None, 6.0)
    kc, ks, vc, vs, keys = oracle.kv_store(w, nk, nk)
    phys0 = int(w.page_table[0, 0])
    assert np.all(ks[phys0, :, 63] == 0x38) and np.all(kc[phys0, :, 63] == 0x77)
    assert np.array_equal(kc[:, :, :63], w.k_codes[:, :, :63])
    # the store into request 1 is skipped: no plane changes outside requests 0 and 2
    phys2 = int(w.page_table[2, 0])
    mask = np.ones(w.NP, bool)
    mask[[phys0, phys2]] = False
    assert np.array_equal(kc[mask], w.k_codes[mask]) and np.array_equal(keys[mask], w.index_keys[mask])
    # a page filled only by the store: one request with one row and L = 1
    w1 = _small(seed=94, batch=1, rows=1, context=(1, 1))
    kc, ks, vc, vs, keys = oracle.kv_store(w1, _new_tokens(w1, None, 6.0), _new_tokens(w1, None, 6.0))
    phys = int(w1.page_table[0, 0])
    assert np.all(synth.f32_from_bf16_bits(keys[phys]) == 6.0)
