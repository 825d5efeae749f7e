"""Pins for the oracle's format decoders and dequantisation (CPU only).

What pins them:
* hand tables from the OCP format specs (tests/golden/e2m1_values.txt, e4m3_spot.txt);
* every E4M3 code decoded by torch's float8_e4m3fn (a library routine);
* every bf16 pattern decoded by torch.bfloat16;
* a hand-worked page (tests/golden/dequant_page.txt);
* the pages' KV byte counts, which fix the NVFP4 cost at 9/16 byte per element.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import read_golden


def test_e2m1_table():
    rows = read_golden("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1(int(code, 16))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_e4m3_spot_values():
    for byte, val in read_golden("e4m3_spot.txt"):
        got = oracle.e4m3(int(byte, 16))
        if val == "nan":
            assert math.isnan(got), byte
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), byte


def test_e4m3_all_codes_match_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        got = oracle.e4m3(b)
        if math.isnan(ref[b]):
            assert math.isnan(got), hex(b)
        else:
            assert got == ref[b] and math.copysign(1, got) == math.copysign(1, ref[b]), hex(b)


def test_e4m3_nan_only_at_7f_ff_and_monotone():
    vals = [oracle.e4m3(b) for b in range(256)]
    nans = [b for b in range(256) if math.isnan(vals[b])]
    assert nans == [0x7F, 0xFF]
    pos = vals[:0x7F]
    assert all(pos[i] < pos[i + 1] for i in range(len(pos) - 1))
    assert max(pos) == 448.0
    assert all(vals[0x80 + i] == -vals[i] for i in range(0x7F))


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    sample = list(range(0, 65536, 97)) + [0x0000, 0x8000, 0x3F80, 0x7F7F, 0x0001, 0xFF80]
    for b in sample:
        got = oracle.bf16(b)
        if math.isnan(ref[b]):
            assert math.isnan(got)
        else:
            assert got == ref[b], hex(b)


def _page_from_fixture():
    rows = read_golden("dequant_page.txt")
    shape = [r for r in rows if r[0] == "shape"][0]
    Hkv, P, d = map(int, shape[1:])
    codes = np.zeros((1, Hkv, P, d // 2), np.uint8)
    scales = np.zeros((1, Hkv, P, d // 16), np.uint8)
    for r in rows:
        if r[0] == "code":
            codes[0, int(r[1]), int(r[2]), int(r[3])] = int(r[4], 16)
        elif r[0] == "scale":
            scales[0, int(r[1]), int(r[2]), int(r[3])] = int(r[4], 16)
    expects = [(float(r[1]), int(r[2]), int(r[3]), int(r[4]), float(r[5])) for r in rows if r[0] == "expect"]
    return codes, scales, expects


def test_dequant_hand_worked_page():
    codes, scales, expects = _page_from_fixture()
    for g in sorted({e[0] for e in expects}):
        out = oracle.dequant_pages(codes, scales, g, np.array([0], np.int32))
        for gg, h, t, i, want in expects:
            if gg == g:
                assert out[0, h, t, i] == want, (g, h, t, i, out[0, h, t, i], want)


def test_dequant_is_exact_product_of_element_and_block_scale():
    """Every (code, scale) pair: the value is e2m1(code) * e4m3(scale); block index = i // 16."""
    Hkv, P, d = 1, 256, 32
    codes = np.zeros((1, Hkv, P, d // 2), np.uint8)
    scales = np.zeros((1, Hkv, P, d // 16), np.uint8)
    t = np.arange(P)
    codes[0, 0, :, :] = t[:, None].astype(np.uint8)           # byte t in every position of token t
    scales[0, 0, :, 0] = t.astype(np.uint8)                    # block 0 scale = byte t
    scales[0, 0, :, 1] = 0x38                                  # block 1 scale = 1.0
    out = oracle.dequant_pages(codes, scales, 1.0, np.array([0], np.int32))[0, 0]
    e2m1 = [float(r[1]) for r in read_golden("e2m1_values.txt")]
    e4m3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for tok in range(P):
        lo, hi = tok & 0xF, tok >> 4
        for i in range(d):
            code = lo if i % 2 == 0 else hi
            s = e4m3[tok] if i < 16 else 1.0
            want = e2m1[code] * s
            got = out[tok, i]
            if math.isnan(want):
                assert math.isnan(got)
            else:
                assert got == want, (tok, i, got, want)


def test_nvfp4_bytes_per_element_matches_pages():
    """bf16 : FP8 : NVFP4 = 29976 : 16664 : 10840 bytes per token.

    With a per-token remainder r that does not depend on the format:
    bf16 - fp8 = E bytes (E elements at 2 vs 1 byte), fp8 - nvfp4 = E (1 - c).
    So c = 1 - (fp8 - nvfp4) / (bf16 - fp8), and it must equal this layout's
    (d/2 + d/16) / d = 9/16.
    """
    v = {r[0]: int(r[1]) for r in read_golden("kv_bytes_per_token.txt")}
    E = v["bf16"] - v["fp8"]
    c = 1.0 - (v["fp8"] - v["nvfp4"]) / E
    w = synth.generate("tiny")
    d = w.cfg.head_dim
    per_token_per_head = w.k_codes.shape[-1] + w.k_scales.shape[-1]
    assert c == per_token_per_head / d == 9 / 16
    # and the remainder is the same for all three formats
    r_bf16 = v["bf16"] - 2 * E
    r_fp8 = v["fp8"] - E
    r_nv = v["nvfp4"] - E * 9 // 16
    assert r_bf16 == r_fp8 == r_nv


def test_encoder_round_trip_within_half_step():
    """The generator's encoder, read back by the oracle: |x - deq| <= half a grid step."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 2, 8, 32)).astype(np.float32)
    x[0, 0, 0, :16] = 0.0                       # an all-zero block
    x[1, 1, 3, 5] = 40.0                         # a large element sets its block's scale
    codes, scales = synth.encode_nvfp4(x)
    deq = oracle.dequant_pages(codes, scales, 1.0, np.arange(3, dtype=np.int32))
    for idx in np.ndindex(x.shape[:-1]):
        for blk in range(2):
            s = oracle.e4m3(int(scales[idx][blk]))
            seg = slice(16 * blk, 16 * blk + 16)
            err = np.abs(x[idx][seg].astype(np.float64) - deq[idx][seg])
            amax = np.abs(x[idx][seg]).max()
            if amax == 0:
                assert s == 0.0 and np.all(deq[idx][seg] == 0)
                continue
            # half the widest e2m1 gap (4 -> 6) times the scale, plus saturation slack
            bound = 1.0 * s + max(0.0, amax - 6 * s)
            assert np.all(err <= bound + 1e-12), (idx, blk)


def test_encoder_midpoint_ties():
    """E2M1 RNE at the midpoints: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    x = np.zeros((1, 16), np.float32)
    x[0, :7] = mids
    x[0, 15] = 6.0                               # amax 6 -> scale 1.0 exactly
    codes, scales = synth.encode_nvfp4(x)
    assert scales[0, 0] == 0x38
    deq = oracle.dequant_pages(codes.reshape(1, 1, 1, 8), scales.reshape(1, 1, 1, 1), 1.0,
                               np.array([0], np.int32))[0, 0, 0]
    assert list(deq[:7]) == want
    assert deq[15] == 6.0
