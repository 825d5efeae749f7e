"""GPU parity of the attention variants against the oracle: the FP8 (unit-scale E4M3) K/V
format and the gated epilogue (out = o * sigmoid(gate)), through both attention entry points
and several split counts. Bars as in the base parity tests: selections bit-exact, outputs
within |gpu - ref| <= 2e-3 + 1e-2 |ref| of the fp64 oracle, lse within 2e-3.
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


def _gate(w, seed):
    g = np.random.default_rng(seed).standard_normal(w.q.shape).astype(np.float32) * 3.0
    bits = synth.bf16_bits_from_f32(g)
    return bits, torch.from_numpy(bits.view(np.int16)).cuda()


FP8_CASES = [
    synth.Config("f8_d128", 4, 4, 16, 2, 128, 64, (70, 3000), 6, 2, seed=701, kv_format="fp8"),
    synth.Config("f8_d64_p128", 3, 2, 8, 4, 64, 128, (130, 5000), 4, 1, seed=702, kv_format="fp8",
                 invalid_frac=0.1),
    synth.Config("f8_r1_g8", 5, 1, 32, 4, 128, 64, (1, 9000), 8, 2, seed=703, kv_format="fp8", v_global=0.5),
    synth.Config("f8_r3", 2, 3, 12, 4, 128, 64, (3, 1200), 3, 1, seed=704, kv_format="fp8", outlier_frac=0.01),
]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("cfg", FP8_CASES, ids=lambda c: c.name)
def test_fp8_attention_vs_oracle(cfg, splits, fused):
    w = synth.generate(cfg)
    print(f"[fp8] {cfg.name} splits={splits} fused={fused}", flush=True)
    b = DeviceBatch.upload(w)
    assert b.kv_format == q.QSA_KV_FP8
    st = Step(b, num_splits=splits, fused=fused)
    st()
    torch.cuda.synchronize()
    sel = st.selected.cpu().numpy()
    assert np.array_equal(sel, oracle.select_w(w, oracle.index_scores(w)))
    ref_out, ref_lse = oracle.attention(w, sel)
    _check(st.out, st.lse, ref_out, ref_lse, cfg.name)
    assert int(b.error_word[0].item()) == 0


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("splits", [0, 2])
@pytest.mark.parametrize("fused", [True, False])
def test_gated_epilogue_vs_oracle(fmt, splits, fused):
    cfg = synth.Config("gate", 4, 4, 16, 2, 128, 64, (70, 3000), 6, 2, seed=705, kv_format=fmt)
    w = synth.generate(cfg)
    print(f"[gate] {fmt} splits={splits} fused={fused}", flush=True)
    gbits, gdev = _gate(w, 11)
    b = DeviceBatch.upload(w)
    st = Step(b, num_splits=splits, fused=fused, gate=gdev)
    st()
    torch.cuda.synchronize()
    sel = st.selected.cpu().numpy()
    ref_out, ref_lse = oracle.attention(w, sel, gate=gbits)
    _check(st.out, st.lse, ref_out, ref_lse, f"gate {fmt}")
    # the same launch without the gate is the ungated attention
    ug = Step(b, num_splits=splits, fused=fused)
    ug()
    torch.cuda.synchronize()
    ref_u, _ = oracle.attention(w, sel)
    _check(ug.out, ug.lse, ref_u, ref_lse, f"ungated {fmt}")


def test_fp8_full_size_sampled():
    cfg = synth.CONFIGS["mtp_verify_32k"].with_(kv_format="fp8", name="mtp_verify_32k_fp8")
    w = synth.generate(cfg)
    print("[fp8 full] mtp_verify_32k", flush=True)
    gbits, gdev = _gate(w, 12)
    b = DeviceBatch.upload(w)
    st = Step(b, gate=gdev)
    st()
    torch.cuda.synchronize()
    sel = st.selected.cpu().numpy()
    out = synth.f32_from_bf16_bits(st.out.cpu().numpy().view(np.uint16)).astype(np.float64)
    lse = st.lse.cpu().numpy()
    assert int(b.error_word[0].item()) == 0
    rng = np.random.default_rng(8)
    Hq = w.cfg.q_heads
    pairs = {(0, 0), (w.N - 1, Hq - 1)} | {(int(r), int(h)) for r, h in
                                            zip(rng.integers(0, w.N, 20), rng.integers(0, Hq, 20))}
    for r, h in sorted(pairs):
        ref_o, ref_l = oracle.attention_one(w, sel, r, h, gate=gbits)
        assert np.all(np.abs(out[r, h] - ref_o) <= ATOL + RTOL * np.abs(ref_o)), (r, h)
        assert abs(lse[r, h] - ref_l) <= LSE_TOL
