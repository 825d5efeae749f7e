"""GPU attention on inputs with closed-form answers (isolate the QK, PV and merge paths).

* Equal keys: every logit ties, so the output is the mean of V over the visible tokens.
* One visible token (a one-token request): the output is that token's V.
* Constant V: the output is that constant whatever the weights.
Each case is also checked against the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from block_sparse_decode_amd.batch import DeviceBatch, Step

pytestmark = pytest.mark.gpu


def _run(w, splits=1):
    b = DeviceBatch.upload(w)
    st = Step(b, num_splits=splits)
    st()
    torch.cuda.synchronize()
    out = synth.f32_from_bf16_bits(st.out.cpu().numpy().view(np.uint16)).astype(np.float64)
    return out, st.lse.cpu().numpy(), st.selected.cpu().numpy()


def _base(**kw):
    cfg = synth.Config("cf", 2, 1, 8, 2, 128, 64, 256, 2, 1, seed=401).with_(**kw)
    return synth.generate(cfg)


def _report(name, out, ref):
    err = np.abs(out - ref)
    print(f"[{name}] max abs err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}", flush=True)
    return err


@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("d", [64, 128])
def test_equal_keys_give_mean_of_v(d, splits):
    w = _base(head_dim=d)
    w = dataclasses.replace(w, k_codes=np.full_like(w.k_codes, 0x22), k_scales=np.full_like(w.k_scales, 0x38))
    out, lse, sel = _run(w, splits)
    ref, ref_lse = oracle.attention(w, sel)
    err = _report(f"equal-keys d{d} s{splits}", out, ref)
    assert np.all(err <= 2e-3 + 1e-2 * np.abs(ref))


@pytest.mark.parametrize("d", [64, 128])
def test_single_token_gives_v(d):
    w = _base(head_dim=d, context=1, batch=3)
    out, lse, sel = _run(w)
    ref, _ = oracle.attention(w, sel)
    err = _report(f"single-token d{d}", out, ref)
    assert np.all(err <= 2e-3 + 1e-2 * np.abs(ref))


@pytest.mark.parametrize("d", [64, 128])
def test_constant_v(d):
    w = _base(head_dim=d)
    w = dataclasses.replace(w, v_codes=np.full_like(w.v_codes, 0x22), v_scales=np.full_like(w.v_scales, 0x40))
    out, lse, sel = _run(w)
    ref, ref_lse = oracle.attention(w, sel)
    err = _report(f"constant-v d{d}", out, ref)
    assert np.all(err <= 2e-3 + 1e-2 * np.abs(ref))
    assert np.all(np.abs(lse - ref_lse) <= 2e-3)


@pytest.mark.parametrize("d", [64, 128])
def test_one_hot_v_columns(d):
    """V[t][i] nonzero only at i = t mod d: each output column isolates one token's weight."""
    w = _base(head_dim=d, context=64, batch=1)
    vc = np.zeros_like(w.v_codes)
    vs = np.full_like(w.v_scales, 0x38)
    P = w.cfg.page_size
    for t in range(P):
        i = t % d
        vc[:, :, t, i // 2] |= np.uint8(0x2 << (4 * (i % 2)))       # value 1.0 at column i
    w = dataclasses.replace(w, v_codes=vc, v_scales=vs)
    out, lse, sel = _run(w)
    ref, _ = oracle.attention(w, sel)
    err = _report(f"one-hot-v d{d}", out, ref)
    assert np.all(err <= 2e-3 + 1e-2 * np.abs(ref))
