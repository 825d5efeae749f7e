"""GPU parity of qsa_kv_store (the KV-store prologue: NVFP4 quantisation of the step's new
tokens and the index keys of the pages they land in) against the oracle, bit for bit, on
every plane; and the decode path run on the updated cache.
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

PLANES = ("k_codes", "k_scales", "v_codes", "v_scales", "index_keys")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    yield


def _tokens(w, rng, scale=1.0):
    x = (rng.standard_normal((w.N, w.cfg.kv_heads, w.cfg.head_dim)) * scale).astype(np.float32)
    return synth.bf16_bits_from_f32(x)


def _store_gpu(w, nk, nv):
    b = DeviceBatch.upload(w)
    nk_d = torch.from_numpy(nk.view(np.int16)).cuda()
    nv_d = torch.from_numpy(nv.view(np.int16)).cuda()
    q.qsa_kv_store(b.shape(), b.paged(), nk_d, nv_d)
    torch.cuda.synchronize()
    got = {}
    for name in PLANES:
        t = getattr(b, name).cpu().numpy()
        got[name] = t.view(np.uint16) if name == "index_keys" else t
    return b, got


def _check(w, nk, nv):
    b, got = _store_gpu(w, nk, nv)
    ref = dict(zip(PLANES, oracle.kv_store(w, nk, nv)))
    for name in PLANES:
        assert np.array_equal(got[name], ref[name]), name
    return b


STORE_CASES = [
    synth.Config("st_d128_p64", 4, 4, 16, 2, 128, 64, (70, 3000), 6, 2, seed=501),
    synth.Config("st_d64_p128", 3, 2, 8, 4, 64, 128, (130, 5000), 4, 1, seed=502, invalid_frac=0.1),
    synth.Config("st_r1", 5, 1, 32, 4, 128, 64, (1, 9000), 8, 2, seed=503),
    synth.Config("st_r3_g1", 2, 3, 4, 4, 64, 64, (3, 700), 3, 1, seed=504, k_global=0.5, v_global=2.0),
]


@pytest.mark.parametrize("cfg", STORE_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("scale", [1.0, 1e-3, 300.0])
def test_kv_store_bitwise(cfg, scale):
    w = synth.generate(cfg)
    print(f"[kv store] {cfg.name} scale={scale}", flush=True)
    rng = np.random.default_rng(int(scale * 1000) + cfg.seed)
    b = _check(w, _tokens(w, rng, scale), _tokens(w, rng, scale))
    assert int(b.error_word[0].item()) == 0


def test_kv_store_rounding_ties():
    """Blocks of amax 6 (scale 1.0) made of the E2M1 midpoints, and blocks whose amax / 6 is
    the midpoint of two E4M3 codes: ties go to the even code on both sides."""
    cfg = synth.Config("st_ties", 2, 2, 4, 2, 64, 64, (100, 300), 4, 1, seed=505)
    w = synth.generate(cfg)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0,
                     -6.0], np.float32)
    nk = np.tile(mids, (w.N, cfg.kv_heads, cfg.head_dim // 16))
    nv = nk.copy()
    nv[..., ::16] = 6.375          # amax / 6 = 1.0625, halfway between 1.0 and 1.125
    _check(w, synth.bf16_bits_from_f32(nk), synth.bf16_bits_from_f32(nv))


def test_kv_store_full_size():
    w = synth.generate("mtp_verify_32k")
    rng = np.random.default_rng(11)
    print("[kv store] mtp_verify_32k", flush=True)
    b = _check(w, _tokens(w, rng), _tokens(w, rng))
    assert int(b.error_word[0].item()) == 0


def test_kv_store_bad_page_ids_and_short_requests():
    cfg = synth.Config("st_bad", 3, 2, 8, 2, 64, 64, (200, 600), 4, 1, seed=506)
    w = synth.generate(cfg)
    w.page_table = w.page_table.copy()
    w.seq_lens = w.seq_lens.copy()
    L0 = int(w.seq_lens[0])
    w.page_table[0, (L0 - 1) // 64] = -1            # the last page of request 0: skipped silently
    L1 = int(w.seq_lens[1])
    w.page_table[1, (L1 - 1) // 64] = w.NP + 5      # out of range: skipped and reported
    w.seq_lens[2] = 1                               # 2 rows but 1 token: reported
    rng = np.random.default_rng(12)
    nk, nv = _tokens(w, rng), _tokens(w, rng)
    b, got = _store_gpu(w, nk, nv)
    err = int(b.error_word[0].item())
    assert err & q.QSA_DEVERR_PAGE_ID and err & q.QSA_DEVERR_SEQ_LEN
    # requests 0 and 1: only their valid slots changed, as in the oracle with the bad entry as -1
    w2 = dataclasses.replace(w)
    w2.page_table = w.page_table.copy()
    w2.page_table[1, (L1 - 1) // 64] = -1
    ref = dict(zip(PLANES, oracle.kv_store(w2, nk, nv)))
    for name in PLANES:
        assert np.array_equal(got[name], ref[name]), name


def test_store_then_step_matches_oracle():
    """The decode path on the cache the store just updated: scores and rows bit for bit,
    attention within the tolerance of the parity tests."""
    cfg = synth.Config("st_step", 4, 4, 16, 2, 128, 64, (200, 4000), 6, 2, seed=507)
    w = synth.generate(cfg)
    rng = np.random.default_rng(13)
    nk, nv = _tokens(w, rng), _tokens(w, rng)
    b = DeviceBatch.upload(w)
    q.qsa_kv_store(b.shape(), b.paged(), torch.from_numpy(nk.view(np.int16)).cuda(),
                   torch.from_numpy(nv.view(np.int16)).cuda())
    st = Step(b)
    st()
    torch.cuda.synchronize()
    planes = oracle.kv_store(w, nk, nv)
    w_new = dataclasses.replace(w, k_codes=planes[0], k_scales=planes[1], v_codes=planes[2], v_scales=planes[3],
                                index_keys=planes[4])
    ref_s = oracle.index_scores(w_new)
    assert np.array_equal(st.scores.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    sel = oracle.select_w(w_new, ref_s)
    assert np.array_equal(st.selected.cpu().numpy(), sel)
    ref_o, ref_l = oracle.attention(w_new, sel)
    out = synth.f32_from_bf16_bits(st.out.cpu().numpy().view(np.uint16)).astype(np.float64)
    assert np.all(np.abs(out - ref_o) <= 2e-3 + 1e-2 * np.abs(ref_o))
    lse = st.lse.cpu().numpy()
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(np.abs(lse[fin] - ref_l[fin]) <= 2e-3)
    assert int(b.error_word[0].item()) == 0
