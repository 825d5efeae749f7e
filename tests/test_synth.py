"""The seeded generator: shapes of the five workloads, determinism, structure."""
import numpy as np
import pytest

import synth


def test_tiny_and_decode_shapes():
    w = synth.generate("tiny")
    assert (w.N, w.NP, w.MP) == (1, 16, 16)
    assert np.array_equal(w.page_table[0], np.arange(16))           # identity table
    assert w.k_codes.shape == (16, 1, 64, 32) and w.k_scales.shape == (16, 1, 64, 4)
    assert w.index_keys.shape == (16, 1, 64) and w.q.shape == (1, 4, 64)
    w = synth.generate("decode_8k")
    assert (w.N, w.NP, w.MP) == (8, 1024, 128)
    assert sorted(w.page_table.reshape(-1).tolist()) == list(range(1024))   # a permutation


def test_deterministic_and_thread_count_invariant():
    a = synth.generate("decode_8k")
    b = synth.generate("decode_8k", threads=1)
    assert a.digest() == b.digest()


def test_verify_workload_structure():
    w = synth.generate("mtp_verify_32k")
    assert (w.N, w.max_rows, w.NP, w.MP) == (64, 4, 8192, 512)
    # copied keys: some pages share a bit-identical index key with another page of the request
    dup = 0
    for b in range(w.B):
        keys = w.index_keys[w.page_table[b]].reshape(512, -1)
        _, counts = np.unique(keys, axis=0, return_counts=True)
        dup += int((counts > 1).sum())
    assert dup >= w.B


@pytest.mark.slow
def test_wide_mixed_structure():
    w = synth.generate("wide_mixed")
    n = (w.seq_lens.astype(np.int64) + 63) // 64
    assert w.seq_lens.min() >= 1024 and w.seq_lens.max() <= 65536
    holes = sum(int((w.page_table[b, :n[b]] < 0).sum()) for b in range(w.B))
    assert holes == sum(int(round(0.05 * x)) for x in n)
    assert w.NP == int(n.sum()) and w.N == 192


def test_tail_tokens_are_zero():
    w = synth.generate(synth.CONFIGS["decode_8k"].with_(batch=2, context=100))
    last = w.page_table[0, 1]                     # page 1 holds tokens 64..99
    assert np.all(w.k_codes[last, :, 36:] == 0) and np.all(w.k_scales[last, :, 36:] == 0)
    assert np.any(w.k_codes[last, :, :36] != 0)
