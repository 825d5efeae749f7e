"""qsa_select_sparse_decode_static (the entry point for callers that cannot allocate: its split
workspace is the library's own device array) against qsa_select_sparse_decode with a caller
workspace, through the C ABI: the same selection rows and the same outputs, bit for bit (the
same kernels at the same split count), and the oracle's attention within tolerance. Two calls
in a row, the second on a smaller batch with a different split count, so the second call runs
on what the first left in the array. A graph test captures the static call with the index scores
and replays it between eager calls of the program's own.
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


def _check(out_bits, lse, ref_out, ref_lse, where):
    out = synth.f32_from_bf16_bits(out_bits).astype(np.float64)
    err = np.abs(out - ref_out) - (ATOL + RTOL * np.abs(ref_out))
    assert err.max(initial=-1) <= 0, f"{where}: out beyond tolerance by {err.max()}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)), where
    if fin.any():
        assert np.abs(lse[fin] - ref_lse[fin]).max() <= LSE_TOL, where


def _static_vs_workspace(w, splits, where):
    b = DeviceBatch.upload(w)
    plan = q.qsa_plan_decode(b.shape(), splits, True)
    assert plan.splits > 1 and plan.workspace_bytes > 0, "the case must split its tiles"
    print(f"[no-alloc] {where} B={w.B} N={w.N} splits={plan.splits} ws={plan.workspace_bytes}", flush=True)
    ref = Step(b, num_splits=splits)           # qsa_index_scores + qsa_select_sparse_decode
    ref()
    sel = torch.full_like(ref.selected, -7)
    out = torch.full_like(ref.out, 0x1234)
    lse = torch.full_like(ref.lse, 3.0)
    q.qsa_select_sparse_decode_static(ref.shape_, ref.paged_, b.q, ref.scores, sel, out, lse, splits)
    torch.cuda.synchronize()
    assert torch.equal(sel, ref.selected), where
    assert torch.equal(out, ref.out), where
    assert torch.equal(lse, ref.lse), where
    ref_sel = oracle.select_w(w, oracle.index_scores(w))
    assert np.array_equal(sel.cpu().numpy(), ref_sel), where
    ref_out, ref_lse = oracle.attention(w, ref_sel)
    _check(out.cpu().numpy().view(np.uint16), lse.cpu().numpy(), ref_out, ref_lse, where)
    assert int(b.error_word[0].item()) == 0


def test_static_entry_point_two_calls_then_smaller():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    big = synth.generate(synth.Config("na_big", 6, 4, 16, 2, 128, 64, (300, 5000), 6, 2, seed=951,
                                      invalid_frac=0.1))
    small = synth.generate(synth.Config("na_small", 2, 3, 8, 2, 64, 64, (100, 2000), 4, 1, seed=952))
    _static_vs_workspace(big, 0, "first call")          # the library's split count
    _static_vs_workspace(small, 3, "second call, smaller")


def test_static_entry_point_refuses_oversize_and_runs_unsplit():
    """A split workspace beyond the array's 8 MiB is refused before any launch (nothing written);
    the same shape at one split needs no workspace and runs."""
    w = synth.generate(synth.Config("na_wide", 48, 4, 32, 4, 128, 64, (300, 3000), 6, 2, seed=953))
    b = DeviceBatch.upload(w)
    sh = b.shape()
    assert q.qsa_workspace_bytes(sh, 64) > (8 << 20)
    st = Step(b, num_splits=1)
    st.scores_call()
    out = torch.full_like(st.out, 0x1234)
    with pytest.raises(q.QsaError) as ei:
        q.qsa_select_sparse_decode_static(sh, st.paged_, b.q, st.scores, st.selected, out, st.lse, 64)
    assert ei.value.status == 3
    torch.cuda.synchronize()
    assert bool((out == 0x1234).all())
    st.select_decode_call()
    q.qsa_select_sparse_decode_static(sh, st.paged_, b.q, st.scores, st.selected, out, None, 1)
    torch.cuda.synchronize()
    assert torch.equal(out, st.out)


def test_static_entry_point_gated_split():
    """The gated epilogue through the static entry point at 2 splits equals the workspace call."""
    w = synth.generate(synth.Config("na_gate", 3, 4, 16, 2, 128, 64, (300, 4000), 5, 2, seed=954))
    b = DeviceBatch.upload(w)
    rng = np.random.default_rng(5)
    gate = torch.from_numpy(synth.bf16_bits_from_f32(rng.standard_normal(w.q.shape, dtype=np.float32)).view(
        np.int16)).cuda()
    ref = Step(b, num_splits=2, gate=gate)
    ref()
    out = torch.full_like(ref.out, 0x1234)
    q.qsa_select_sparse_decode_static(ref.shape_, ref.paged_, b.q, ref.scores, ref.selected, out, None, 2,
                                      gate=gate)
    torch.cuda.synchronize()
    assert torch.equal(out, ref.out)


def test_static_entry_point_in_a_graph():
    """The callers it is for include code under HIP graph capture: the index scores and the
    static call captured in one graph, replayed four times with eager work of the program's own
    (refilled outputs, another call of the static entry point on a different batch, which
    leaves its own contents in the array) and synchronisations between the replays. Every
    replay equals the eager step bit for bit; the counters are cleared inside the graph by a
    fill kernel, not a memset node."""
    w = synth.generate(synth.Config("na_graph", 5, 4, 16, 2, 128, 64, (300, 4000), 6, 2, seed=955,
                                    invalid_frac=0.1))
    other = synth.generate(synth.Config("na_other", 2, 2, 8, 2, 64, 64, (200, 2000), 4, 1, seed=956))
    b, bo = DeviceBatch.upload(w), DeviceBatch.upload(other)
    splits = 3
    st = Step(b, num_splits=splits)
    so = Step(bo, num_splits=2)
    sel = torch.full_like(st.selected, -7)
    out = torch.full_like(st.out, 0x1234)
    lse = torch.full_like(st.lse, 3.0)

    def step(stream):
        st.scores_call(stream)
        q.qsa_select_sparse_decode_static(st.shape_, st.paged_, b.q, st.scores, sel, out, lse, splits, stream)

    step(None)
    torch.cuda.synchronize()
    eager = (st.scores.clone(), sel.clone(), out.clone(), lse.clone())
    ref = Step(b, num_splits=splits)
    ref()
    torch.cuda.synchronize()
    assert torch.equal(out, ref.out) and torch.equal(lse, ref.lse) and torch.equal(sel, ref.selected)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for i in range(4):
        out.fill_(0x1234)
        sel.fill_(-7)
        lse.fill_(3.0)
        st.scores.fill_(1.0)
        so.scores_call()
        q.qsa_select_sparse_decode_static(so.shape_, so.paged_, bo.q, so.scores, so.selected, so.out, so.lse, 2)
        torch.cuda.synchronize()
        print(f"[no-alloc] graph replay {i}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.scores, eager[0]) and torch.equal(sel, eager[1]), f"replay {i}"
        assert torch.equal(out, eager[2]) and torch.equal(lse, eager[3]), f"replay {i}"
