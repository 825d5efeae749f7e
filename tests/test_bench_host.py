"""Host-side logic of bench.py, without a GPU: the algorithmic byte count against a hand count,
the counter-to-bytes scaling of the traffic record, the code-only source hash, and the kernel
name the traffic lookup searches for against the launch plan the library reports.
"""
import csv
import math
import types

import numpy as np
import pytest

import bench


def _mini():
    """Two requests of two rows, 4 KV heads, d 128, pages of 64, MP 6; request 1's page 2 has
    no physical page."""
    cfg = types.SimpleNamespace(page_size=64, head_dim=128, q_heads=8, kv_heads=4, topk=2, window=1,
                                kv_format="nvfp4")
    pt = np.array([[10, 11, 12, 13, 14, 15], [20, 21, -1, 23, 24, -1]], np.int32)
    w = types.SimpleNamespace(cfg=cfg, B=2, N=4, MP=6, page_table=pt,
                              seq_lens=np.array([300, 260], np.int32),
                              row_offsets=np.array([0, 2, 4], np.int32))
    # rows of request 0 list pages {0, 3, 4} and {1, 3, 4}; request 1 lists {0, 2, 4} and {1, 4}
    sel = np.array([[0, 3, 4], [1, 3, 4], [0, 2, 4], [1, 4, -1]], np.int32)
    return w, sel


def test_algorithmic_bytes_hand_count():
    w, sel = _mini()
    got = bench.algorithmic_bytes(w, sel)
    page = 64 * (128 // 2 + 128 // 16) * 2            # K + V codes and scales of one (page, KV head)
    # request 0: distinct listed pages {0, 1, 3, 4}, all valid; request 1: {0, 1, 2, 4}, page 2 invalid
    kv = (4 + 3) * 4 * page
    assert got["attention_kv"] == kv
    qo = 4 * 8 * 128 * 2
    listed = 4 + 4                                     # page-table entries read: distinct listed pages
    assert got["attention"] == kv + 2 * qo + 4 * 8 * 4 + 4 * 3 * 4 + listed * 4
    assert got["select_attention"] == got["attention"] + 4 * 6 * 4
    # index keys: candidates (valid pages before the window) per request and KV head; request 0
    # rows see 299 and 300 tokens (5 pages), request 1 rows 259 and 260 (5 pages); window 1
    cand0, cand1 = {0, 1, 2, 3}, {0, 1, 3}
    assert got["index"] == (len(cand0) + len(cand1)) * 4 * 128 * 2 + qo + 4 * 6 * 4
    assert got["step"] == got["index"] + got["select_attention"]


def test_traffic_scaling_from_counter_runs(tmp_path, monkeypatch):
    kernel = "sparse_decode_kernel<128, 8, 0, true, 8>"
    name = f"void qsa::{kernel}(qsa::DecodeParams)"

    def write(path, counter, dec_values, copy_value):
        with open(path, "w", newline="") as fh:
            wr = csv.writer(fh)
            wr.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
            for v in dec_values:
                wr.writerow([name, counter, v])
            wr.writerow(["void qsa::sparse_decode_kernel<128, 0, 0, true, 8>(qsa::DecodeParams)", counter, 1.0])
            wr.writerow(["__amd_rocclr_copyBuffer", counter, copy_value / 4])
            wr.writerow(["__amd_rocclr_copyBuffer", counter, copy_value])

    fetch, write_ = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the copy moves 1 GiB each way: FETCH_SIZE reads half of it (scale 2), WRITE_SIZE all of it
    write(fetch, "FETCH_SIZE", [100.0, 300.0, 200.0], (1 << 30) / 1024 / 2)
    write(write_, "WRITE_SIZE", [10.0, 12.0, 11.0], (1 << 30) / 1024)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic_{workload}.json"))
    bench.traffic_from_counters(str(fetch), str(write_), "w", kernel)
    t = __import__("json").load(open(tmp_path / "traffic_w.json"))
    assert t["dispatches"] == [3, 3]
    assert t["fetch_bytes"] == pytest.approx(200.0 * 1024 * 2)
    assert t["write_bytes"] == pytest.approx(11.0 * 1024)
    assert t["traffic_bytes"] == pytest.approx(200.0 * 1024 * 2 + 11.0 * 1024)
    assert t["source_sha256"] == bench.kernel_source_hash()


def test_source_hash_follows_code_not_comments():
    code = 'int f(int x) { // add one\n  return x + 1; /* "no" */ }\nconst char *s = "a // b /* c */";\n'
    same = '/* header */\nint f(int x) {\n\n  return x + 1;   }\n// trailer\nconst char *s = "a // b /* c */";'
    other = code.replace("x + 1", "x + 2")
    literal = code.replace('"a // b /* c */"', '"a // b"')
    st = bench._strip_comments
    assert st(code) == st(same)
    assert st(code) != st(other)
    assert st(code) != st(literal)                   # comment markers inside strings are code
    assert "add one" not in st(code) and '"a // b /* c */"' in st(code)


def _expected_select_cols(MP):
    return 2 if MP <= 128 else 4 if MP <= 256 else 8 if MP <= 512 else 16 if MP <= 1024 else 0


# the workloads' launch shapes: (B, rows, q heads, KV heads, d, page, MP, k, W)
SHAPES = {
    "tiny": (1, 1, 4, 1, 64, 64, 16, 4, 1),
    "decode_8k": (8, 1, 32, 4, 128, 64, 128, 16, 2),
    "mtp_verify_32k": (16, 4, 32, 4, 128, 64, 512, 32, 2),
    "long_131k": (4, 1, 64, 8, 128, 128, 1024, 64, 1),
    "wide_mixed": (48, 4, 32, 4, 128, 64, 1024, 32, 2),
    "context_8k": (4, 256, 32, 4, 128, 64, 128, 32, 2),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_fused_kernel_name_matches_the_launch(name):
    """The rocprofv3 name bench.py looks up: head dim, selection columns per lane (the fewest
    covering the table), one-row tiles, and 4-wave workgroups exactly when a one-row launch has
    more than two items per CU (all from the plan the library reports)."""
    import block_sparse_decode_amd as q
    B, R, Hq, Hkv, d, P, MP, k, W = SHAPES[name]
    cfg = types.SimpleNamespace(q_heads=Hq, kv_heads=Hkv, head_dim=d, page_size=P, topk=k, window=W,
                                kv_format="nvfp4")
    w = types.SimpleNamespace(cfg=cfg, B=B, N=B * R, max_rows=R, MP=MP, NP=B * MP, sm_scale=1.0 / math.sqrt(d))
    got = bench.fused_kernel_name(w)
    sh = q.Shape(B, B * R, R, Hq, Hkv, d, P, MP, B * MP, k, W, 1.0 / math.sqrt(d), 0)
    plan = q.qsa_plan_decode(sh, 0, True)
    G = Hq // Hkv
    one = plan.tile_cols == G
    items = B * Hkv * plan.col_tiles * plan.splits
    waves = 4 if (one and items > 512) else 8
    assert plan.select_cols == _expected_select_cols(MP)
    assert plan.waves == waves
    assert got == f"sparse_decode_kernel<{d}, {_expected_select_cols(MP)}, 0, {'true' if one else 'false'}, {waves}>"
    if name == "wide_mixed":
        assert waves == 4 and one
    if name in ("mtp_verify_32k", "long_131k", "decode_8k"):
        assert waves == 8 and one
    if name == "context_8k":
        assert not one
