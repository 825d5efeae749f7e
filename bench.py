"""Benchmark: query-sparse NVFP4 decode / verify attention, one step = one layer's hot path.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mtp_verify_32k]

A step runs the whole path over one batch on one GPU in two launches:
index scores, then the canonical top-k fused into the split-KV attention launch
(qsa_select_sparse_decode).

Inputs are synthetic and seeded (module `synth`), already resident in HBM. The paged
cache is replicated over several "layers", and consecutive steps walk through them,
as a decode step walks through a model's attention layers. So each step reads its K/V
from HBM, not from the 256 MB MALL (the pages a step touches are evicted before that
layer comes round again).

Output: one JSON line with the contract's fields plus
  roofline      -- the dominant kernel (the fused selection + attention launch) against
                   MI355X's 8 TB/s HBM peak, from algorithmic bytes per launch and HIP-event
                   durations on its stream;
  cpu_baseline  -- the CPU oracle on a bounded sample of the same workload (single thread);
  stages        -- mean HIP-event microseconds of each call, the fused one and the separate
                   selection and attention calls.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse NVFP4 decode attention: µs/step + achieved HBM GB/s (% of peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
COPY_BYTES = 1 << 30           # the calibration copy (--copy-calibration)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sparse_decode_{workload}.json")


# the sources that build and launch the fused selection + attention kernel
DECODE_SOURCES = ("qsa_api.hip", "qsa_decode.hip", "qsa_device.hpp", "qsa_internal.hpp", "qsa_select_row.hpp")


def _strip_comments(text):
    """C/C++ source without its comments and with each run of white space made one space (string
    and character literals kept as they are), so that the hash below follows the code the
    compiler sees, not the prose and layout around it."""
    import re
    tok = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)
    code = tok.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), text)
    return " ".join(code.split())


def kernel_source_hash():
    """SHA-256 over the sources of the fused kernel and the header, comments and layout removed;
    traffic counters are valid for this hash only."""
    import hashlib
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "block_sparse_decode_amd", "csrc", f) for f in DECODE_SOURCES] + \
        [os.path.join(ROOT, "include", "qsa.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_strip_comments(fh.read()).encode())
    return h.hexdigest()


def traffic_from_counters(fetch_csv, write_csv, workload, kernel):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of this
    script with --copy-calibration into HBM bytes per sparse_decode_kernel launch.

    Each counter is scaled by what it reads for the calibration copy, a plain device copy of
    COPY_BYTES read and COPY_BYTES written (the copy dispatch is the one with the largest
    reading). Writes the result next to the kernel-time summaries, tagged with the source hash.
    """
    import csv
    import statistics

    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        dec = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
        cpy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        assert dec, f"no {kernel} dispatch in {path}"
        return statistics.median(dec), cpy, len(dec)

    f_dec, f_cpy, n_f = load(fetch_csv, "FETCH_SIZE")
    w_dec, w_cpy, n_w = load(write_csv, "WRITE_SIZE")
    f_scale = COPY_BYTES / (f_cpy * 1024.0)
    w_scale = COPY_BYTES / (w_cpy * 1024.0)
    out = {
        "kernel": kernel, "workload": workload, "source_sha256": kernel_source_hash(),
        "fetch_kib_per_dispatch_median": f_dec, "write_kib_per_dispatch_median": w_dec,
        "dispatches": [n_f, n_w],
        "copy_fetch_kib": f_cpy, "copy_write_kib": w_cpy, "fetch_scale": f_scale, "write_scale": w_scale,
        "fetch_bytes": f_dec * 1024.0 * f_scale, "write_bytes": w_dec * 1024.0 * w_scale,
    }
    out["traffic_bytes"] = out["fetch_bytes"] + out["write_bytes"]
    path = TRAFFIC_FILE.format(workload=workload)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def measured_traffic(workload):
    """HBM bytes per decode launch from the committed counter runs, if they match this source."""
    path = TRAFFIC_FILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha256") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t["traffic_bytes"]


def algorithmic_bytes(w, selected):
    """Bytes the method must move per step (the layout's minimum), from the actual selection.

    attention: for each request and KV head, every distinct valid page that any of its rows
    selected, K + V codes and scales (P * (d/2 + d/16) * 2 bytes); plus q, out, lse, the
    selection rows and the page-table entries it reads.
    select_attention: the fused launch; attention plus the score table it reads (the
    selection rows are then written instead of read).
    index:     every candidate page's key for every KV head, q, and the score table written.
    select:    the score table read and the selection written.
    """
    import numpy as np
    c = w.cfg
    P, d, Hq, Hkv = c.page_size, c.head_dim, c.q_heads, c.kv_heads
    KW = c.topk + c.window
    fp8 = getattr(c, "kv_format", "nvfp4") == "fp8"
    page_bytes = P * (d if fp8 else d // 2 + d // 16) * 2       # K + V of one (page, KV head)
    attn_kv = 0
    pt_entries = 0
    index_keys = 0
    for b in range(w.B):
        r0, r1 = int(w.row_offsets[b]), int(w.row_offsets[b + 1])
        R = r1 - r0
        listed = set()
        cand = set()
        for j in range(R):
            for p in selected[r0 + j]:
                if p >= 0:
                    listed.add(int(p))
            L = int(w.seq_lens[b]) - (R - 1 - j)
            n = min(-(-max(L, 0) // P), w.MP)
            for p in range(max(0, n - c.window)):
                if w.page_table[b, p] >= 0:
                    cand.add(p)
        valid = [p for p in listed if w.page_table[b, p] >= 0]
        attn_kv += len(valid) * Hkv * page_bytes
        pt_entries += len(listed)
        index_keys += len(cand) * Hkv * d * 2
    qo = w.N * Hq * d * 2
    attn = attn_kv + qo + qo + w.N * Hq * 4 + w.N * KW * 4 + pt_entries * 4
    index = index_keys + qo + w.N * w.MP * 4
    select = w.N * w.MP * 4 + w.N * KW * 4
    fused = attn + w.N * w.MP * 4
    return dict(attention=attn, attention_kv=attn_kv, index=index, select=select, select_attention=fused,
                step=index + fused)


def store_bytes(w):
    """Bytes the KV store must move per step: the new K and V rows read (bf16), their codes and
    scales written, the stored K of each touched page's other valid tokens read back for the
    key, and the keys written."""
    c = w.cfg
    P, d, Hkv = c.page_size, c.head_dim, c.kv_heads
    tok = d // 2 + d // 16
    new_in = new_out = old_k = keys = 0
    for b in range(w.B):
        r0, r1 = int(w.row_offsets[b]), int(w.row_offsets[b + 1])
        R, L = r1 - r0, int(w.seq_lens[b])
        new_in += R * Hkv * d * 2 * 2
        pages = {}
        for j in range(R):
            pos = L - R + j
            if pos < 0 or pos // P >= w.MP or w.page_table[b, pos // P] < 0:
                continue
            new_out += Hkv * tok * 2
            pages.setdefault(pos // P, 0)
            pages[pos // P] += 1
        for page, fresh in pages.items():
            n = min(P, L - page * P)
            old_k += (n - fresh) * Hkv * tok
            keys += Hkv * d * 2
    return new_in + new_out + old_k + keys


def attention_flop(w, selected):
    """MFMA work the attention must do: 4 d flop (q.k and p.v) per (row, q head, visible
    selected token)."""
    c = w.cfg
    P = c.page_size
    toks = 0
    for b in range(w.B):
        r0, r1 = int(w.row_offsets[b]), int(w.row_offsets[b + 1])
        for j in range(r1 - r0):
            L = int(w.seq_lens[b]) - (r1 - r0 - 1 - j)
            for p in set(int(x) for x in selected[r0 + j] if x >= 0):
                if w.page_table[b, p] >= 0:
                    toks += max(0, min(P, L - p * P))
    return 4 * c.head_dim * c.q_heads * toks


def fused_kernel_name(w):
    """Name rocprofv3 gives the fused selection + attention kernel for this workload, from the
    launch plan the library reports (selection columns per lane, one-row tiles, waves per
    workgroup)."""
    import block_sparse_decode_amd as q
    from block_sparse_decode_amd.batch import DeviceBatch
    c = w.cfg
    fmt = 1 if getattr(c, "kv_format", "nvfp4") == "fp8" else 0
    sh = q.Shape(int(w.B), int(w.N), max(1, int(w.max_rows)), c.q_heads, c.kv_heads, c.head_dim, c.page_size,
                 int(w.MP), int(w.NP), c.topk, c.window, float(w.sm_scale), fmt)
    plan = q.qsa_plan_decode(sh, 0, True)
    G = c.q_heads // c.kv_heads
    one = plan.tile_cols == G if G <= 16 else G % 16 == 0
    return (f"sparse_decode_kernel<{c.head_dim}, {plan.select_cols}, {fmt}, {'true' if one else 'false'}, "
            f"{plan.waves}>")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _sub_workload(w, b0, b1):
    """Requests [b0, b1) of a workload (whole requests, their rows and the shared pools)."""
    import synth
    r0, r1 = int(w.row_offsets[b0]), int(w.row_offsets[b1])
    return synth.Workload(w.cfg, w.page_table[b0:b1], w.seq_lens[b0:b1], w.row_offsets[b0:b1 + 1] - r0,
                          w.q[r0:r1], w.k_codes, w.k_scales, w.v_codes, w.v_scales, w.index_keys)


def _oracle_step(sub):
    import oracle
    s = oracle.index_scores(sub)
    sel = oracle.select_w(sub, s)
    oracle.attention(sub, sel)


def cpu_baseline(w, max_rows, runs=5):
    """The CPU oracle (plain C, -O2, no fast-math) timed on this host: single-threaded on the
    first requests (up to max_rows rows), median of `runs` runs; then the whole step with the
    requests spread over every host thread (the oracle's calls release the interpreter lock,
    and requests are independent), median of 3 runs. Both scaled to a step of w."""
    import concurrent.futures
    import statistics
    nb = 0
    while nb < w.B and int(w.row_offsets[nb + 1]) <= max_rows:
        nb += 1
    nb = max(1, nb)
    rows = int(w.row_offsets[nb])
    sub = _sub_workload(w, 0, nb)
    single = []
    for _ in range(runs):
        t0 = time.perf_counter()
        _oracle_step(sub)
        single.append(time.perf_counter() - t0)
    single_step = statistics.median(single) * w.N / rows
    # this process's share of the host: the affinity mask, capped by OMP_NUM_THREADS where the
    # environment sets it (a shared GPU host gives each GPU a share of its cores)
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = max(1, min(avail, cap if cap > 0 else avail, w.B))
    parts = [_sub_workload(w, b, b + 1) for b in range(w.B)]
    multi = []
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        for _ in range(3):
            t0 = time.perf_counter()
            list(ex.map(_oracle_step, parts))
            multi.append(time.perf_counter() - t0)
    return dict(single_step_s=single_step, single_rows=rows, single_runs=single, threads=threads,
                multi_step_s=statistics.median(multi), multi_runs=multi, model=_cpu_model())


def timed_us(fn, seq, stream, K, reps=1):
    """µs per launch of fn over K back-to-back calls rotating through seq, between one HIP
    event pair on the launch stream, after as many warmup calls (at least two per element of
    seq). A stage timed right after other, lighter stages otherwise starts below its steady
    clock: the gated attention read 1.4 µs slow after a warmup of 32 calls (0.7 ms).
    With reps > 1 the K calls are timed in `reps` batches and the batch means are returned."""
    import torch
    n = len(seq)
    for i in range(max(K, 2 * n)):
        fn(seq[i % n])
    torch.cuda.synchronize()
    per = max(1, K // reps)
    out = []
    for r in range(reps):
        a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(per):
            fn(seq[(r * per + i) % n])
        b2.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b2) * 1e3 / per)
    return out if reps > 1 else out[0]


def spread(xs):
    """median, p10, p90 of a list of batch means (µs)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


def context_stage(args, q, synth, DeviceBatch, Step, dev, stream, K):
    """Index scores and the fused attention of a context step (4 requests x 256 causal rows
    of 8K tokens, 16 layer copies of the pools), each timed over K back-to-back launches."""
    import torch
    wc = synth.generate("context_8k")
    basec = DeviceBatch.upload(wc, dev)
    layersc = [basec]
    for _ in range(15):
        bc = DeviceBatch(**{**basec.__dict__})
        for name in ("k_codes", "k_scales", "v_codes", "v_scales", "index_keys"):
            setattr(bc, name, getattr(basec, name).clone())
        layersc.append(bc)
    stepsc = [Step(b, num_splits=args.splits) for b in layersc]
    for st in stepsc:
        st(stream)
    torch.cuda.synchronize()
    selc = stepsc[0].selected.cpu().numpy()

    def stagec_us(fn):
        return timed_us(fn, stepsc, stream, K)
    ctx_index_us = stagec_us(lambda st: st.scores_call(stream))
    ctx_attn_us = stagec_us(lambda st: st.select_decode_call(stream))
    ctx_flop = attention_flop(wc, selc)
    return {"context_8k_index_scores_us": round(ctx_index_us, 2),
            "context_8k_select_sparse_decode_us": round(ctx_attn_us, 2),
            "context_8k_attention_tflops": round(ctx_flop / (ctx_attn_us * 1e-6) / 1e12, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="mtp_verify_32k")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--cpu-rows", type=int, default=8,
                    help="rows of the single-threaded CPU-oracle sample (0 = skip the CPU baseline)")
    ap.add_argument("--context", action="store_true",
                    help="also time a context step (4 x 256 rows of 8K; its attention launches the same kernel as "
                         "the verify step, so it is off when profiling that kernel)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for PMC byte-counter scaling)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 counter runs into the traffic file and exit")
    args = ap.parse_args()
    if args.traffic_from:
        import synth
        traffic_from_counters(args.traffic_from[0], args.traffic_from[1], args.workload,
                              fused_kernel_name(synth.generate(args.workload)))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "requests are independent, so a deployment shards them across GPUs with no exchange", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import block_sparse_decode_amd as q
    from block_sparse_decode_amd.batch import DeviceBatch, Step

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    q.lib()
    w = synth.generate(args.workload)
    base = DeviceBatch.upload(w, dev)
    # layer copies of the pools (distinct HBM addresses, same contents)
    layers = [base]
    for _ in range(1, args.layers):
        b = DeviceBatch(**{**base.__dict__})
        for name in ("k_codes", "k_scales", "v_codes", "v_scales", "index_keys"):
            setattr(b, name, getattr(base, name).clone())
        layers.append(b)
    steps = [Step(b, num_splits=args.splits) for b in layers]
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        steps[i % len(steps)](stream)
    torch.cuda.synchronize()
    sel = steps[0].selected.cpu().numpy()
    splits = args.splits if args.splits > 0 else None

    K = args.steps
    # (1) whole steps: the contract's wall-clock region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        steps[i % len(steps)](stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # (1b) the same steps replayed from one captured HIP graph (one step per layer copy)
    graph = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    with torch.cuda.stream(gs):
        for st in steps:
            st(gs)
    stream.wait_stream(gs)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        cur = torch.cuda.current_stream()
        for st in steps:
            st(cur)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    reps_g = max(2, K // len(steps))
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ga.record()
    for _ in range(reps_g):
        graph.replay()
    gb.record()
    torch.cuda.synchronize()
    graph_step_us = ga.elapsed_time(gb) * 1e3 / (reps_g * len(steps))
    del graph

    # (2) each call alone: back-to-back launches between one pair of HIP events on the launch
    # stream (per-call events would add the event round trip to every launch), in 20 batches
    # of 25 launches whose means give the median and the p10 / p90 spread; the mean over all
    # batches is the stage's average launch time
    STAGE_LAUNCHES, STAGE_REPS = 500, 20
    spreads = {}

    def stage_us(fn, name=None):
        xs = timed_us(fn, steps, stream, STAGE_LAUNCHES, STAGE_REPS)
        if name:
            spreads[name] = spread(xs)
        return sum(xs) / len(xs)
    fus_us = stage_us(lambda st: st.select_decode_call(stream), "select_sparse_decode")
    dec_us = stage_us(lambda st: st.decode_call(stream), "sparse_decode")
    idx_us = stage_us(lambda st: st.scores_call(stream), "index_scores")
    sel_us = stage_us(lambda st: st.select_call(stream), "select_topk")

    # (3) the KV store that precedes a step (this step's new K / V rows into the pools); run
    # last, since it rewrites the rows' slots and the touched pages' index keys
    import ctypes
    gen = np.random.default_rng(0)
    new_kv = [torch.from_numpy(synth.bf16_bits_from_f32(
        gen.standard_normal((w.N, w.cfg.kv_heads, w.cfg.head_dim), dtype=np.float32)).view(np.int16)).to(dev)
        for _ in range(2)]
    L = q.lib()
    store_args = {id(st): (ctypes.byref(st.shape_), ctypes.byref(st.paged_), new_kv[0].data_ptr(),
                           new_kv[1].data_ptr(), stream.cuda_stream) for st in steps}

    def store(st):
        status = L.qsa_kv_store(*store_args[id(st)])
        if status != 0:
            raise q.QsaError(status, "qsa_kv_store")
    store_us = stage_us(store)

    # (4) the rollback around a verify step: gather the plane rows the step's rows overwrite,
    # and restore half of them (the rejected drafts)
    ctx = {}
    for st in steps:
        n = w.N
        pages = torch.empty(n, dtype=torch.int32, device=dev)
        within = torch.empty(n, dtype=torch.int32, device=dev)
        q.qsa_step_slots(st.shape_, st.paged_, pages, within, stream)
        planes = st.b.rollback_planes()
        arr = (q.Plane * len(planes))(*planes)
        sb = q.qsa_rollback_stash_bytes(planes, n)
        stash = torch.zeros(sb, dtype=torch.uint8, device=dev)
        rej = torch.from_numpy((np.arange(n) % 2).astype(np.int32)).to(dev)
        ctx[id(st)] = (arr, len(planes), pages, within, rej, stash, sb)

    def gather(st):
        arr, npl, pages, within, rej, stash, sb = ctx[id(st)]
        status = L.qsa_rollback_gather(arr, npl, pages.data_ptr(), within.data_ptr(), w.N, stash.data_ptr(), sb,
                                       None, stream.cuda_stream)
        if status != 0:
            raise q.QsaError(status, "qsa_rollback_gather")

    def restore(st):
        arr, npl, pages, within, rej, stash, sb = ctx[id(st)]
        status = L.qsa_rollback_restore(arr, npl, pages.data_ptr(), within.data_ptr(), rej.data_ptr(), w.N,
                                        stash.data_ptr(), sb, None, stream.cuda_stream)
        if status != 0:
            raise q.QsaError(status, "qsa_rollback_restore")
    gather_us = stage_us(gather)
    restore_us = stage_us(restore)
    row_bytes = sum(pl.nseg * pl.seg_bytes for pl in steps[0].b.rollback_planes())

    # (5) the attention variants: the gated epilogue (same pools), and FP8 pools (unit-scale
    # E4M3, two layers of the same workload re-encoded)
    gen = np.random.default_rng(1)
    gate = torch.from_numpy(synth.bf16_bits_from_f32(gen.standard_normal(w.q.shape, dtype=np.float32)).view(
        np.int16)).to(dev)
    gsteps = {id(st): Step(st.b, num_splits=args.splits, gate=gate) for st in steps}
    for st in steps:
        gsteps[id(st)].scores.copy_(st.scores)      # the same scores, so the same selections
    gated_us = stage_us(lambda st: gsteps[id(st)].select_decode_call(stream))
    w8 = synth.generate(w.cfg.with_(kv_format="fp8", name=w.cfg.name + "_fp8"))
    base8 = DeviceBatch.upload(w8, dev)
    layers8 = [base8]
    b8 = DeviceBatch(**{**base8.__dict__})
    for name in ("k_codes", "k_scales", "v_codes", "v_scales", "index_keys"):
        setattr(b8, name, getattr(base8, name).clone())
    layers8.append(b8)
    steps8 = [Step(b, num_splits=args.splits) for b in layers8]
    for st in steps8:
        st(stream)
    torch.cuda.synchronize()
    sel8 = steps8[0].selected.cpu().numpy()

    def stage8_us(fn):
        return timed_us(fn, steps8, stream, K)
    fp8_us = stage8_us(lambda st: st.select_decode_call(stream))
    fp8_bytes = algorithmic_bytes(w8, sel8)["select_attention"]
    del steps8, layers8, base8, b8

    # (7) the reference the measurement is read against: a plain 512 MiB device-to-device copy
    csrc = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    torch.cuda.synchronize()
    ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ca.record(stream)
    for _ in range(20):
        cdst.copy_(csrc)
    cb.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * csrc.numel() / (ca.elapsed_time(cb) * 1e-3 / 20) / 1e9
    del csrc, cdst

    # (6) a context step (--context): 4 requests x 256 causal rows of 8K tokens
    ctx_stages = {}
    if args.context:
        ctx_stages = context_stage(args, q, synth, DeviceBatch, Step, dev, stream, K)

    err = int(base.error_word[0].item())

    ab = algorithmic_bytes(w, sel)
    ab["kv_store"] = store_bytes(w)
    ab["rollback_gather"] = 2 * w.N * row_bytes                 # read the rows, write the stash
    ab["rollback_restore"] = 2 * (w.N // 2) * row_bytes         # half the rows rejected
    us_step = wall / K * 1e6
    achieved = ab["select_attention"] / (fus_us * 1e-6) / 1e9
    step_gbs = ab["step"] / (us_step * 1e-6) / 1e9

    c = w.cfg
    out = {
        "metric": METRIC,
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 5),
        "us_per_step": round(us_step, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": c.name, "batch": c.batch, "rows_per_request": c.rows, "q_heads": c.q_heads,
                   "kv_heads": c.kv_heads, "head_dim": c.head_dim, "page_size": c.page_size,
                   "context": c.context, "topk": c.topk, "window": c.window, "kv_cache": "nvfp4",
                   "layers_rotated": args.layers,
                   "num_splits": splits or "auto"},
        "stages": {"index_scores_us": round(idx_us, 2), "select_sparse_decode_us": round(fus_us, 2),
                   "separate_select_topk_us": round(sel_us, 2), "separate_sparse_decode_us": round(dec_us, 2),
                   "kv_store_us": round(store_us, 2),
                   "kv_store_gbs": round(ab["kv_store"] / (store_us * 1e-6) / 1e9, 1),
                   "rollback_gather_us": round(gather_us, 2), "rollback_restore_us": round(restore_us, 2),
                   "gated_select_sparse_decode_us": round(gated_us, 2),
                   "fp8_select_sparse_decode_us": round(fp8_us, 2),
                   "fp8_select_attention_gbs": round(fp8_bytes / (fp8_us * 1e-6) / 1e9, 1),
                   **ctx_stages,
                   "graph_step_us": round(graph_step_us, 2),
                   "spread_us": spreads,
                   "timing": "mean of back-to-back launches between HIP event pairs on the launch stream (20 batches "
                             "of 25), after as many warmup launches; spread_us: median, p10, p90 of the batch means; "
                             "graph_step_us: one step per layer copy replayed from a captured HIP graph"},
        "bytes": ab,
        "reference_copy_gbs": round(copy_gbs, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(c.name),
                     "kernel": "qsa_select_sparse_decode (" + fused_kernel_name(w) + ")"},
        "error_word": err,
    }
    if args.cpu_rows > 0:
        cb = cpu_baseline(w, args.cpu_rows)
        one = cb["single_step_s"]
        allt = cb["multi_step_s"]
        out["cpu_baseline"] = {
            "value": round(ab["step"] / allt / 1e9, 4), "unit": "GB/s", "us_per_step": round(allt * 1e6, 1),
            "cores": cb["threads"], "kind": "oracle", "cpu_model": cb["model"],
            "sample": f"the whole step ({w.N} rows, all three stages) with the {w.B} requests spread over "
                      f"{cb['threads']} host threads, median of 3 runs "
                      f"({', '.join(f'{x:.2f}' for x in cb['multi_runs'])} s)",
            "single_thread": {"value": round(ab["step"] / one / 1e9, 4), "unit": "GB/s",
                              "us_per_step": round(one * 1e6, 1), "cores": 1,
                              "sample": f"first {cb['single_rows']} of {w.N} rows (whole requests), median of "
                                        f"{len(cb['single_runs'])} runs "
                                        f"({', '.join(f'{x:.2f}' for x in cb['single_runs'])} s), scaled to the "
                                        "full step"}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
