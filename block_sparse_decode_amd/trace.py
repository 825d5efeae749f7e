"""Phase breakdown of the attention kernel: a traced build of the library (-DQSA_TRACE) stamps
the 100 MHz real-time clock per wave at fixed points of sparse_decode_kernel, and this script
prints their distribution over the workgroups of one launch.

    python -m block_sparse_decode_amd.trace build                 # on any host (hipcc)
    python -m block_sparse_decode_amd.trace run [--workload W]    # on the GPU

Times are microseconds from the earliest workgroup's entry. The traced library is built into
_build/ and loaded in place of libqsa.so. A wave keeps its stamps in LDS and writes them out when
it leaves, so the stamps add no stores for later loads to wait behind; a stamp still waits for
the LDS and scalar operations in flight before it, so the traced kernel runs slightly slower
than the product build.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(ROOT, "_build", "libqsa_trace.so")

GROUPS, WAVES, POINTS = 4096, 8, 16
# point -> (name, waves that stamp it: None = every wave, 0 = the selecting wave)
NAMES = {
    0: ("entry", None), 1: ("row range", None), 2: ("scores -> keys", 0), 3: ("bit search", 0),
    4: ("tie ranking", 0), 5: ("union published", 0), 6: ("before barrier", None), 7: ("after barrier", None),
    12: ("union placed", None),
    8: ("first loads", None), 9: ("loop end", None), 11: ("wave merge", None), 10: ("output written", None),
}


def build(verbose: bool = True) -> str:
    from . import build as b
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = b.command(OUT)
    cmd.insert(1, "-DQSA_TRACE=1")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(res.stderr)
    return OUT


def run(workload: str, launches: int = 200, fused: bool = True, groups: int = 0):
    import numpy as np
    import torch
    import block_sparse_decode_amd as q
    import synth
    from .batch import DeviceBatch, Step

    if not os.path.exists(OUT):
        raise FileNotFoundError(f"{OUT} is missing: run `python -m block_sparse_decode_amd.trace build` first")
    q.LIB_PATH = OUT
    L = q.lib()
    L.qsa_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.qsa_trace_read.restype = ctypes.c_int
    w = synth.generate(workload)
    b = DeviceBatch.upload(w, "cuda:0")
    st = Step(b, fused=fused)
    st.scores_call()
    st.select_call()
    call = st.select_decode_call if fused else st.decode_call
    for _ in range(20):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    plan = q.qsa_plan_decode(b.shape(), 0, fused)
    n = min(int(plan.workgroups), GROUPS) if groups <= 0 else min(groups, GROUPS)
    buf = np.zeros(GROUPS * WAVES * POINTS, np.uint64)
    rc = L.qsa_trace_read(buf.ctypes.data, buf.size)
    if rc != 0:
        raise RuntimeError(f"qsa_trace_read: HIP error {rc}")
    a = buf.reshape(GROUPS, WAVES, POINTS)[:n].astype(np.int64)
    live = a[:, :, 0] > 0
    t0 = a[:, :, 0][live].min()
    rel = (a - t0) * 0.01                       # 100 MHz ticks -> microseconds
    kind = "fused selection + attention" if fused else "attention (selection given)"
    print(f"workload {workload}: {kind}, {n} workgroups of {plan.waves} waves ({plan.rows_per_tile} row(s) per "
          f"tile, {plan.splits} split(s)), traced launch mean {us:.2f} us over {launches} back-to-back launches")
    print(f"{'point':18s} {'p10':>7s} {'p50':>7s} {'p90':>7s} {'max':>7s}   (us from the first workgroup's entry)")
    # a stamp belongs to this launch when it is not older than its wave's entry (workgroups of
    # split tiles that are not the last to finish leave the later points of an earlier launch)
    entry = a[:, :, 0:1]
    for k, (name, who) in NAMES.items():
        if who is None:
            v = rel[:, :, k]
            ok = (a[:, :, k] > 0) & (a[:, :, k] >= entry[:, :, 0])
        else:
            # stamped by the selecting wave alone (which wave that is may vary by workgroup)
            sw = np.argmax(a[:, :, k], axis=1)
            rows = np.arange(a.shape[0])
            v = rel[rows, sw, k]
            ok = (a[rows, sw, k] > 0) & (a[rows, sw, k] >= entry[rows, sw, 0])
        v = v[ok]
        if v.size == 0:
            continue
        print(f"{name:18s} {np.percentile(v, 10):7.2f} {np.percentile(v, 50):7.2f} {np.percentile(v, 90):7.2f} "
              f"{v.max():7.2f}")
    ends = [np.percentile(rel[:, wv, 9][a[:, wv, 9] > 0], 50) for wv in range(WAVES) if (a[:, wv, 9] > 0).any()]
    print("loop end per wave (p50):", " ".join(f"{x:.2f}" for x in ends))
    sys.stdout.flush()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["build", "run"])
    ap.add_argument("--workload", default="mtp_verify_32k")
    ap.add_argument("--launches", type=int, default=200)
    ap.add_argument("--unfused", action="store_true")
    args = ap.parse_args()
    if args.what == "build":
        print(build())
    else:
        sys.path.insert(0, ROOT)
        run(args.workload, args.launches, not args.unfused)


if __name__ == "__main__":
    main()
