"""CPU oracle for query-sparse NVFP4 decode / verify attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path never calls it and
has no fallback to it.

This is a thin ctypes wrapper over `qsa_oracle.c`, where each definition is
written out in plain C (see that file's comments for the passages it follows).
It shares no code with the GPU library. Every function takes numpy arrays in
the layouts documented in `synth` and returns numpy arrays.

Parity status (see tests/test_oracle_*.py):
  e2m1 / e4m3 decode   pinned: hand tables from the OCP specs, exhaustive torch float8_e4m3fn
  dequant              pinned: hand-multiplied page, byte-size identity of the pages
  rows                 pinned: closed forms
  index scores         pinned: integer-exact cases, fp64 error bound, per-head brute force
  selection            pinned: brute force over all tie patterns, invariants
  attention            pinned: brute-force dense softmax, torch SDPA (fp64) on full windows,
                       single-token and equal-key closed forms; the FP8 format against a
                       dense softmax over table-decoded bytes; the gate against scipy's
                       expit, gate 0 (exact half) and a saturating gate (unchanged)
  KV store             pinned: brute-force nearest-code search over every E2M1 / E4M3 code,
                       exactly representable blocks, closed-form index keys
  rollback (rollback.py, numpy)
                       pinned: array indexing of the cache layouts, restore invariants,
                       round trip, skipped and reported rows
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "qsa_oracle.c")

GCC_FLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (no fast-math, no contraction)."""
    cmd = ["gcc", *GCC_FLAGS, "-o", LIB_PATH, SRC_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_D = ctypes.c_double


def _declare(L):
    L.oracle_e2m1.argtypes = [_I]
    L.oracle_e2m1.restype = _D
    L.oracle_e4m3.argtypes = [_I]
    L.oracle_e4m3.restype = _D
    L.oracle_bf16.argtypes = [ctypes.c_uint16]
    L.oracle_bf16.restype = _D
    L.oracle_dequant_pages.argtypes = [_P, _P, _D, _I, _I, _I, _P, _I, _P]
    L.oracle_rows.argtypes = [_I, _P, _P, _I, _I, _P, _P, _P]
    L.oracle_index_scores.argtypes = [_I, _P, _P, _P, _I, _I64, _I, _I, _I, _I, _I, _F, _P, _P, _P]
    L.oracle_select.argtypes = [_I, _P, _P, _I, _I, _I, _I, _P, _P]
    L.oracle_attention.argtypes = [_I, _P, _P, _P, _I, _I64, _I, _I, _I, _I, _F, _D, _D,
                                   _P, _P, _P, _P, _P, _I, _P, _I, _P, _P, _P]
    L.oracle_attention_one.argtypes = [_I, _P, _P, _P, _I, _I64, _I, _I, _I, _I, _F, _D, _D,
                                       _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _P, _P]
    L.oracle_fp8_elem.argtypes = [_P, _D, _I, _I, _I, _I64, _I, _I, _I]
    L.oracle_fp8_elem.restype = _D
    L.oracle_e4m3_encode.argtypes = [_F]
    L.oracle_e4m3_encode.restype = ctypes.c_uint8
    L.oracle_e2m1_encode.argtypes = [_F]
    L.oracle_e2m1_encode.restype = ctypes.c_uint8
    L.oracle_nvfp4_encode_block.argtypes = [_P, _F, _P, _P]
    L.oracle_kv_store.argtypes = [_I, _P, _P, _P, _I, _I64, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P, _P, _P]


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(_P)


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(int(code))


def e4m3(byte: int) -> float:
    return lib().oracle_e4m3(int(byte))


def bf16(bits: int) -> float:
    return lib().oracle_bf16(int(bits))


def dequant_pages(codes, scales, global_scale, pages):
    """fp64 values of the listed physical pages: [n][Hkv][P][d]."""
    NP, Hkv, P, half = codes.shape
    d = half * 2
    codes, cp = _c(codes, np.uint8)
    scales, sp = _c(scales, np.uint8)
    pages, pp = _c(pages, np.int32)
    out = np.empty((len(pages), Hkv, P, d), np.float64)
    lib().oracle_dequant_pages(cp, sp, float(global_scale), Hkv, P, d, pp, len(pages),
                               out.ctypes.data_as(_P))
    return out


def rows(seq_lens, row_offsets, P, MP):
    """(request, visible tokens, visible pages) per row."""
    seq_lens, sl = _c(seq_lens, np.int32)
    row_offsets, ro = _c(row_offsets, np.int32)
    B = len(seq_lens)
    N = int(row_offsets[-1])
    rq = np.empty(N, np.int32)
    rl = np.empty(N, np.int32)
    rn = np.empty(N, np.int32)
    lib().oracle_rows(B, sl, ro, P, MP, rq.ctypes.data_as(_P), rl.ctypes.data_as(_P),
                      rn.ctypes.data_as(_P))
    return rq, rl, rn


def index_scores(w, *, window=None, sm_scale=None, q=None, keys=None, page_table=None):
    """fp32 score table [N][MP] for workload `w` (overrides for tests)."""
    cfg = w.cfg
    W = cfg.window if window is None else window
    s = np.float32(w.sm_scale if sm_scale is None else sm_scale)
    q = w.q if q is None else q
    keys = w.index_keys if keys is None else keys
    pt = w.page_table if page_table is None else page_table
    sl, slp = _c(w.seq_lens, np.int32)
    ro, rop = _c(w.row_offsets, np.int32)
    pt, ptp = _c(pt, np.int32)
    qa, qp = _c(q, np.uint16)
    ka, kp = _c(keys, np.uint16)
    NP, Hkv, d = ka.shape
    Hq = qa.shape[1]
    MP = pt.shape[1]
    out = np.empty((int(ro[-1]), MP), np.float32)
    lib().oracle_index_scores(len(sl), slp, rop, ptp, MP, NP, cfg.page_size, W, Hq, Hkv, d, s,
                              qp, kp, out.ctypes.data_as(_P))
    return out


def select(seq_lens, row_offsets, P, MP, k, W, scores):
    """int32 [N][k+W]: canonical top-k plus window, ascending, -1 padded."""
    sl, slp = _c(seq_lens, np.int32)
    ro, rop = _c(row_offsets, np.int32)
    sc, scp = _c(scores, np.float32)
    assert sc.shape == (int(ro[-1]), MP)
    out = np.empty((int(ro[-1]), k + W), np.int32)
    lib().oracle_select(len(sl), slp, rop, P, MP, k, W, scp, out.ctypes.data_as(_P))
    return out


def select_w(w, scores):
    c = w.cfg
    return select(w.seq_lens, w.row_offsets, c.page_size, w.MP, c.topk, c.window, scores)


KV_FORMATS = {"nvfp4": 0, "fp8": 1}


def _attn_args(w, selected, sm_scale, gate):
    c = w.cfg
    arrs = dict(
        sl=_c(w.seq_lens, np.int32), ro=_c(w.row_offsets, np.int32), pt=_c(w.page_table, np.int32),
        q=_c(w.q, np.uint16), kc=_c(w.k_codes, np.uint8), ks=_c(w.k_scales, np.uint8),
        vc=_c(w.v_codes, np.uint8), vs=_c(w.v_scales, np.uint8), sel=_c(selected, np.int32))
    arrs["gate"] = _c(gate, np.uint16) if gate is not None else (None, None)
    s = np.float32(w.sm_scale if sm_scale is None else sm_scale)
    return c, arrs, s, KV_FORMATS[getattr(c, "kv_format", "nvfp4")]


def attention(w, selected, sm_scale=None, gate=None):
    """fp64 (out [N][Hq][d], lse [N][Hq]) for workload `w` and selection rows; `gate`
    (bf16 bits [N][Hq][d], optional) multiplies out by its sigmoid."""
    c, a, s, fmt = _attn_args(w, selected, sm_scale, gate)
    N, Hq, d = w.q.shape
    sel = a["sel"][0]
    out = np.empty((N, Hq, d), np.float64)
    lse = np.empty((N, Hq), np.float64)
    lib().oracle_attention(w.B, a["sl"][1], a["ro"][1], a["pt"][1], w.MP, w.NP, c.page_size,
                           Hq, c.kv_heads, d, s, c.k_global, c.v_global, a["q"][1], a["kc"][1],
                           a["ks"][1], a["vc"][1], a["vs"][1], fmt, a["sel"][1], sel.shape[1],
                           a["gate"][1], out.ctypes.data_as(_P), lse.ctypes.data_as(_P))
    return out, lse


def attention_one(w, selected, row, head, sm_scale=None, gate=None):
    """fp64 (out [d], lse) for one (row, q head)."""
    c, a, s, fmt = _attn_args(w, selected, sm_scale, gate)
    N, Hq, d = w.q.shape
    sel = a["sel"][0]
    out = np.empty(d, np.float64)
    lse = np.empty(1, np.float64)
    lib().oracle_attention_one(w.B, a["sl"][1], a["ro"][1], a["pt"][1], w.MP, w.NP, c.page_size,
                               Hq, c.kv_heads, d, s, c.k_global, c.v_global, a["q"][1],
                               a["kc"][1], a["ks"][1], a["vc"][1], a["vs"][1], fmt, a["sel"][1],
                               sel.shape[1], a["gate"][1], int(row), int(head), out.ctypes.data_as(_P),
                               lse.ctypes.data_as(_P))
    return out, float(lse[0])


def e4m3_encode(t: float) -> int:
    """The E4M3 code nearest to a non-negative fp32 value (ties to the even code, at most 448)."""
    return int(lib().oracle_e4m3_encode(float(t)))


def e2m1_encode(y: float) -> int:
    """The E2M1 code nearest to an fp32 value (ties to the even code, magnitude at most 6)."""
    return int(lib().oracle_e2m1_encode(float(y)))


def nvfp4_encode_block(x, global_scale=1.0):
    """One block of 16 fp32 values -> (8 code bytes, scale byte)."""
    x, xp = _c(np.asarray(x, np.float32).reshape(16), np.float32)
    codes = np.zeros(8, np.uint8)
    sc = np.zeros(1, np.uint8)
    lib().oracle_nvfp4_encode_block(xp, float(global_scale), codes.ctypes.data_as(_P), sc.ctypes.data_as(_P))
    return codes, int(sc[0])


def kv_store(w, new_k, new_v):
    """The KV store of one step on copies of the workload's planes.

    new_k / new_v: bf16 bits [N][Hkv][d]. Returns (k_codes, k_scales, v_codes, v_scales,
    index_keys) after the store; the workload itself is not modified.
    """
    c = w.cfg
    sl, slp = _c(w.seq_lens, np.int32)
    ro, rop = _c(w.row_offsets, np.int32)
    pt, ptp = _c(w.page_table, np.int32)
    nk, nkp = _c(new_k, np.uint16)
    nv, nvp = _c(new_v, np.uint16)
    planes = [np.array(a, copy=True) for a in (w.k_codes, w.k_scales, w.v_codes, w.v_scales, w.index_keys)]
    ptrs = [a.ctypes.data_as(_P) for a in planes]
    lib().oracle_kv_store(w.B, slp, rop, ptp, w.MP, w.NP, c.kv_heads, c.page_size, c.head_dim,
                          float(c.k_global), float(c.v_global), nkp, nvp, *ptrs)
    return tuple(planes)
