"""Seeded synthetic inputs for query-sparse NVFP4 decode / verify attention.

This module only *makes data*. It draws seeded normal values and stores them in
the paged NVFP4 cache format. It also draws bf16 queries and builds the page
table, sequence lengths and row offsets of a batch. Both the CPU oracle and
the GPU path consume what it produces. It computes none of the method's steps:
no index scores, no selection and no attention. The only arithmetic here is what
turns normal draws into stored bytes:

* the NVFP4 *encoder*: an e4m3 block scale per 16 elements, then e2m1 codes;
* the per-page index key: the mean over the page's valid tokens of the
  unquantised K, rounded to bf16.

Both stages read NVFP4 back through the decoders in `oracle/` and
`block_sparse_decode_amd/`, never through this module.

Workload shapes follow the five configurations of the benchmark, each named by
what it is. The pages measure with 8K-token prompts, MTP with three drafts,
131K tables and 48 x (1+3) verify rows. Since no dataset is used, synthetic
inputs of those shapes stand in for them.

Memory layout (device and host alike, all C-contiguous):
    q           uint16 (bf16 bits)  [N][Hq][d]
    k_codes     uint8               [NP][Hkv][P][d/2]   e2m1, low nibble = even element
    k_scales    uint8               [NP][Hkv][P][d/16]  OCP E4M3FN
    v_codes     uint8               [NP][Hkv][P][d/2]
    v_scales    uint8               [NP][Hkv][P][d/16]
    index_keys  uint16 (bf16 bits)  [NP][Hkv][d]
    page_table  int32               [B][MP]             -1 = invalid entry
    seq_lens    int32               [B]                 tokens incl. this step's rows
    row_offsets int32               [B+1]               rows of request b
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import hashlib
import math
import os
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "Config", "Workload", "CONFIGS", "generate", "bf16_bits_from_f32",
    "f32_from_bf16_bits", "encode_nvfp4", "encode_e4m3", "encode_fp8", "E4M3_POS_VALUES",
]

# --------------------------------------------------------------------------
# Format tables used by the encoder (OCP 8-bit FP spec, E4M3FN; OCP MX v1.0, E2M1)
# --------------------------------------------------------------------------


def _e4m3_positive_values() -> np.ndarray:
    """Values of the finite non-negative E4M3FN codes 0x00..0x7E, in code order."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3_POS_VALUES = _e4m3_positive_values()
_E4M3_MIDS = 0.5 * (E4M3_POS_VALUES[1:] + E4M3_POS_VALUES[:-1])
_E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float64)


def _rne_index(mids: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Index of the nearest grid point for non-negative `a` (ties to the even index).

    `mids` are the midpoints between consecutive grid values. Values past the
    last midpoint saturate to the last grid point.
    """
    j = np.searchsorted(mids, a, side="left")
    jc = np.minimum(j, len(mids) - 1)
    tie = (a == mids[jc]) & (j < len(mids)) & ((j & 1) == 1)
    return (j + tie).astype(np.uint8)


def encode_e4m3(y: np.ndarray) -> np.ndarray:
    """Round non-negative float64 values to E4M3FN codes (RNE, saturating at 448)."""
    return _rne_index(_E4M3_MIDS, y)


def encode_nvfp4(x: np.ndarray, global_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise float32 `x[..., d]` to NVFP4: packed e2m1 codes and e4m3 block scales.

    Per block of 16 elements the scale is E4M3_RNE(amax / 6 / global). Each
    element then becomes E2M1_RNE(x / (scale * global)), saturating at +-6. An
    all-zero block gets scale 0 and codes 0. Returns (codes uint8[..., d/2] with
    the even element in the low nibble, scales uint8[..., d/16]).

    The e2m1 rounding compares |x| with the midpoints times the block's scale.
    Those products need at most 7 significant bits, so for a power-of-two
    global scale they are exact in float32, and the comparison is the exact
    RNE decision (ties go to the even code).
    """
    d = x.shape[-1]
    assert d % 16 == 0
    g = float(global_scale)
    m_, e_ = math.frexp(g)
    pow2 = (m_ == 0.5)
    blocks = x.reshape(x.shape[:-1] + (d // 16, 16))
    absb = np.abs(blocks)
    amax = absb.max(axis=-1).astype(np.float64)
    s_code = encode_e4m3(amax / 6.0 / g)
    denom = E4M3_POS_VALUES[s_code] * g
    zero = denom == 0.0
    ftype = np.float32 if pow2 else np.float64
    mag = np.zeros(absb.shape, dtype=np.uint8)
    for j, mid in enumerate(_E2M1_MIDS):
        t = (mid * denom).astype(ftype)[..., None]
        if j & 1:       # tie goes up to the even code above
            mag += absb >= t
        else:           # tie stays on the even code below
            mag += absb > t
    code = mag | (np.signbit(blocks).astype(np.uint8) << 3)
    code[zero] = 0
    code = code.reshape(x.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(s_code)


def encode_fp8(x: np.ndarray, global_scale: float = 1.0) -> np.ndarray:
    """Quantise float32 `x` to signed E4M3FN bytes with a unit block scale: the code nearest
    to x / global (RNE, saturating at +-448; +0 for values that round to zero)."""
    y = np.asarray(x, dtype=np.float64) / float(global_scale)
    mag = encode_e4m3(np.abs(y))
    sign = (np.signbit(y) & (mag != 0)).astype(np.uint8) << 7
    return np.ascontiguousarray(mag | sign)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (RNE) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values straight to bf16 (RNE), with no float32 double rounding."""
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    m8 = np.rint(m * 256.0) / 256.0          # 8 significant bits, ties to even
    v = np.ldexp(m8, e).astype(np.float32)   # exact: 8 bits fit in float32
    return bf16_bits_from_f32(v)


# --------------------------------------------------------------------------
# Workload configurations
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload.

    `context` is either one length for every request or an inclusive
    (lo, hi) range drawn uniformly per request.
    """
    name: str
    batch: int
    rows: object                 # rows per request (1 = plain decode): an int, or (lo, hi) drawn per request
    q_heads: int
    kv_heads: int
    head_dim: int
    page_size: int
    context: object              # int or (lo, hi)
    topk: int
    window: int
    seed: int
    shuffled: bool = True        # random physical page ids (else identity)
    dup_key_frac: float = 0.0    # fraction of candidate pages given a copied index key
    dup_group: int = 8           # pages per copied-key group
    outlier_frac: float = 0.0    # fraction of K/V elements replaced by +-outlier
    outlier_value: float = 8.0
    invalid_frac: float = 0.0    # fraction of page-table entries set to -1
    k_global: float = 1.0
    v_global: float = 1.0
    max_pages: Optional[int] = None  # page-table stride; default = max pages per request
    kv_format: str = "nvfp4"     # "nvfp4": e2m1 codes + e4m3 block scales; "fp8": e4m3 bytes, unit scales

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # 1 row, 4/1 heads, d 64, 1024 tokens in 16 pages of 64, identity table.
    "tiny": Config("tiny", 1, 1, 4, 1, 64, 64, 1024, 4, 1, seed=0, shuffled=False),
    # 8 decode rows, 32/4 heads, d 128, 8K context, shuffled table.
    "decode_8k": Config("decode_8k", 8, 1, 32, 4, 128, 64, 8192, 16, 2, seed=1),
    # 16 requests x (1+3) causal verify rows, 32K context, 10% copied index keys.
    "mtp_verify_32k": Config("mtp_verify_32k", 16, 4, 32, 4, 128, 64, 32768, 32, 2, seed=2,
                             dup_key_frac=0.10),
    # 4 rows, 64/8 heads, 131K context in 128-token pages, 1% +-8.0 outliers.
    "long_131k": Config("long_131k", 4, 1, 64, 8, 128, 128, 131072, 64, 1, seed=3,
                        outlier_frac=0.01),
    # a context step: 4 requests x 256 causal rows (the last 256 of 8K tokens), 32/4 heads,
    # d 128, each row selecting k 32 + W 2 of its pages.
    "context_8k": Config("context_8k", 4, 256, 32, 4, 128, 64, 8192, 32, 2, seed=5),
    # 48 requests x 4 rows, context U[1024, 65536], 5% invalid page-table entries.
    "wide_mixed": Config("wide_mixed", 48, 4, 32, 4, 128, 64, (1024, 65536), 32, 2, seed=4,
                         invalid_frac=0.05),
}


@dataclasses.dataclass
class Workload:
    cfg: Config
    page_table: np.ndarray
    seq_lens: np.ndarray
    row_offsets: np.ndarray
    q: np.ndarray
    k_codes: np.ndarray
    k_scales: np.ndarray
    v_codes: np.ndarray
    v_scales: np.ndarray
    index_keys: np.ndarray

    # shape helpers ---------------------------------------------------------
    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def N(self) -> int:
        return int(self.row_offsets[-1])

    @property
    def MP(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def NP(self) -> int:
        return int(self.k_codes.shape[0])

    @property
    def max_rows(self) -> int:
        return int(np.max(np.diff(self.row_offsets))) if self.B else 0

    @property
    def sm_scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.cfg.head_dim)))

    def digest(self) -> str:
        """SHA-256 over every generated array, in a fixed order."""
        h = hashlib.sha256()
        for a in (self.page_table, self.seq_lens, self.row_offsets, self.q, self.k_codes,
                  self.k_scales, self.v_codes, self.v_scales, self.index_keys):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


CHUNK_PAGES = 256   # physical pages per independently seeded K/V chunk (part of the recipe)


def _fill_chunk(args):
    (seq_child, c0, c1, cfg, valid_tokens, k_codes, k_scales, v_codes, v_scales, index_keys) = args
    rng = np.random.Generator(np.random.PCG64(seq_child))
    Hkv, P, d = cfg.kv_heads, cfg.page_size, cfg.head_dim
    live = np.arange(P)[None, :] < valid_tokens[c0:c1, None]                  # [C][P]
    for which in ("k", "v"):
        x = rng.standard_normal((c1 - c0, Hkv, P, d), dtype=np.float32)
        if cfg.outlier_frac > 0:
            cnt = int(round(cfg.outlier_frac * x.size))
            pos = rng.integers(0, x.size, size=cnt)
            sgn = np.where(rng.integers(0, 2, size=cnt) == 1, 1.0, -1.0).astype(np.float32)
            x.reshape(-1)[pos] = sgn * np.float32(cfg.outlier_value)
        x *= live[:, None, :, None]                                          # tokens past L_b are zero
        gs = cfg.k_global if which == "k" else cfg.v_global
        if cfg.kv_format == "fp8":
            codes, scales = encode_fp8(x, gs), np.zeros(x.shape[:-1] + (0,), np.uint8)
        else:
            codes, scales = encode_nvfp4(x, gs)
        if which == "k":
            k_codes[c0:c1], k_scales[c0:c1] = codes, scales
            cnt_t = np.maximum(valid_tokens[c0:c1], 1).astype(np.float64)
            mean = np.sum(x, axis=2, dtype=np.float64) / cnt_t[:, None, None]
            index_keys[c0:c1] = _bf16_bits_from_f64(mean)
        else:
            v_codes[c0:c1], v_scales[c0:c1] = codes, scales


def generate(cfg, threads: Optional[int] = None) -> Workload:
    """Build the seeded workload for `cfg` (a Config or the name of one in CONFIGS).

    The result depends only on `cfg`: K/V chunks are drawn from child seeds of
    `cfg.seed`, so the thread count does not change a single byte.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    root = np.random.SeedSequence(cfg.seed)
    meta_seed, kv_seed = root.spawn(2)
    rng = np.random.Generator(np.random.PCG64(meta_seed))
    B, Hq, Hkv, d, P = cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.page_size
    assert d % 16 == 0 and Hq % Hkv == 0
    # rows per request: fixed, or drawn per request from a child seed of its own (so fixed-row
    # workloads draw exactly what they always did)
    if isinstance(cfg.rows, (tuple, list)):
        (rows_seed,) = root.spawn(1)
        lo_r, hi_r = cfg.rows
        rows_b = np.random.Generator(np.random.PCG64(rows_seed)).integers(lo_r, hi_r, size=B,
                                                                          endpoint=True).astype(np.int32)
    else:
        rows_b = np.full(B, int(cfg.rows), dtype=np.int32)

    # context lengths (include this step's R rows)
    if isinstance(cfg.context, (tuple, list)):
        lo, hi = cfg.context
        seq = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    else:
        seq = np.full(B, int(cfg.context), dtype=np.int32)
    seq = np.maximum(seq, rows_b)                  # a request holds at least its own rows
    n_pages = (seq.astype(np.int64) + P - 1) // P
    MP = int(cfg.max_pages) if cfg.max_pages is not None else int(max(1, n_pages.max(initial=0)))
    assert MP >= n_pages.max(initial=0)
    NP = int(n_pages.sum())

    # page table: request b's logical pages map to a slice of a permutation of [0, NP)
    phys = rng.permutation(NP).astype(np.int32) if cfg.shuffled else np.arange(NP, dtype=np.int32)
    page_table = np.full((B, MP), -1, dtype=np.int32)
    owner_req = np.zeros(NP, dtype=np.int64)      # physical page -> request
    owner_lp = np.zeros(NP, dtype=np.int64)       # physical page -> logical page
    start = 0
    for b in range(B):
        n = int(n_pages[b])
        ids = phys[start:start + n]
        page_table[b, :n] = ids
        owner_req[ids] = b
        owner_lp[ids] = np.arange(n)
        start += n
    if cfg.invalid_frac > 0:
        for b in range(B):
            n = int(n_pages[b])
            m = int(round(cfg.invalid_frac * n))
            if m:
                page_table[b, rng.choice(n, size=m, replace=False)] = -1

    row_offsets = np.concatenate([[0], np.cumsum(rows_b)]).astype(np.int32)
    N = int(row_offsets[-1])
    q = bf16_bits_from_f32(rng.standard_normal((N, Hq, d), dtype=np.float32))

    # K / V pages in physical-page order, one child seed per chunk
    assert cfg.kv_format in ("nvfp4", "fp8")
    fp8 = cfg.kv_format == "fp8"
    k_codes = np.empty((NP, Hkv, P, d if fp8 else d // 2), np.uint8)
    v_codes = np.empty((NP, Hkv, P, d if fp8 else d // 2), np.uint8)
    k_scales = np.empty((NP, Hkv, P, 0 if fp8 else d // 16), np.uint8)
    v_scales = np.empty((NP, Hkv, P, 0 if fp8 else d // 16), np.uint8)
    index_keys = np.empty((NP, Hkv, d), np.uint16)
    valid_tokens = np.minimum(P, seq[owner_req].astype(np.int64) - owner_lp * P)  # per physical page
    starts = list(range(0, NP, CHUNK_PAGES))
    children = kv_seed.spawn(len(starts))
    jobs = [(children[i], c0, min(NP, c0 + CHUNK_PAGES), cfg, valid_tokens, k_codes, k_scales,
             v_codes, v_scales, index_keys) for i, c0 in enumerate(starts)]
    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads > 1 and len(jobs) > 1:
        with concurrent.futures.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(_fill_chunk, jobs))
    else:
        for j in jobs:
            _fill_chunk(j)

    # copied index keys: groups of candidate pages share one source page's key
    if cfg.dup_key_frac > 0:
        for b in range(B):
            r_b = int(rows_b[b])
            n_min = -(-max(0, int(seq[b]) - r_b + 1) // P)            # pages of the shortest row
            cand = [p for p in range(max(0, n_min - cfg.window)) if page_table[b, p] >= 0]
            m = int(round(cfg.dup_key_frac * len(cand)))
            if m < 2:
                continue
            order = rng.permutation(len(cand))
            n_groups = max(1, m // cfg.dup_group)
            srcs = [cand[i] for i in order[:n_groups]]
            copies = [cand[i] for i in order[n_groups:n_groups + m]]
            for j, p in enumerate(copies):
                index_keys[page_table[b, p]] = index_keys[page_table[b, srcs[j % n_groups]]]

    return Workload(cfg, page_table, seq, row_offsets, q, k_codes, k_scales, v_codes, v_scales,
                    index_keys)
