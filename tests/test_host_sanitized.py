"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (gcc, CPU only).

* The constant-divisor division that every launch's work-item arithmetic uses: FastDiv::make
  (block_sparse_decode_amd/csrc/qsa_fastdiv.hpp, the host half; Granlund and Montgomery's
  method) computes (m, l) once per launch, and the kernels take n / d as
  (umulhi(n, m) + n) >> l for 0 <= n < 2^31. A C++ program built from that header checks the
  identity for every divisor up to 2^16 at the boundary numerators and for random divisors
  up to 2^31, with both sanitizers on and any report fatal.
* The C oracle, built with both sanitizers, runs its index scores, selection, attention,
  dequant and KV store on small workloads with -1 page-table entries, copied index keys and
  requests of 1 to 4 rows, in a child process that preloads the ASan runtime.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_decode_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not p or not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc's ASan runtime is not installed")
    return p


FASTDIV_CHECK = r'''
#include <stdio.h>
#include <stdlib.h>
#include "qsa_fastdiv.hpp"

static uint32_t quot(uint32_t n, qsa::FastDiv f)
{
    // the kernels' formula: (umulhi(n, m) + n) >> l
    const uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);
    return (hi + n) >> f.l;
}

static int check(uint32_t d, uint32_t n, qsa::FastDiv f)
{
    if (n >= 0x80000000u) return 0;
    if (quot(n, f) != n / d) {
        printf("mismatch d=%u n=%u got %u want %u\n", d, n, quot(n, f), n / d);
        return 1;
    }
    return 0;
}

int main(void)
{
    long checked = 0;
    int bad = 0;
    uint64_t s = 0x9e3779b97f4a7c15ull;
    for (uint32_t d = 1; d <= 65536u && !bad; ++d) {
        const qsa::FastDiv f = qsa::FastDiv::make(d);
        const uint32_t last = 0x7fffffffu;
        const uint32_t ns[] = {0u, 1u, d - 1u, d, d + 1u, 2u * d - 1u, 2u * d, last, last - 1u,
                               last - last % d, last - last % d - 1u};
        for (uint32_t n : ns) bad |= check(d, n, f), ++checked;
        for (int i = 0; i < 16; ++i) {
            s = s * 6364136223846793005ull + 1442695040888963407ull;
            const uint32_t n = (uint32_t)(s >> 33);
            bad |= check(d, n, f), ++checked;
            bad |= check(d, (n / d) * d, f), ++checked;
            bad |= check(d, (n / d) * d + d - 1u, f), ++checked;
        }
    }
    for (int i = 0; i < 200000 && !bad; ++i) {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        const uint32_t d = 1u + (uint32_t)(s >> 33);               // 1 .. 2^31
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        const uint32_t n = (uint32_t)(s >> 33);
        const qsa::FastDiv f = qsa::FastDiv::make(d);
        bad |= check(d, n, f), ++checked;
        bad |= check(d, (n / d) * d, f), ++checked;
        if ((n / d) * d >= 1u) bad |= check(d, (n / d) * d - 1u, f), ++checked;
    }
    const qsa::FastDiv top = qsa::FastDiv::make(0x80000000u);
    bad |= check(0x80000000u, 0x7fffffffu, top) | check(0x80000000u, 0u, top);
    printf("%s %ld\n", bad ? "FAIL" : "ok", checked);
    return bad;
}
'''


def test_fastdiv_magic_under_sanitizers(tmp_path):
    src = tmp_path / "fastdiv_check.cpp"
    src.write_text(FASTDIV_CHECK)
    exe = tmp_path / "fastdiv_check"
    subprocess.run(["g++", "-O1", "-std=c++17", *SAN, "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok") and "runtime error" not in r.stderr, r.stdout + r.stderr


ORACLE_RUN = textwrap.dedent('''
    import sys
    import numpy as np
    sys.path.insert(0, {root!r})
    import oracle, synth
    oracle.LIB_PATH = {lib!r}
    cfgs = [
        synth.Config("san_verify", 5, (1, 4), 16, 4, 64, 64, (60, 2000), 6, 2, seed=71, invalid_frac=0.15,
                     dup_key_frac=0.3),
        synth.Config("san_p128", 3, 2, 8, 2, 128, 128, (130, 3000), 5, 1, seed=72, invalid_frac=0.1),
        synth.Config("san_tiny", 1, 1, 4, 1, 64, 64, 1024, 4, 1, seed=73),
    ]
    for c in cfgs:
        w = synth.generate(c)
        s = oracle.index_scores(w)
        sel = oracle.select_w(w, s)
        out, lse = oracle.attention(w, sel)
        assert np.isfinite(out).all()
        oracle.rows(w.seq_lens, w.row_offsets, c.page_size, w.MP)
        pages = np.array([0, 1, w.k_codes.shape[0] - 1], np.int32)   # valid pages: the oracle's contract
        oracle.dequant_pages(w.k_codes, w.k_scales, 1.0, pages)
        if max(np.diff(w.row_offsets)) <= 4:
            rng = np.random.default_rng(c.seed)
            x = rng.standard_normal((w.N, c.kv_heads, c.head_dim)).astype(np.float32)
            nk = synth.bf16_bits_from_f32(x)
            oracle.kv_store(w, nk, nk)
    print("ok")
''')


def test_oracle_under_sanitizers(tmp_path):
    asan = _libasan()
    import oracle
    lib = tmp_path / "liboracle_san.so"
    flags = [f for f in oracle.GCC_FLAGS if f != "-O2"]
    subprocess.run(["gcc", "-O1", *flags, *SAN, "-o", str(lib), oracle.SRC_PATH, "-lm"], check=True)
    script = tmp_path / "run.py"
    script.write_text(ORACLE_RUN.format(root=ROOT, lib=str(lib)))
    env = dict(ENV, LD_PRELOAD=asan)
    r = subprocess.run([sys.executable, str(script)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.strip().endswith("ok") and "runtime error" not in r.stderr, r.stderr[-4000:]
