// qsa_fastdiv.hpp -- the host half of the launches' constant-divisor division: the magic
// numbers FastDiv::make computes once per launch. Plain C++ (no HIP), so that a host-only
// build can check them; the kernels' fast_div is in qsa_internal.hpp.
#pragma once

#include <assert.h>
#include <stdint.h>

namespace qsa {

// Division by a divisor fixed for the whole launch, as a multiply and a shift (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, n / d = (umulhi(n, m) + n) >> l for
// every 0 <= n < 2^31 (the sum then fits 32 bits) and 1 <= d <= 2^31. The host fills it in;
// the divisors used (splits, column tiles, heads per KV head, k + W) are small.
struct FastDiv {
    uint32_t d, m, l;

    static FastDiv make(uint32_t d)
    {
        assert(d >= 1u && d <= 0x80000000u);
        FastDiv f;
        f.d = d;
        uint32_t l = 0;
        while (l < 31 && (1u << l) < d) ++l;
        f.l = l;
        f.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
        return f;
    }
};

}  // namespace qsa
