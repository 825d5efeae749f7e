// qsa_select_row.hpp -- canonical top-k plus window of one query row, by one wave.
//
// Method: TensorRT-LLM PR #20276, Features, "Canonical QSA selection" row, and Decisions worth
// knowing. The rule: a row's selection depends on its scores, W and k alone. Candidates whose
// score exceeds the k-th largest are kept; among candidates equal to that value, the larger
// page index is ranked first; and no launch order may change the result. Shared by the select
// kernel and the attention kernel's fused selection.
//
// One wave, no LDS, no barrier. Lane l holds columns l*C .. l*C + C - 1 (C >= MP/64) as
// order-preserving uint32 keys in registers, so lane-major order is ascending page order.
//  1. Non-candidates get key 0 (every candidate key is >= 0x00800000).
//  2. The k-th largest key T is found bit by bit, most significant first: a bit is kept
//     when at least k keys are >= the prefix with that bit set. Each count is a ballot per
//     register slot and a scalar popcount, exact in any order. The search starts at the
//     highest bit in which the candidates differ (the bits above it are common to all of
//     them, so T has them too), and stops early when exactly k keys are >= the prefix:
//     those k keys are then the top k, with no tie across the boundary. A search still
//     running after kRederiveStep steps (in practice a row with several keys equal to the
//     k-th) takes the common bits of the keys left in its interval in one step the same way,
//     and ends there when they are all equal.
//  3. Keys above T are all taken. Of the keys equal to T, the highest page indices fill
//     the remaining slots, ranked by a wave suffix count of ties.
//  4. The union with the window is compacted in ascending page order by a wave prefix
//     sum, then padded with -1.
// So the output is a function of the scores alone.
#pragma once

#include "qsa_device.hpp"

// Phase stamps of a traced build (see qsa_decode.hip); nothing otherwise.
#ifndef QSA_SELECT_STAMP
#define QSA_SELECT_STAMP(k) ((void)0)
#endif

namespace qsa {

// Bit steps after which a search still running re-derives its interval's common bits (see
// select_row_take): on the workloads' score tables only rows with several keys equal to the
// k-th get that far (their search otherwise takes every remaining bit of that value, 27 steps
// on the 32K verify workload against at most 18 for the other rows).
constexpr int kRederiveStep = 16;

// Keys of the whole wave at or above t (wave-uniform): one ballot per register slot, all
// compares of a group of (up to) 8 slots issued before the first scalar popcount reads a mask,
// so their vector-to-scalar latencies overlap instead of adding up.
template <int C>
__device__ __forceinline__ uint32_t wave_count_ge(const uint32_t (&key)[C], uint32_t t)
{
    constexpr int GN = C < 8 ? C : 8;     // slots per group
    uint32_t c = 0;
#pragma unroll
    for (int g = 0; g < C; g += GN) {
        uint64_t m[GN];
#pragma unroll
        for (int i = 0; i < GN; ++i) m[i] = __ballot(key[g + i] >= t);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < GN; ++i) c += (uint32_t)__builtin_popcountll(m[i]);
    }
    return c;
}

// Bitwise AND / OR over the 64 lanes (all active): DPP within each 16-lane row (swap lane
// pairs, then pairs of pairs, then the mirrored half row and the mirrored row), then the
// four rows' results through readlane.
template <bool OR>
__device__ __forceinline__ uint32_t wave_bitreduce(uint32_t x)
{
    auto op = [](uint32_t a, uint32_t b) { return OR ? (a | b) : (a & b); };
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, true));    // quad_perm [1,0,3,2]
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, true));    // quad_perm [2,3,0,1]
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, true));   // row_half_mirror
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, true));   // row_mirror
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
    return op(op(r0, r1), op(r2, r3));
}

// The row's scores as raw bits, lane l holding columns l*C .. l*C + C - 1. Split from the
// selection itself so that a caller can issue these loads early; no value is used here, so
// every load issues before the first is waited on. A lane whose columns all lie in the row
// takes them in 16-byte loads when the rows are 16-byte aligned (C/4 loads instead of C: on
// the 32K verify workload the fused launch's prologue got 0.5 us shorter); otherwise one load
// per column, with the address clamped into the row. Columns past the row are never
// candidates (they lie past the row's pages), so their values are never read.
template <int C>
__device__ __forceinline__ void select_row_load(const float *srow, int MP, uint32_t (&key)[C])
{
    const int c0 = (threadIdx.x & 63) * C;
    if (C >= 4 && (MP & 3) == 0 && c0 + C <= MP) {
        // the lane's columns in 16-byte loads (the row starts 16-byte aligned when MP is a
        // multiple of 4: the score table itself is)
        const uint4 *v = reinterpret_cast<const uint4 *>(srow + c0);
#pragma unroll
        for (int j = 0; j < C / 4; ++j) {
            const uint4 t = v[j];
            key[4 * j] = t.x;
            key[4 * j + 1] = t.y;
            key[4 * j + 2] = t.z;
            key[4 * j + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int c = c0 + i;
            key[i] = __float_as_uint(srow[c < MP ? c : 0]);
        }
    }
}

// The selection from the loaded score bits, as a mask per lane: bit i set when column
// lane * C + i is selected. n: the row's visible pages. (`key` is overwritten.)
template <int C>
__device__ __forceinline__ uint64_t select_row_take(uint32_t (&key)[C], int n, int k_, int W)
{
    const int lane = threadIdx.x & 63;
    const int wlo = n - W > 0 ? n - W : 0;
    const int c0 = lane * C;

    // 1. keys; 0 marks a non-candidate
    // (class mask 0x007: signaling NaN, quiet NaN, -inf)
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int p = c0 + i;
        const float s = __uint_as_float(key[i]);
        key[i] = (p < wlo && !__builtin_amdgcn_class(s, 0x007)) ? float_order_key(s) : 0u;
    }
    const uint32_t ncand = wave_count_ge<C>(key, 1u);
    QSA_SELECT_STAMP(2);

    // 2. the k-th largest key T; keys above T are all taken, and krem of the keys equal
    //    to T (with krem = 0 no tie rule applies)
    // k in a register the compiler may not re-derive: under scalar-register pressure it would
    // otherwise reload it from the kernel arguments (and wait for the load) in every bit step
    uint32_t k = (uint32_t)k_;
    asm volatile("" : "+s"(k));
    uint32_t T, krem = 0u;
    if (k == 0) {
        T = 0xffffffffu;                  // no key is above it: the window only
    } else if (ncand <= k) {
        T = 0u;                           // every candidate (key > 0) is taken
    } else {
        // the bits above the highest one in which the candidates differ
        uint32_t kand = 0xffffffffu, kor = 0u;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            kand &= key[i] != 0u ? key[i] : 0xffffffffu;
            kor |= key[i];
        }
        kand = wave_bitreduce<false>(kand);
        kor = wave_bitreduce<true>(kor);
        const uint32_t diff = kand ^ kor;
        const int hb = diff != 0u ? 31 - __builtin_clz(diff) : -1;
        T = hb >= 0 ? kand & ~((2u << hb) - 1u) : kand;   // hb = -1: all candidates are equal
        // the loop state stays scalar: `left` counts the bits still to decide
        int left = hb + 1;
        uint32_t bitv = hb >= 0 ? 1u << hb : 0u;
        // at most kRederiveStep steps, then (a search still running) one re-derivation and the
        // remaining steps; `left` > 0 after a loop means it stopped at exactly k keys
        const int stop = left > kRederiveStep ? left - kRederiveStep : 0;
        bool exact = false;
        for (; left > stop; --left, bitv >>= 1) {
            const uint32_t t = T | bitv;
            const uint32_t c = wave_count_ge<C>(key, t);
            if (c >= k) T = t;
            if (c == k) {
                exact = true;
                break;
            }
        }
        if (!exact && left > 0) {
            // A row still searching here almost always has several keys equal to the k-th (no
            // prefix leaves exactly k keys at or above it), and the search would go on through
            // every remaining bit of that value. The k-th key lies in the interval
            // [T, T + 2 bitv): every key at or above T + 2 bitv is one of fewer than k, and at
            // least k are at or above T. So the bits in which the interval's keys agree are the
            // k-th key's, and the search restarts below the highest bit in which they differ,
            // as it started below the candidates' common bits (both counts stay as they were).
            // When they all agree the k-th key is their value.
            uint32_t iand = 0xffffffffu, ior = 0u;
#pragma unroll
            for (int i = 0; i < C; ++i) {
                const bool in = key[i] != 0u && key[i] >= T && ((key[i] - T) >> 1) < bitv;
                iand &= in ? key[i] : 0xffffffffu;
                ior |= in ? key[i] : 0u;
            }
            iand = wave_bitreduce<false>(iand);
            ior = wave_bitreduce<true>(ior);
            const uint32_t d = iand ^ ior;
            if (d == 0u) {
                T = iand;
                left = 0;
            } else {
                const int hb2 = 31 - __builtin_clz(d);
                T = iand & ~((2u << hb2) - 1u);
                left = hb2 + 1;
                bitv = 1u << hb2;
            }
            for (; left > 0; --left, bitv >>= 1) {
                const uint32_t t = T | bitv;
                const uint32_t c = wave_count_ge<C>(key, t);
                if (c >= k) T = t;
                if (c == k) break;
            }
        }
        if (left > 0) {
            T -= 1u;                      // the k keys >= the prefix are exactly the keys > T
        } else {
            const uint32_t ngt = wave_count_ge<C>(key, T + 1u);   // T < 2^32 - 1: T is a finite score's key
            krem = k - ngt;               // >= 1
        }
    }

    QSA_SELECT_STAMP(3);

    // 3. ties at T go to the highest pages: rank each tie by the ties at higher pages (later
    //    lanes, then later slots of this lane)
    uint64_t take = 0;                    // bit i: column c0 + i is in the row's selection
    if (krem == 0u) {
        // no tie at T: the keys above it (the common case, and the only one after an early
        // exit of the search)
#pragma unroll
        for (int i = 0; i < C; ++i) take |= (uint64_t)(key[i] > T) << i;
    } else {
        uint32_t eq_lane = 0;
#pragma unroll
        for (int i = 0; i < C; ++i) eq_lane += key[i] == T ? 1u : 0u;
        const uint32_t eq_incl = wave_inclusive_scan(eq_lane);
        uint32_t higher = (uint32_t)__builtin_amdgcn_readlane((int)eq_incl, 63) - eq_incl;
#pragma unroll
        for (int i = C - 1; i >= 0; --i) {
            bool t = key[i] > T;
            if (key[i] == T) {
                t = higher < krem;
                ++higher;
            }
            if (t) take |= 1ull << i;
        }
    }
    // the window [wlo, n) is always kept: this lane's columns lo .. hi - 1 of it
    const int lo = min(max(wlo - c0, 0), C), hi = min(max(n - c0, 0), C);
    take |= ((1ull << hi) - 1ull) & ~((1ull << lo) - 1ull);   // (C <= 32)

    return take;
}

// 4. ascending compaction of a selection mask into the row's KW = k + W slots, then -1
//    padding.
template <int C>
__device__ __forceinline__ void select_row_emit(uint64_t take, int KW, int32_t *dst)
{
    const int lane = threadIdx.x & 63;
    const int c0 = lane * C;
    const uint32_t cnt_lane = (uint32_t)__builtin_popcountll(take);
    const uint32_t incl = wave_inclusive_scan(cnt_lane);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    uint32_t pos = incl - cnt_lane;
#pragma unroll
    for (int i = 0; i < C; ++i) {
        if ((take >> i) & 1ull) {
            if (pos < (uint32_t)KW) dst[pos] = c0 + i;
            ++pos;
        }
    }
    for (int i = (int)total + lane; i < KW; i += 64) dst[i] = -1;
}

// The selection from the loaded score bits. n: the row's visible pages; dst: the row's
// k + W output slots.
template <int C>
__device__ __forceinline__ void select_row_keys(uint32_t (&key)[C], int n, int k_, int W, int32_t *dst)
{
    select_row_emit<C>(select_row_take<C>(key, n, k_, W), k_ + W, dst);
}

// srow: the row's MP scores; n: the row's visible pages; dst: the row's k + W output slots.
template <int C>
__device__ __forceinline__ void select_row(const float *srow, int MP, int n, int k_, int W, int32_t *dst)
{
    uint32_t key[C];
    select_row_load<C>(srow, MP, key);
    select_row_keys<C>(key, n, k_, W, dst);
}

}  // namespace qsa
