// qsa_select.hip -- canonical top-k page selection plus local window.
//
// Method: TensorRT-LLM PR #20276, Features, "Canonical QSA selection". The selection row is
// a pure function of the scores, the window and k: every block strictly above the k-th
// score, with ties going to the highest index. "Decisions worth knowing" adds that a radix
// top-k whose result follows launch order is not acceptable.
//
// Design for gfx950: one wave per query row, with no LDS and no barrier. Lane l holds the
// row's columns l*C .. l*C + C - 1 (C = MP/64 rounded up to 8, 16, 32 or 64) as
// order-preserving uint32 keys in registers, so lane-major order is ascending page order.
//  1. Non-candidates get key 0 (every candidate key is >= 0x00800000).
//  2. The k-th largest key T is found bit by bit, most significant first: a bit is kept
//     when at least k keys are >= the prefix with that bit set. Each count is a ballot per
//     register slot and a scalar popcount, so it does not depend on any schedule.
//  3. Keys above T are all taken. Of the keys equal to T, the highest page indices fill
//     the remaining slots, ranked by a wave suffix count of ties.
//  4. The union with the window is compacted in ascending page order by a wave prefix
//     sum, then padded with -1.
// So the output is a function of the scores alone.
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

template <int C>
__global__ __launch_bounds__(64) void select_topk_kernel(SelectParams prm)
{
    const int j = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x;
    const int r0 = prm.row_offsets[b], r1 = prm.row_offsets[b + 1];
    const int R = clip_rows(r0, r1, prm.N, prm.rmax, prm.err, j == 0 && lane == 0);
    if (j >= R) return;
    const int row = r0 + j;
    const int MP = prm.MP, KW = prm.k + prm.W;
    const RowGeom geo = row_geom(prm.seq_lens[b], r1 - r0, j, prm.log2P, MP);
    const int n = geo.pages;
    const int wlo = n - prm.W > 0 ? n - prm.W : 0;
    const int c0 = lane * C;

    // 1. keys; 0 marks a non-candidate
    uint32_t key[C];
    const float *srow = prm.scores + (int64_t)row * MP;
    if ((MP & 3) == 0 && c0 + C <= MP) {
#pragma unroll
        for (int i = 0; i < C; i += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(srow + c0 + i);
            key[i] = __float_as_uint(v.x); key[i + 1] = __float_as_uint(v.y);
            key[i + 2] = __float_as_uint(v.z); key[i + 3] = __float_as_uint(v.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < C; ++i) key[i] = c0 + i < MP ? __float_as_uint(srow[c0 + i]) : 0u;
    }
    uint32_t ncand = 0;
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int p = c0 + i;
        const float s = __uint_as_float(key[i]);
        key[i] = (p < wlo && !(s != s) && s != -__builtin_inff()) ? float_order_key(s) : 0u;
        ncand += (uint32_t)__builtin_popcountll(__ballot(key[i] != 0u));
    }

    // 2. the k-th largest key T; keys above T are all taken, and krem of the keys equal
    //    to T (with krem = 0 no tie rule applies)
    const uint32_t k = (uint32_t)prm.k;
    uint32_t T, krem = 0u;
    if (k == 0) {
        T = 0xffffffffu;                  // no key is above it: the window only
    } else if (ncand <= k) {
        T = 0u;                           // every candidate (key > 0) is taken
    } else {
        T = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t t = T | (1u << bit);
            uint32_t cnt = 0;
#pragma unroll
            for (int i = 0; i < C; ++i) cnt += (uint32_t)__builtin_popcountll(__ballot(key[i] >= t));
            if (cnt >= k) T = t;
        }
        uint32_t ngt = 0;
#pragma unroll
        for (int i = 0; i < C; ++i) ngt += (uint32_t)__builtin_popcountll(__ballot(key[i] > T));
        krem = k - ngt;                   // >= 1
    }

    // 3. ties at T go to the highest pages: rank each tie by the ties at higher pages (later
    //    lanes, then later slots of this lane)
    uint32_t eq_lane = 0;
#pragma unroll
    for (int i = 0; i < C; ++i) eq_lane += (krem != 0u && key[i] == T) ? 1u : 0u;
    const uint32_t eq_incl = wave_inclusive_scan(eq_lane);
    uint32_t higher = (uint32_t)__shfl((int)eq_incl, 63, 64) - eq_incl;
    uint64_t take = 0;                    // bit i: column c0 + i is in the row's selection
#pragma unroll
    for (int i = C - 1; i >= 0; --i) {
        const int p = c0 + i;
        bool t = key[i] > T;
        if (krem != 0u && key[i] == T) {
            t = higher < krem;
            ++higher;
        }
        if (p >= wlo && p < n) t = true;  // the window is always kept
        if (t) take |= 1ull << i;
    }

    // 4. ascending compaction, then -1 padding
    int32_t *dst = prm.selected + (int64_t)row * KW;
    const uint32_t cnt_lane = (uint32_t)__builtin_popcountll(take);
    const uint32_t incl = wave_inclusive_scan(cnt_lane);
    const uint32_t total = (uint32_t)__shfl((int)incl, 63, 64);
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

hipError_t launch_select_topk(const SelectParams &prm, int B, hipStream_t stream)
{
    dim3 grid(prm.rmax, B);
    if (prm.MP <= 512)
        select_topk_kernel<8><<<grid, 64, 0, stream>>>(prm);
    else if (prm.MP <= 1024)
        select_topk_kernel<16><<<grid, 64, 0, stream>>>(prm);
    else if (prm.MP <= 2048)
        select_topk_kernel<32><<<grid, 64, 0, stream>>>(prm);
    else
        select_topk_kernel<64><<<grid, 64, 0, stream>>>(prm);
    return hipGetLastError();
}

}  // namespace qsa
