// qsa_select.hip -- canonical top-k page selection plus local window.
//
// Method: TensorRT-LLM PR #20276, Features, "Canonical QSA selection". The selection row is
// a pure function of the scores, the window and k: every block strictly above the k-th
// score, with ties going to the highest index. "Decisions worth knowing" adds that a radix
// top-k whose result follows launch order is not acceptable.
//
// Design for gfx950: one workgroup (4 waves) per query row; the row's scores sit in LDS
// as order-preserving uint32 keys. A radix select over 8-bit digits, most significant
// first, finds the k-th largest key T. Digit histograms are LDS atomics, whose counts do
// not depend on order. Keys above T are all taken. Of the keys equal to T, the highest page
// indices fill the remaining slots, counted by a block suffix scan. The union with the
// window is marked in an LDS flag array and compacted in ascending page order by a
// block prefix sum. So the output is a function of the scores alone, whatever the
// schedule.
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

constexpr int kSelNT = 256;
constexpr int kSelMaxMP = 4096;

__global__ __launch_bounds__(kSelNT) void select_topk_kernel(SelectParams prm)
{
    __shared__ uint32_t keys[kSelMaxMP];
    __shared__ uint8_t flag[kSelMaxMP];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t scan_tmp[kSelNT / 64 + 1];
    __shared__ uint32_t bcast[4];

    const int j = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const int r0 = prm.row_offsets[b], r1 = prm.row_offsets[b + 1];
    const int R = clip_rows(r0, r1, prm.N, prm.rmax, prm.err, j == 0 && tid == 0);
    if (j >= R) return;
    const int row = r0 + j;
    const int MP = prm.MP, KW = prm.k + prm.W;
    const RowGeom geo = row_geom(prm.seq_lens[b], r1 - r0, j, prm.log2P, MP);
    const int n = geo.pages;
    const int wlo = n - prm.W > 0 ? n - prm.W : 0;
    const int C = (MP + kSelNT - 1) / kSelNT;          // columns per thread (contiguous)
    const int c0 = tid * C;

    // 1. keys; 0 marks a non-candidate (every candidate key is >= 0x00800000)
    uint32_t ncand_local = 0;
    for (int i = 0; i < C; ++i) {
        const int p = c0 + i;
        if (p >= MP) break;
        uint32_t key = 0;
        if (p < wlo) {
            const float s = prm.scores[(int64_t)row * MP + p];
            if (!(s != s) && s != -__builtin_inff()) key = float_order_key(s);
        }
        keys[p] = key;
        flag[p] = (p >= wlo && p < n) ? 1 : 0;            // the window is always kept
        ncand_local += key != 0;
    }
    uint32_t ncand;
    block_exclusive_scan<kSelNT>(ncand_local, scan_tmp, &ncand);   // also a barrier

    const uint32_t k = (uint32_t)prm.k;
    if (k == 0) {
        // window only
    } else if (ncand <= k) {
        for (int i = 0; i < C; ++i) {
            const int p = c0 + i;
            if (p < MP && keys[p] != 0) flag[p] = 1;
        }
    } else {
        // 2. radix select of the k-th largest key
        uint32_t prefix = 0, pmask = 0, krem = k;
        for (int shift = 24; shift >= 0; shift -= 8) {
            hist[tid] = 0;
            __syncthreads();
            for (int i = 0; i < C; ++i) {
                const int p = c0 + i;
                if (p >= MP) break;
                const uint32_t key = keys[p];
                if (key != 0 && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            // suffix sums over the 256 bins: bin t gets the count of digits >= t
            const uint32_t h = hist[255 - tid];
            uint32_t tot;
            const uint32_t before = block_exclusive_scan<kSelNT>(h, scan_tmp, &tot);
            // thread tid looks at bin d = 255 - tid: elements with digit > d number `before`
            if (before < krem && before + h >= krem) {
                bcast[0] = 255u - tid;
                bcast[1] = before;
            }
            __syncthreads();
            const uint32_t dstar = bcast[0], above = bcast[1];
            prefix |= dstar << shift;
            pmask |= 255u << shift;
            krem -= above;
            __syncthreads();
        }
        const uint32_t T = prefix;        // k-th largest key; `krem` of the keys == T are taken
        // 3. keys > T: all; keys == T: the `krem` highest page indices
        uint32_t eq_local = 0;
        for (int i = 0; i < C; ++i) {
            const int p = c0 + i;
            if (p < MP && keys[p] == T) ++eq_local;
        }
        // exclusive suffix count of ties in higher columns: scan over threads in reverse
        uint32_t eq_tot;
        const uint32_t eq_before_rev = block_exclusive_scan<kSelNT>(eq_local, scan_tmp, &eq_tot);
        uint32_t higher = eq_tot - eq_before_rev - eq_local;
        for (int i = C - 1; i >= 0; --i) {
            const int p = c0 + i;
            if (p >= MP) continue;
            const uint32_t key = keys[p];
            if (key > T) {
                flag[p] = 1;
            } else if (key == T && key != 0) {
                if (higher < krem) flag[p] = 1;
                ++higher;
            }
        }
    }
    __syncthreads();

    // 4. ascending compaction of the flagged pages, then -1 padding
    uint32_t cnt_local = 0;
    for (int i = 0; i < C; ++i) {
        const int p = c0 + i;
        if (p < MP) cnt_local += flag[p];
    }
    uint32_t total;
    uint32_t pos = block_exclusive_scan<kSelNT>(cnt_local, scan_tmp, &total);
    int32_t *dst = prm.selected + (int64_t)row * KW;
    for (int i = 0; i < C; ++i) {
        const int p = c0 + i;
        if (p < MP && flag[p]) {
            if (pos < (uint32_t)KW) dst[pos] = p;
            ++pos;
        }
    }
    for (int i = (int)total + tid; i < KW; i += kSelNT) dst[i] = -1;
}

hipError_t launch_select_topk(const SelectParams &prm, int B, hipStream_t stream)
{
    dim3 grid(prm.rmax, B);
    select_topk_kernel<<<grid, kSelNT, 0, stream>>>(prm);
    return hipGetLastError();
}

}  // namespace qsa
