// qsa_rollback.hip -- the index-plane rollback of a verify step: the plane rows that the
// step's rows overwrite are gathered into a stash before the step and written back for the
// rejected rows afterwards; and the (page, slot) each step row occupies.
//
// Method: TensorRT-LLM PR #20937, Description > What changes > Rollback and PLE (the index
// planes' writes of rejected rows undone in one batch) and its file list (a gather and a
// restore operation for that rollback); the placement of a step row is the KV store's (the token at position
// L - R + j of its request).
//
// Design: pure data movement, a few hundred bytes per (row, plane). One 64-lane workgroup
// per (row, plane): the row's validity and the rejected flag are wave-uniform, and the
// lanes move its segments as 4-byte words (consecutive lanes, consecutive words of a
// segment). Rows of one plane are independent, so the launch has no ordering inside it.
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

template <bool RESTORE>
__global__ __launch_bounds__(64) void rollback_kernel(RollbackParams prm)
{
    const int r = blockIdx.x, k = blockIdx.y, lane = threadIdx.x;
    const PlaneDesc &pl = prm.planes[k];
    const int32_t page = prm.pages[r], slot = prm.within[r];
    if (page == -1) return;
    if (page < -1 || (int64_t)page >= pl.num_pages) {
        if (lane == 0) set_error(prm.err, QSA_DEVERR_PAGE_ID);
        return;
    }
    if (slot < 0 || slot >= pl.num_slots) {
        if (lane == 0) set_error(prm.err, QSA_DEVERR_SLOT);
        return;
    }
    if (RESTORE && prm.rejected[r] == 0) return;
    char *row = pl.base + (int64_t)page * pl.page_stride + (int64_t)slot * pl.slot_stride;
    const int sw = pl.seg_words;
    const int words = pl.nseg * sw;
    uint32_t *st = reinterpret_cast<uint32_t *>(prm.stash + pl.stash_off) + (int64_t)r * words;
    for (int w = lane; w < words; w += 64) {
        const int s = w / sw;
        uint32_t *at = reinterpret_cast<uint32_t *>(row + (int64_t)s * pl.seg_stride) + (w - s * sw);
        if constexpr (RESTORE)
            *at = st[w];
        else
            st[w] = *at;
    }
}

// one thread per request: its rows' (physical page, slot), as the KV store places them
__global__ __launch_bounds__(64) void step_slots_kernel(SlotParams prm, int B)
{
    const int b = blockIdx.x * 64 + threadIdx.x;
    if (b >= B) return;
    const int r0 = prm.row_offsets[b], r1 = prm.row_offsets[b + 1];
    const int R = clip_rows(r0, r1, prm.N, prm.rmax, prm.err, true);
    const int Rb = r1 - r0;
    const int64_t L = prm.seq_lens[b];
    for (int j = 0; j < R; ++j) {
        const int64_t pos = L - Rb + j;
        int32_t page = -1, slot = 0;
        if (pos >= 0 && pos / prm.P < prm.MP) {
            const int32_t ph = prm.page_table[(int64_t)b * prm.MP + pos / prm.P];
            if (ph >= 0 && (int64_t)ph < prm.NP) {
                page = ph;
                slot = (int32_t)(pos % prm.P);
            } else if (ph != -1) {
                set_error(prm.err, QSA_DEVERR_PAGE_ID);
            }
        } else {
            set_error(prm.err, QSA_DEVERR_SEQ_LEN);
        }
        prm.pages[r0 + j] = page;
        prm.within[r0 + j] = slot;
    }
}

hipError_t launch_rollback(const RollbackParams &prm, int num_planes, bool restore, hipStream_t stream)
{
    dim3 grid(prm.nrows, num_planes);
    if (restore)
        rollback_kernel<true><<<grid, 64, 0, stream>>>(prm);
    else
        rollback_kernel<false><<<grid, 64, 0, stream>>>(prm);
    return hipGetLastError();
}

hipError_t launch_step_slots(const SlotParams &prm, int B, hipStream_t stream)
{
    step_slots_kernel<<<(B + 63) / 64, 64, 0, stream>>>(prm, B);
    return hipGetLastError();
}

}  // namespace qsa
