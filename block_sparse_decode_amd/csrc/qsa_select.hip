// qsa_select.hip -- canonical top-k page selection plus local window (the separate call).
//
// Method: TensorRT-LLM PR #20276, Features, "Canonical QSA selection", and Decisions worth
// knowing. One wave per query row runs select_row (qsa_select_row.hpp).
#include "qsa_device.hpp"
#include "qsa_internal.hpp"
#include "qsa_select_row.hpp"

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
    const RowGeom geo = row_geom(prm.seq_lens[b], r1 - r0, j, prm.log2P, prm.MP);
    select_row<C>(prm.scores + (int64_t)row * prm.MP, prm.MP, geo.pages, prm.k, prm.W,
                         prm.selected + (int64_t)row * (prm.k + prm.W));
}

hipError_t launch_select_topk(const SelectParams &prm, int B, hipStream_t stream)
{
    dim3 grid(prm.rmax, B);
    if (prm.MP <= 128)
        select_topk_kernel<2><<<grid, 64, 0, stream>>>(prm);
    else if (prm.MP <= 256)
        select_topk_kernel<4><<<grid, 64, 0, stream>>>(prm);
    else if (prm.MP <= 512)
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
