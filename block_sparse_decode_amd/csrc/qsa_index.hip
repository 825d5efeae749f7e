// qsa_index.hip -- per-page index scores for query-sparse decode / verify rows.
//
// Method: TensorRT-LLM PR #20276, "What runs on the fast paths" (index store and compression,
// then index scores, then the block top-k); PR #20937, MTP > Verify (request-tiled index
// scores). The score of page p for a row is sm_scale * max over q heads of q_h . key[p][h/G],
// each dot an fp32 sum taken in ascending element order.
//
// Design for gfx950. This stage feeds an exact integer decision (the top-k), so its fp32
// arithmetic must be reproducible bit for bit. It therefore runs on the plain ALUs, never
// on MFMA, whose internal summation order is not specified. Each lane owns one page and
// keeps that page's key in registers. The q row is wave-uniform, so it comes through scalar
// loads and feeds v_fma_f32 as an SGPR operand. A product of two bf16 values is exact in
// fp32, so the fma equals the separate multiply and add. Waves split the KV heads, and an
// LDS max combines them (max is exact in any order).
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

template <int D>
__global__ __launch_bounds__(256) void index_scores_kernel(IndexParams prm)
{
    constexpr int NW = 4;
    __shared__ float red[NW][kWave];

    const int tile = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = prm.row_offsets[b], r1 = prm.row_offsets[b + 1];
    const bool first = (j == 0 && tile == 0 && threadIdx.x == 0);
    const int R = clip_rows(r0, r1, prm.N, prm.rmax, prm.err, first);
    if (first && R > 0) {
        int64_t L_b = prm.seq_lens[b];
        if (L_b < r1 - r0 || L_b > (int64_t)prm.MP * prm.P) set_error(prm.err, QSA_DEVERR_SEQ_LEN);
    }
    if (j >= R) return;
    const int row = r0 + j;
    const RowGeom geo = row_geom(prm.seq_lens[b], r1 - r0, j, prm.log2P, prm.MP);

    const int p = tile * kWave + lane;
    int phys = -1;
    bool cand = false;
    if (p < prm.MP) {
        phys = prm.page_table[(int64_t)b * prm.MP + p];
        if (p < geo.pages && (phys < -1 || (int64_t)phys >= prm.NP)) set_error(prm.err, QSA_DEVERR_PAGE_ID);
        cand = (p < geo.pages - prm.W) && phys >= 0 && (int64_t)phys < prm.NP;
    }

    const int G = prm.Hq / prm.Hkv;
    float best = __builtin_nanf("");
    if (cand) {
        for (int g = wave; g < prm.Hkv; g += NW) {
            // this page's key for KV head g, as fp32 in registers
            float k[D];
            const uint4 *kp = reinterpret_cast<const uint4 *>(prm.keys + ((int64_t)phys * prm.Hkv + g) * D);
#pragma unroll
            for (int c = 0; c < D / 8; ++c) {
                uint4 v = kp[c];
                k[8 * c + 0] = bf16lo(v.x); k[8 * c + 1] = bf16hi(v.x);
                k[8 * c + 2] = bf16lo(v.y); k[8 * c + 3] = bf16hi(v.y);
                k[8 * c + 4] = bf16lo(v.z); k[8 * c + 5] = bf16hi(v.z);
                k[8 * c + 6] = bf16lo(v.w); k[8 * c + 7] = bf16hi(v.w);
            }
            for (int hh = 0; hh < G; ++hh) {
                const int h = g * G + hh;
                const uint32_t *qv = prm.q32 + ((int64_t)row * prm.Hq + h) * (D / 2);
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < D / 2; ++i) {
                    const uint32_t u = qv[i];                       // wave-uniform (scalar load)
                    acc = __builtin_fmaf(bf16lo(u), k[2 * i], acc);
                    acc = __builtin_fmaf(bf16hi(u), k[2 * i + 1], acc);
                }
                if (!(acc != acc) && ((best != best) || acc > best)) best = acc;
            }
        }
    }
    red[wave][lane] = best;
    __syncthreads();
    if (wave == 0 && p < prm.MP) {
        float m = red[0][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            float v = red[w][lane];
            if (!(v != v) && ((m != m) || v > m)) m = v;
        }
        float s = prm.sm_scale * m;
        if (s == 0.0f) s = 0.0f;                 // store +0 for either zero
        prm.scores[(int64_t)row * prm.MP + p] = cand ? s : -__builtin_inff();
    }
}

hipError_t launch_index_scores(const IndexParams &prm, int D, int B, hipStream_t stream)
{
    dim3 grid((prm.MP + kWave - 1) / kWave, prm.rmax, B);
    if (D == 64)
        index_scores_kernel<64><<<grid, 256, 0, stream>>>(prm);
    else
        index_scores_kernel<128><<<grid, 256, 0, stream>>>(prm);
    return hipGetLastError();
}

}  // namespace qsa
