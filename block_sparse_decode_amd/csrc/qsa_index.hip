// qsa_index.hip -- per-page index scores for query-sparse decode / verify rows.
//
// Method: TensorRT-LLM PR #20276, "What runs on the fast paths" (index store and compression,
// then index scores, then the block top-k); PR #20937, MTP > Verify (request-tiled index
// scores). The score of page p for a row is sm_scale * max over q heads of q_h . key[p][h/G],
// each dot an fp32 sum taken in ascending element order.
//
// Design for gfx950. This stage feeds an exact integer decision (the top-k), so its fp32
// arithmetic must be reproducible bit for bit. It therefore runs on the plain ALUs, never
// on MFMA, whose internal summation order is not specified. A workgroup covers 64 pages of
// one query row; each lane owns one page and keeps that page's key for the current KV head
// in VGPRs as fp32. Each wave takes KV heads in turn. The q heads of a KV head are
// wave-uniform: their bf16 pairs come through scalar loads and are unpacked on the scalar
// ALU, and four q heads are summed at once as four independent chains, each still one fp32
// fma after another in ascending element order. A product of two bf16 values is exact in
// fp32, so the fma equals the separate multiply and add. An LDS max over the waves combines
// the KV heads (max is exact in any order).
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

template <int D>
__global__ __launch_bounds__(256, 3) void index_scores_kernel(IndexParams prm)
{
    constexpr int NW = 4;
    __shared__ float red[NW][kWave];

    const int tile = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = prm.row_offsets[b], r1 = prm.row_offsets[b + 1];
    // Errors are reported at the end: a global atomic before the loop would keep the
    // compiler from reading q through the scalar cache.
    const bool first = (j == 0 && tile == 0 && threadIdx.x == 0);
    const int R = clip_rows(r0, r1, prm.N, prm.rmax, prm.err, false);
    if (j >= R) {
        if (first) clip_rows(r0, r1, prm.N, prm.rmax, prm.err, true);
        return;
    }
    const int row = r0 + j;
    const RowGeom geo = row_geom(prm.seq_lens[b], r1 - r0, j, prm.log2P, prm.MP);

    const int p = tile * kWave + lane;
    int phys = -1;
    bool cand = false, bad_page = false;
    if (p < prm.MP) {
        phys = prm.page_table[(int64_t)b * prm.MP + p];
        bad_page = p < geo.pages && (phys < -1 || (int64_t)phys >= prm.NP);
        cand = (p < geo.pages - prm.W) && phys >= 0 && (int64_t)phys < prm.NP;
    }
    const bool any_cand = __any(cand);

    const int G = prm.Hq / prm.Hkv;
    const int wv = __builtin_amdgcn_readfirstlane(wave);     // wave-uniform: q comes by scalar loads
    float best = __builtin_nanf("");
    for (int g = wv; g < prm.Hkv && any_cand; g += NW) {
        // this page's key for KV head g, as fp32 in registers
        float k[D];
        {
            const uint4 *kp = reinterpret_cast<const uint4 *>(prm.keys + ((int64_t)(cand ? phys : 0) * prm.Hkv + g) * D);
#pragma unroll
            for (int c = 0; c < D / 8; ++c) {
                const uint4 v = kp[c];
                k[8 * c + 0] = bf16lo(v.x); k[8 * c + 1] = bf16hi(v.x);
                k[8 * c + 2] = bf16lo(v.y); k[8 * c + 3] = bf16hi(v.y);
                k[8 * c + 4] = bf16lo(v.z); k[8 * c + 5] = bf16hi(v.z);
                k[8 * c + 6] = bf16lo(v.w); k[8 * c + 7] = bf16hi(v.w);
            }
        }
        // four q heads at a time, each its own sequential fp32 chain; their bf16 pairs are
        // wave-uniform, so they arrive in scalar registers and unpack on the scalar ALU
        for (int h4 = 0; h4 < G; h4 += 4) {
            const int nh = min(4, G - h4);
            const uint32_t *q0 = prm.q32 + ((int64_t)row * prm.Hq + g * G + h4) * (D / 2);
            const uint32_t *q1 = nh > 1 ? q0 + D / 2 : q0;
            const uint32_t *q2 = nh > 2 ? q0 + D : q0;
            const uint32_t *q3 = nh > 3 ? q0 + 3 * (D / 2) : q0;
            float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
            for (int i = 0; i < D / 2; ++i) {
                const uint32_t u0 = q0[i], u1 = q1[i], u2 = q2[i], u3 = q3[i];
                a0 = __builtin_fmaf(bf16lo(u0), k[2 * i], a0);
                a1 = __builtin_fmaf(bf16lo(u1), k[2 * i], a1);
                a2 = __builtin_fmaf(bf16lo(u2), k[2 * i], a2);
                a3 = __builtin_fmaf(bf16lo(u3), k[2 * i], a3);
                a0 = __builtin_fmaf(bf16hi(u0), k[2 * i + 1], a0);
                a1 = __builtin_fmaf(bf16hi(u1), k[2 * i + 1], a1);
                a2 = __builtin_fmaf(bf16hi(u2), k[2 * i + 1], a2);
                a3 = __builtin_fmaf(bf16hi(u3), k[2 * i + 1], a3);
            }
            const float acc[4] = {a0, a1, a2, a3};
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (t < nh && !(acc[t] != acc[t]) && ((best != best) || acc[t] > best)) best = acc[t];
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
    if (bad_page) set_error(prm.err, QSA_DEVERR_PAGE_ID);
    if (first) {
        clip_rows(r0, r1, prm.N, prm.rmax, prm.err, true);
        const int64_t L_b = prm.seq_lens[b];
        if (L_b < r1 - r0 || L_b > (int64_t)prm.MP * prm.P) set_error(prm.err, QSA_DEVERR_SEQ_LEN);
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
