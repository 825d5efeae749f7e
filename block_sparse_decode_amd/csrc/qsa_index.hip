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
// in VGPRs as fp32. Each wave takes KV heads in turn. For its KV head it stages the group's
// q heads, 8 at a time, as fp32 in its own slice of LDS (converted once, instead of once per
// lane and use), and every lane reads them with broadcast LDS loads. Four q heads are summed
// at once as four independent chains, each still one fp32 fma after another in ascending
// element order; a product of two bf16 values is exact in fp32, so the fma equals the
// separate multiply and add. An LDS max over the waves combines the KV heads (max is exact
// in any order).
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

template <int D>
__global__ __launch_bounds__(256, 3) void index_scores_kernel(IndexParams prm)
{
    constexpr int NW = 4;
    constexpr int QH = 8;                    // q heads staged per wave at a time
    __shared__ float red[NW][kWave];
    __shared__ __attribute__((aligned(16))) float qs[NW][QH][D];

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
    const bool any_cand = __any(cand);

    const int G = prm.Hq / prm.Hkv;
    float *qw = &qs[wave][0][0];
    float best = __builtin_nanf("");
    for (int g = wave; g < prm.Hkv && any_cand; g += NW) {
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
        for (int hc = 0; hc < G; hc += QH) {
            const int nh = min(QH, G - hc);
            // stage q heads g*G + hc .. + nh of this row as fp32: lane handles QH * D / 64
            // consecutive elements of the chunk
            constexpr int EPL = QH * D / 64;            // elements per lane (16 or 8)
            const int e0 = lane * EPL;
            if (e0 < nh * D) {
                const uint4 *src = reinterpret_cast<const uint4 *>(
                    prm.q32 + ((int64_t)row * prm.Hq + g * G + hc) * (D / 2) + e0 / 2);
#pragma unroll
                for (int c = 0; c < EPL / 8; ++c) {
                    const uint4 v = src[c];
                    const float4 lo = make_float4(bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y));
                    const float4 hi = make_float4(bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w));
                    *reinterpret_cast<float4 *>(qw + e0 + 8 * c) = lo;
                    *reinterpret_cast<float4 *>(qw + e0 + 8 * c + 4) = hi;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): the wave's LDS stores are done
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            for (int h4 = 0; h4 < nh; h4 += 4) {
                const float *q0 = qw + (h4 + 0) * D, *q1 = qw + (h4 + 1) * D;
                const float *q2 = qw + (h4 + 2) * D, *q3 = qw + (h4 + 3) * D;
                float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
                for (int i = 0; i < D; i += 4) {
                    const float4 x0 = *reinterpret_cast<const float4 *>(q0 + i);
                    const float4 x1 = *reinterpret_cast<const float4 *>(q1 + i);
                    const float4 x2 = *reinterpret_cast<const float4 *>(q2 + i);
                    const float4 x3 = *reinterpret_cast<const float4 *>(q3 + i);
                    a0 = __builtin_fmaf(x0.x, k[i], a0); a1 = __builtin_fmaf(x1.x, k[i], a1);
                    a2 = __builtin_fmaf(x2.x, k[i], a2); a3 = __builtin_fmaf(x3.x, k[i], a3);
                    a0 = __builtin_fmaf(x0.y, k[i + 1], a0); a1 = __builtin_fmaf(x1.y, k[i + 1], a1);
                    a2 = __builtin_fmaf(x2.y, k[i + 1], a2); a3 = __builtin_fmaf(x3.y, k[i + 1], a3);
                    a0 = __builtin_fmaf(x0.z, k[i + 2], a0); a1 = __builtin_fmaf(x1.z, k[i + 2], a1);
                    a2 = __builtin_fmaf(x2.z, k[i + 2], a2); a3 = __builtin_fmaf(x3.z, k[i + 2], a3);
                    a0 = __builtin_fmaf(x0.w, k[i + 3], a0); a1 = __builtin_fmaf(x1.w, k[i + 3], a1);
                    a2 = __builtin_fmaf(x2.w, k[i + 3], a2); a3 = __builtin_fmaf(x3.w, k[i + 3], a3);
                }
                const float acc[4] = {a0, a1, a2, a3};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (h4 + t >= nh) break;
                    if (!(acc[t] != acc[t]) && ((best != best) || acc[t] > best)) best = acc[t];
                }
            }
            // the next chunk overwrites this wave's slice: every lane has read it
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
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
