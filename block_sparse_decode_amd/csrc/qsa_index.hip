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
// in VGPRs as fp32. Each wave takes KV heads in turn. The q heads of a KV head are staged
// per wave in LDS as fp32, eight heads per element, so one broadcast read (all lanes at one
// address) feeds eight fma chains, one per head, each still one fp32 fma after another in
// ascending element order. A product of two bf16 values is exact in fp32, so the fma equals
// the separate multiply and add. The loads that do not depend on each other (row offsets,
// the request's length, the page-table entries, q) are issued together at the start. An
// LDS max over the waves combines the KV heads (max is exact in any order).
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

constexpr int kIndexWaves = 4;
constexpr int kHeadGroup = 8;        // q heads per pass: one LDS row of 8 fp32 per element

template <int D>
__global__ __launch_bounds__(kIndexWaves * 64, 2) void index_scores_kernel(IndexParams prm)
{
    constexpr int NW = kIndexWaves;
    constexpr int HG = kHeadGroup;
    __shared__ float red[NW][kWave];
    __shared__ __align__(16) float qs[NW][D][HG];   // per wave: q[head][i] of one head group, element-major

    const int tile = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wv = __builtin_amdgcn_readfirstlane(wave);     // wave-uniform
    // independent loads first: the row range, the request's length and this lane's page
    const int r0 = prm.row_offsets[b], r1 = prm.row_offsets[b + 1];
    const int64_t L_b = prm.seq_lens[b];
    const int p = tile * kWave + lane;
    const int32_t phys = p < prm.MP ? prm.page_table[(int64_t)b * prm.MP + p] : -1;
    // errors are reported at the end, after the loop
    const bool first = (j == 0 && tile == 0 && threadIdx.x == 0);
    const int R = clip_rows(r0, r1, prm.N, prm.rmax, prm.err, false);
    if (j >= R) {
        if (first) clip_rows(r0, r1, prm.N, prm.rmax, prm.err, true);
        return;
    }
    const int row = r0 + j;
    const RowGeom geo = row_geom(L_b, r1 - r0, j, prm.log2P, prm.MP);
    bool cand = false, bad_page = false;
    if (p < prm.MP) {
        bad_page = p < geo.pages && (phys < -1 || (int64_t)phys >= prm.NP);
        cand = (p < geo.pages - prm.W) && phys >= 0 && (int64_t)phys < prm.NP;
    }
    const bool any_cand = __any(cand);

    const int G = prm.Hq / prm.Hkv;
    float(*qw)[HG] = qs[wv];
    float best = __builtin_nanf("");
    // q heads h0 .. h0 + nh - 1 of KV head g, as bf16 pairs: lane l holds elements 2l, 2l + 1
    // of every head (zeros past nh, and for lanes past d / 2)
    auto load_q = [&](int g, int h0, uint32_t (&qu)[HG]) {
        const int nh = min(HG, G - h0);
        const uint32_t *qb = prm.q32 + ((int64_t)row * prm.Hq + g * G + h0) * (D / 2) + lane;
#pragma unroll
        for (int t = 0; t < HG; ++t) qu[t] = (lane < D / 2 && t < nh) ? qb[t * (D / 2)] : 0u;
    };
    auto stage_q = [&](const uint32_t (&qu)[HG]) {
        if (lane < D / 2) {
            float4 *d0 = reinterpret_cast<float4 *>(qw[2 * lane]);
            float4 *d1 = reinterpret_cast<float4 *>(qw[2 * lane + 1]);
            d0[0] = make_float4(bf16lo(qu[0]), bf16lo(qu[1]), bf16lo(qu[2]), bf16lo(qu[3]));
            d0[1] = make_float4(bf16lo(qu[4]), bf16lo(qu[5]), bf16lo(qu[6]), bf16lo(qu[7]));
            d1[0] = make_float4(bf16hi(qu[0]), bf16hi(qu[1]), bf16hi(qu[2]), bf16hi(qu[3]));
            d1[1] = make_float4(bf16hi(qu[4]), bf16hi(qu[5]), bf16hi(qu[6]), bf16hi(qu[7]));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): this wave's q rows are in LDS
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // the eight chains over elements i0 .. i0 + 7, each in ascending element order
    auto chains8 = [&](const float (&k)[D], int i0, float (&a)[HG]) {
#pragma unroll
        for (int i = i0; i < i0 + 8; ++i) {
            const float4 qa = *reinterpret_cast<const float4 *>(&qw[i][0]);
            const float4 qb2 = *reinterpret_cast<const float4 *>(&qw[i][4]);
            a[0] = __builtin_fmaf(qa.x, k[i], a[0]);
            a[1] = __builtin_fmaf(qa.y, k[i], a[1]);
            a[2] = __builtin_fmaf(qa.z, k[i], a[2]);
            a[3] = __builtin_fmaf(qa.w, k[i], a[3]);
            a[4] = __builtin_fmaf(qb2.x, k[i], a[4]);
            a[5] = __builtin_fmaf(qb2.y, k[i], a[5]);
            a[6] = __builtin_fmaf(qb2.z, k[i], a[6]);
            a[7] = __builtin_fmaf(qb2.w, k[i], a[7]);
        }
    };
    auto fold = [&](const float (&a)[HG], int nh) {
#pragma unroll
        for (int t = 0; t < HG; ++t)
            if (t < nh && !(a[t] != a[t]) && ((best != best) || a[t] > best)) best = a[t];
    };

    for (int g = wv; g < prm.Hkv && any_cand; g += NW) {
        // q of the first head group, then this page's key for KV head g: every load is issued
        // before the first wait, and the q loads first, so waiting for q leaves the key loads
        // in flight (the memory counter is in order)
        uint32_t qu[HG];
        load_q(g, 0, qu);
        const uint4 *kp = reinterpret_cast<const uint4 *>(prm.keys + ((int64_t)(cand ? phys : 0) * prm.Hkv + g) * D);
        uint4 kraw[D / 8];
#pragma unroll
        for (int c = 0; c < D / 8; ++c) kraw[c] = kp[c];
        __builtin_amdgcn_sched_barrier(0);    // keep every key load ahead of the wait for q
        stage_q(qu);
        // first head group: each 8-element chunk of the key is converted to fp32 and used as
        // soon as it has arrived, while the later chunks are still in flight
        float k[D];
        float a[HG];
#pragma unroll
        for (int t = 0; t < HG; ++t) a[t] = 0.0f;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
            const uint4 v = kraw[c];
            k[8 * c + 0] = bf16lo(v.x); k[8 * c + 1] = bf16hi(v.x);
            k[8 * c + 2] = bf16lo(v.y); k[8 * c + 3] = bf16hi(v.y);
            k[8 * c + 4] = bf16lo(v.z); k[8 * c + 5] = bf16hi(v.z);
            k[8 * c + 6] = bf16lo(v.w); k[8 * c + 7] = bf16hi(v.w);
            chains8(k, 8 * c, a);
        }
        fold(a, min(HG, G));
        // further head groups reuse the converted key
        for (int h0 = HG; h0 < G; h0 += HG) {
            __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's reads of the previous group are done
            load_q(g, h0, qu);
            stage_q(qu);
#pragma unroll
            for (int t = 0; t < HG; ++t) a[t] = 0.0f;
#pragma unroll
            for (int c = 0; c < D / 8; ++c) chains8(k, 8 * c, a);
            fold(a, min(HG, G - h0));
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);       // reads done before the next KV head's staging
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
