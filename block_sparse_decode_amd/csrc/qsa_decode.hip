// qsa_decode.hip -- split-KV sparse GQA attention over NVFP4 pages, with LSE merge.
//
// Method: TensorRT-LLM PR #20937, Description > What changes: NVFP4 sparse GQA decode as a
// split-K + merge kernel with a lean one-split variant, and a request-grouped verify kernel
// with a per-row merge. PR #20276, "What runs on the fast paths": K/V tiles are read once
// per group of rows of one request.
//
// Work item: (split s, KV head g, request b), one workgroup of 4 waves.
//  1. The rows of request b (1..4 causal verify rows) each list their selected pages. The
//     workgroup builds the union of those pages, each with a row bitmask, in ascending
//     page order in LDS, and drops entries whose page-table entry is -1. Each page of the
//     union is read once for all rows.
//  2. Split s takes a contiguous share of the union. Its waves take the pages round-robin
//     and run an online softmax over 32-token sub-chunks.
//       S^T = K Q^T   (16x16x32 f16 MFMA; A = K dequantised straight from the global loads,
//                      B = the request's q rows x G heads, 16 columns per tile)
//       O^T += V^T P^T (A = V^T read from LDS with ds_read_b64_tr_b16, B = P from the
//                      S^T accumulators, so P never leaves registers)
//     Each lane's columns mask tokens past its row's length (causal verify rows) and pages
//     its row did not select.
//  3. The waves merge in LDS in a fixed order. With one split the workgroup writes the
//     final bf16 output and the LSE. Otherwise it writes partials, and the merge kernel
//     combines the splits in ascending split order.
// NVFP4 -> f16 is exact (see nvfp4_dequant8). The global scales fold into the logit scale
// and the output.
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

constexpr int kMaxUnion = 1024;     // rows (<= 4) x (k + W) (<= 256)

__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct RawTile;   // one lane's share of a 16-token M-tile: its d/4 consecutive elements

template <>
struct RawTile<128> {
    uint4 codes;        // 32 e2m1 codes
    uint32_t scales;    // 2 e4m3 bytes in the low half
};

template <>
struct RawTile<64> {
    uint2 codes;        // 16 e2m1 codes
    uint32_t scales;    // 1 e4m3 byte
};

template <int D>
__device__ __forceinline__ RawTile<D> load_raw(const uint8_t *codes_tok, const uint8_t *scales_tok, int gq)
{
    RawTile<D> t;
    if constexpr (D == 128) {
        t.codes = *reinterpret_cast<const uint4 *>(codes_tok + gq * 16);
        t.scales = *reinterpret_cast<const uint16_t *>(scales_tok + gq * 2);
    } else {
        t.codes = *reinterpret_cast<const uint2 *>(codes_tok + gq * 8);
        t.scales = scales_tok[gq];
    }
    return t;
}

template <int D>
__device__ __forceinline__ uint32_t raw_dword(const RawTile<D> &t, int i)
{
    if constexpr (D == 128) {
        return i == 0 ? t.codes.x : i == 1 ? t.codes.y : i == 2 ? t.codes.z : t.codes.w;
    } else {
        return i == 0 ? t.codes.x : t.codes.y;
    }
}

// Dequantise a lane's 8-element group i (elements 8i..8i+7 of its d/4 chunk).
template <int D>
__device__ __forceinline__ f16x8 dequant_group(const RawTile<D> &t, int i)
{
    const uint32_t sb = (D == 128 && i >= 2) ? (t.scales >> 8) & 0xffu : t.scales & 0xffu;
    return nvfp4_dequant8(raw_dword<D>(t, i), e4m3_to_f16(sb));
}

template <int D, int NCT>
__global__ __launch_bounds__(kDecodeWaves * 64) void sparse_decode_kernel(DecodeParams prm)
{
    constexpr int NW = kDecodeWaves;
    constexpr int NT = NW * 64;
    constexpr int VROW = D + 16;            // padded LDS row of one V token (f16)
    constexpr int KS = D / 32;              // k-steps of S^T = K Q^T
    constexpr int DQ = D / 4;               // elements per lane group
    constexpr int NDT = D / 16;             // 16-row d tiles of O^T
    constexpr int NCOL = NCT * 16;
    static_assert(NCOL * D * 4 <= NW * 32 * VROW * 2, "merge buffer must fit the V staging area");

    __shared__ __attribute__((aligned(16))) half_t vsm[NW][32 * VROW];
    __shared__ uint32_t u_pm[kMaxUnion];    // page | row mask << 16
    __shared__ int32_t u_phys[kMaxUnion];
    __shared__ float ml_m[NW][NCOL];
    __shared__ float ml_l[NW][NCOL];
    __shared__ uint32_t scan_tmp[NT / 64 + 1];

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gq = lane >> 4, li = lane & 15;
    const int r0 = prm.row_offsets[b], r1 = prm.row_offsets[b + 1];
    const int R = clip_rows(r0, r1, prm.N, prm.rmax, prm.err, tid == 0 && s == 0 && g == 0);
    const int Rb = r1 - r0;         // the request's own row count fixes each row's length
    if (R <= 0) return;
    const int G = prm.Hq / prm.Hkv;
    const int MP = prm.MP, P = prm.P, KW = prm.KW;
    const int64_t Lb = prm.seq_lens[b];

    // ---- 1. union of the rows' selected pages --------------------------------------
    uint32_t *bm = reinterpret_cast<uint32_t *>(&vsm[0][0]);
    const int nwords = (MP + 3) / 4;
    for (int w = tid; w < nwords; w += NT) bm[w] = 0u;
    __syncthreads();
    for (int idx = tid; idx < R * KW; idx += NT) {
        const int j = idx / KW, e = idx - j * KW;
        const int p = prm.selected[(int64_t)(r0 + j) * KW + e];
        if (p < -1 || p >= MP) {
            set_error(prm.err, QSA_DEVERR_SELECTED);
            continue;
        }
        if (p < 0 || p >= row_geom(Lb, Rb, j, P, MP).pages) continue;   // no visible token
        const int phys = prm.page_table[(int64_t)b * MP + p];
        if (phys == -1) continue;
        if (phys < -1 || (int64_t)phys >= prm.NP) {
            set_error(prm.err, QSA_DEVERR_PAGE_ID);
            continue;
        }
        atomicOr(&bm[p >> 2], 1u << ((p & 3) * 8 + j));
    }
    __syncthreads();
    uint32_t U;
    {
        const int CW = (nwords + NT - 1) / NT;
        uint32_t cnt = 0;
        for (int w = tid * CW; w < (tid + 1) * CW && w < nwords; ++w) {
            const uint32_t x = bm[w];
            cnt += ((x & 0xffu) != 0) + ((x & 0xff00u) != 0) + ((x & 0xff0000u) != 0) + ((x >> 24) != 0);
        }
        uint32_t pos = block_exclusive_scan<NT>(cnt, scan_tmp, &U);
        for (int w = tid * CW; w < (tid + 1) * CW && w < nwords; ++w) {
            const uint32_t x = bm[w];
            for (int q = 0; q < 4; ++q) {
                const uint32_t m = (x >> (8 * q)) & 0xffu;
                if (m) u_pm[pos++] = (uint32_t)(4 * w + q) | (m << 16);
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < (int)U; e += NT) u_phys[e] = prm.page_table[(int64_t)b * MP + (u_pm[e] & 0xffffu)];

    // ---- 2. q operand and per-column bookkeeping ------------------------------------
    f16x8 qop[NCT][KS];
    int jcol[NCT];                  // row of this lane's column (R = padding column)
    uint32_t tile_rows[NCT];        // rows that a column tile touches
    bool qbad = false;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int col = ct * 16 + li;
        const int j = col / G;
        jcol[ct] = j < R ? j : R;
        uint32_t rows = 0;
        for (int jj = 0; jj < R; ++jj)
            if (jj * G < (ct + 1) * 16 && (jj + 1) * G > ct * 16) rows |= 1u << jj;
        tile_rows[ct] = rows;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            f16x8 v = {};
            if (j < R) {
                const int h = g * G + (col - j * G);
                const uint4 raw = *reinterpret_cast<const uint4 *>(
                    prm.q + ((int64_t)(r0 + j) * prm.Hq + h) * D + gq * DQ + ks * 8);
                const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float lo = bf16lo(w4[t]), hi = bf16hi(w4[t]);
                    qbad |= !(fabsf(lo) <= 65504.0f) || !(fabsf(hi) <= 65504.0f);
                    v[2 * t] = (half_t)lo;
                    v[2 * t + 1] = (half_t)hi;
                }
            }
            qop[ct][ks] = v;
        }
    }
    if (qbad) set_error(prm.err, QSA_DEVERR_Q_RANGE);
    __syncthreads();                 // u_phys ready; the bitmap area becomes V staging

    // ---- 3. online softmax over this wave's pages ---------------------------------
    const int S = prm.splits;
    const int e_lo = (int)(((int64_t)s * U) / S), e_hi = (int)(((int64_t)(s + 1) * U) / S);
    const float c1 = prm.qk_scale_log2;
    const float NEG_INF = -__builtin_inff();

    f32x4 oacc[NCT][NDT];
    float m_run[NCT], l_run[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        m_run[ct] = NEG_INF;
        l_run[ct] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[ct][dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    half_t *vs = &vsm[wave][0];
    const int64_t head_stride = (int64_t)P * (D / 2);       // codes bytes of one (page, KV head)
    const int64_t sc_stride = (int64_t)P * (D / 16);

    for (int e = e_lo + wave; e < e_hi; e += NW) {
        const uint32_t pm = __builtin_amdgcn_readfirstlane(u_pm[e]);
        const int phys = __builtin_amdgcn_readfirstlane(u_phys[e]);
        const int p = (int)(pm & 0xffffu);
        const uint32_t rmask = pm >> 16;
        const uint8_t *kc_page = prm.k_codes + ((int64_t)phys * prm.Hkv + g) * head_stride;
        const uint8_t *ks_page = prm.k_scales + ((int64_t)phys * prm.Hkv + g) * sc_stride;
        const uint8_t *vc_page = prm.v_codes + ((int64_t)phys * prm.Hkv + g) * head_stride;
        const uint8_t *vsc_page = prm.v_scales + ((int64_t)phys * prm.Hkv + g) * sc_stride;

        for (int c = 0; c < P / 32; ++c) {
            const int64_t tok0 = (int64_t)p * P + c * 32;
            // longest row of this page decides whether the sub-chunk has any visible token
            int64_t lmax = 0;
            for (int jj = 0; jj < R; ++jj)
                if ((rmask >> jj) & 1u) {
                    const int64_t L = row_geom(Lb, Rb, jj, P, MP).len;
                    lmax = L > lmax ? L : lmax;
                }
            if (lmax <= tok0) break;

            RawTile<D> kr[2], vr[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int t = c * 32 + mt * 16 + li;
                kr[mt] = load_raw<D>(kc_page + (int64_t)t * (D / 2), ks_page + (int64_t)t * (D / 16), gq);
                vr[mt] = load_raw<D>(vc_page + (int64_t)t * (D / 2), vsc_page + (int64_t)t * (D / 16), gq);
            }

            bool act[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) act[ct] = (rmask & tile_rows[ct]) != 0u;

            // S^T = K Q^T
            f32x4 sacc[2][NCT];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) sacc[mt][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const f16x8 a = dequant_group<D>(kr[mt], ks);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        if (act[ct])
                            sacc[mt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qop[ct][ks], sacc[mt][ct], 0, 0, 0);
                }
            }

            // V -> LDS, token-major rows of this 32-token sub-chunk
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int i = 0; i < DQ / 8; ++i) {
                    const f16x8 v = dequant_group<D>(vr[mt], i);
                    *reinterpret_cast<f16x8 *>(vs + (mt * 16 + li) * VROW + gq * DQ + i * 8) = v;
                }
            }
            wave_lds_fence();

            // online softmax; P stays in registers as the B operand of O^T += V^T P^T
            f16x8 pop[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                if (!act[ct]) continue;
                int lim = 0;
                const int j = jcol[ct];
                if (j < R && ((rmask >> j) & 1u)) {
                    const int64_t vis = row_geom(Lb, Rb, j, P, MP).len - tok0;
                    lim = vis <= 0 ? 0 : (vis >= 32 ? 32 : (int)vis);
                }
                float x[8];
                float mloc = NEG_INF;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = mt * 16 + gq * 4 + r;
                        const float v = (t < lim) ? sacc[mt][ct][r] * c1 : NEG_INF;
                        x[mt * 4 + r] = v;
                        mloc = fmaxf(mloc, v);
                    }
                mloc = max_across_groups(mloc);
                const float m_new = fmaxf(m_run[ct], mloc);
                const bool none = (m_new == NEG_INF);
                const float alpha = none ? 1.0f : __builtin_amdgcn_exp2f(m_run[ct] - m_new);
                float psum = 0.0f;
                f16x8 pv;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float pr = none ? 0.0f : __builtin_amdgcn_exp2f(x[i] - m_new);
                    psum += pr;
                    pv[i] = (half_t)pr;
                }
                pop[ct] = pv;
                l_run[ct] = l_run[ct] * alpha + psum;
                m_run[ct] = m_new;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) oacc[ct][dt] *= alpha;
            }

            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const half_t *a0 = vs + (4 * gq + (li >> 2)) * VROW + dt * 16 + 4 * (li & 3);
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(a0));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(a0 + 16 * VROW));
                const f16x8 a = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    if (act[ct])
                        oacc[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop[ct], oacc[ct][dt], 0, 0, 0);
            }
            wave_lds_fence();
        }
    }

    // ---- 4. merge the waves (fixed order), then write ------------------------------
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const float lt = sum_across_groups(l_run[ct]);
        if (gq == 0) {
            ml_m[wave][ct * 16 + li] = m_run[ct];
            ml_l[wave][ct * 16 + li] = lt;
        }
    }
    __syncthreads();
    float wgt[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int col = ct * 16 + li;
        float M = NEG_INF;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, ml_m[w][col]);
        wgt[ct] = (M == NEG_INF) ? 0.0f : __builtin_amdgcn_exp2f(m_run[ct] - M);
    }
    float *obuf = reinterpret_cast<float *>(&vsm[0][0]);    // [NCOL][D]
    for (int w = 0; w < NW; ++w) {
        if (wave == w) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int col = ct * 16 + li, d = dt * 16 + gq * 4 + r;
                        const float v = oacc[ct][dt][r] * wgt[ct];
                        float *dst = obuf + col * D + d;
                        *dst = (w == 0) ? v : *dst + v;
                    }
        }
        __syncthreads();
    }
    const int ncols = R * G < NCOL ? R * G : NCOL;
    for (int idx = tid; idx < ncols * (D / 4); idx += NT) {
        const int col = idx / (D / 4), d4 = idx - col * (D / 4);
        const int j = col / G, hh = col - j * G;
        const int row = r0 + j, head = g * G + hh;
        float M = NEG_INF;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, ml_m[w][col]);
        float L = 0.0f;
        if (M != NEG_INF)
            for (int w = 0; w < NW; ++w) L += ml_l[w][col] * __builtin_amdgcn_exp2f(ml_m[w][col] - M);
        const f32x4 o = *reinterpret_cast<const f32x4 *>(obuf + col * D + 4 * d4);
        if (S == 1) {
            uint2 packed;
            float lse_v;
            if (L > 0.0f) {
                const float sc = prm.v_global / L;
                packed.x = (uint32_t)f32_to_bf16_rne(o[0] * sc) | ((uint32_t)f32_to_bf16_rne(o[1] * sc) << 16);
                packed.y = (uint32_t)f32_to_bf16_rne(o[2] * sc) | ((uint32_t)f32_to_bf16_rne(o[3] * sc) << 16);
                lse_v = (M + __log2f(L)) * 0.69314718055994531f;
            } else {
                packed.x = packed.y = 0u;
                lse_v = NEG_INF;
            }
            *reinterpret_cast<uint2 *>(prm.out + ((int64_t)row * prm.Hq + head) * D + 4 * d4) = packed;
            if (d4 == 0 && prm.lse) prm.lse[(int64_t)row * prm.Hq + head] = lse_v;
        } else {
            const int64_t slot = ((int64_t)s * prm.N + row) * prm.Hq + head;
            *reinterpret_cast<f32x4 *>(prm.part_o + slot * D + 4 * d4) = o;
            if (d4 == 0) {
                prm.part_ml[slot * 2] = M;
                prm.part_ml[slot * 2 + 1] = L;
            }
        }
    }
}

// Combine the splits of every (row, q head): ascending split order, one thread per 4 outputs.
template <int D>
__global__ __launch_bounds__(256) void merge_splits_kernel(DecodeParams prm)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)prm.N * prm.Hq * (D / 4);
    if (idx >= total) return;
    const int64_t rh = idx / (D / 4);
    const int d4 = (int)(idx - rh * (D / 4));
    const int S = prm.splits;
    const int64_t stride = (int64_t)prm.N * prm.Hq;
    const float NEG_INF = -__builtin_inff();
    float M = NEG_INF;
    for (int s = 0; s < S; ++s) M = fmaxf(M, prm.part_ml[(s * stride + rh) * 2]);
    float L = 0.0f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (M != NEG_INF) {
        for (int s = 0; s < S; ++s) {
            const float m = prm.part_ml[(s * stride + rh) * 2];
            const float w = __builtin_amdgcn_exp2f(m - M);
            L += prm.part_ml[(s * stride + rh) * 2 + 1] * w;
            o += *reinterpret_cast<const f32x4 *>(prm.part_o + (s * stride + rh) * D + 4 * d4) * w;
        }
    }
    uint2 packed;
    float lse_v;
    if (L > 0.0f) {
        const float sc = prm.v_global / L;
        packed.x = (uint32_t)f32_to_bf16_rne(o[0] * sc) | ((uint32_t)f32_to_bf16_rne(o[1] * sc) << 16);
        packed.y = (uint32_t)f32_to_bf16_rne(o[2] * sc) | ((uint32_t)f32_to_bf16_rne(o[3] * sc) << 16);
        lse_v = (M + __log2f(L)) * 0.69314718055994531f;
    } else {
        packed.x = packed.y = 0u;
        lse_v = NEG_INF;
    }
    *reinterpret_cast<uint2 *>(prm.out + rh * D + 4 * d4) = packed;
    if (d4 == 0 && prm.lse) prm.lse[rh] = lse_v;
}

template <int D>
static hipError_t launch_decode_d(const DecodeParams &prm, int B, int nct, hipStream_t stream)
{
    dim3 grid(prm.splits, prm.Hkv, B);
    const int nt = kDecodeWaves * 64;
    switch (nct) {
    case 1: sparse_decode_kernel<D, 1><<<grid, nt, 0, stream>>>(prm); break;
    case 2: sparse_decode_kernel<D, 2><<<grid, nt, 0, stream>>>(prm); break;
    default: sparse_decode_kernel<D, 4><<<grid, nt, 0, stream>>>(prm); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || prm.splits == 1) return e;
    const int64_t total = (int64_t)prm.N * prm.Hq * (D / 4);
    if (total > 0) merge_splits_kernel<D><<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(prm);
    return hipGetLastError();
}

hipError_t launch_sparse_decode(const DecodeParams &prm, int D, int B, int ncol_tiles, hipStream_t stream)
{
    return D == 64 ? launch_decode_d<64>(prm, B, ncol_tiles, stream)
                   : launch_decode_d<128>(prm, B, ncol_tiles, stream);
}

// ---- parity hook: whole pages through the same decode as the attention kernel ----------
template <int D>
__global__ __launch_bounds__(256) void dequant_pages_kernel(DequantParams prm)
{
    // one thread per 8 consecutive elements of one token
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_page = (int64_t)prm.Hkv * prm.P * (D / 8);
    const int64_t total = per_page * prm.n;
    if (idx >= total) return;
    const int j = (int)(idx / per_page);
    const int64_t rem = idx - (int64_t)j * per_page;          // (h, t, group)
    const int64_t tok = rem / (D / 8);
    const int grp = (int)(rem - tok * (D / 8));
    const int phys = prm.pages[j];
    float *dst = prm.out + ((int64_t)j * prm.Hkv * prm.P + tok) * D + grp * 8;
    if (phys < 0 || (int64_t)phys >= prm.NP) {
        for (int i = 0; i < 8; ++i) dst[i] = __builtin_nanf("");
        return;
    }
    const int64_t base = (int64_t)phys * prm.Hkv * prm.P + tok;   // token index in the pool
    const uint32_t codes = *reinterpret_cast<const uint32_t *>(prm.codes + base * (D / 2) + grp * 4);
    const uint32_t sb = prm.scales[base * (D / 16) + grp / 2];
    const f16x8 v = nvfp4_dequant8(codes, e4m3_to_f16(sb));
    for (int i = 0; i < 8; ++i) dst[i] = (float)v[i] * prm.global;
}

hipError_t launch_dequant_pages(const DequantParams &prm, int D, hipStream_t stream)
{
    const int64_t total = (int64_t)prm.n * prm.Hkv * prm.P * (D / 8);
    if (total == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (D == 64)
        dequant_pages_kernel<64><<<blocks, 256, 0, stream>>>(prm);
    else
        dequant_pages_kernel<128><<<blocks, 256, 0, stream>>>(prm);
    return hipGetLastError();
}

}  // namespace qsa
