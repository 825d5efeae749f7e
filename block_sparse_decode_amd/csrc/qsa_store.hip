// qsa_store.hip -- the KV-store prologue of a decode / verify step: this step's new K and V
// tokens quantised to NVFP4 into their page slots, and the index keys of the pages that
// received them recomputed.
//
// Method: TensorRT-LLM PR #20276, Performance > What runs on the fast paths (the decode
// prologue covers index store and compression); PR #20937, Description > What changes (a
// fused decode prologue over NVFP4 KV); PR #20276, Features, NVFP4 KV cache row (e2m1 codes
// and e4m3 block scales in parallel planes addressed by one page id). The pages fix neither
// the encoder's rounding nor the index compression; the definitions taken here:
//   placement  row j of a request with R rows and L tokens is the token at position
//              L - R + j: page (L - R + j) / P, slot (L - R + j) % P;
//   scale      per block of 16 elements: E4M3 nearest (ties to even) to
//              fl32(fl32(amax / 6) / global), at most 448;
//   codes      E2M1 nearest (ties to even) to fl32(x / (e4m3(scale) * global)), magnitude
//              at most 6, +0 for values that round to zero; all 0 when the scale is 0;
//   index key  per element: bf16_RNE(fl32(S / n)), S the fp32 sum in ascending token order
//              of the page's stored K (dequantised) over its n valid tokens.
//
// Design: one workgroup per (request, KV head). Phase 1: one thread per 16-element block of
// a new token (K or V): amax, scale and codes in registers, rounding by v_rndne on values
// scaled by exact powers of two. A workgroup barrier makes the new slots visible to the
// workgroup. Phase 2: one thread per (touched page, element) sums the page's dequantised K
// over its valid tokens and writes the key. Contraction is off in this file so that every
// fp32 sum and product is the rounded operation the definition states.
#pragma clang fp contract(off)

#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

// E4M3 code nearest to a non-negative fp32 value, ties to the even code, at most 0x7E (448).
__device__ __forceinline__ uint32_t e4m3_encode(float t)
{
    if (!(t < 448.0f)) return 0x7Eu;                      // 448 and above (and NaN guard)
    if (t < 0.015625f) {                                   // below 2^-6: subnormal step 2^-9
        return (uint32_t)__builtin_rintf(t * 512.0f);      // 0 .. 8 (8 is 2^-6, code 0x08)
    }
    const int e = (int)((__float_as_uint(t) >> 23) & 0xffu) - 127;      // -6 .. 8
    float m = __builtin_rintf(__builtin_ldexpf(t, 3 - e));              // 8 .. 16
    int ee = e;
    if (m == 16.0f) {
        m = 8.0f;
        ++ee;
    }
    const uint32_t code = (uint32_t)((ee + 7) << 3) | (uint32_t)(m - 8.0f);
    return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_value(uint32_t byte)
{
    const int e = (int)((byte >> 3) & 15u), m = (int)(byte & 7u);
    return e == 0 ? (float)m * 0.001953125f : __builtin_ldexpf(1.0f + (float)m * 0.125f, e - 7);
}

// E2M1 code nearest to an fp32 value, ties to the even code, magnitude at most 6.
__device__ __forceinline__ uint32_t e2m1_encode(float y)
{
    const float a = fabsf(y);
    uint32_t mag;
    if (!(a < 6.0f)) {
        mag = 7u;
    } else if (a < 1.0f) {
        mag = (uint32_t)__builtin_rintf(a * 2.0f);         // 0, 1 (0.5) or 2 (1.0)
    } else {
        const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // 0 .. 2
        float m = __builtin_rintf(__builtin_ldexpf(a, 1 - e));          // 2 .. 4
        int ee = e;
        if (m == 4.0f) {
            m = 2.0f;
            ++ee;
        }
        mag = ee > 2 ? 7u : (uint32_t)((ee + 1) << 1) | (uint32_t)(m - 2.0f);
    }
    return mag | ((y < 0.0f && mag != 0u) ? 8u : 0u);
}

__device__ __forceinline__ float e2m1_value(uint32_t c)
{
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const float v = e == 0 ? 0.5f * (float)m : __builtin_ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
    return (c & 8u) ? -v : v;
}

template <int D>
__global__ __launch_bounds__(256) void kv_store_kernel(StoreParams prm)
{
    const int b = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    const int r0 = prm.row_offsets[b], r1 = prm.row_offsets[b + 1];
    const int R = clip_rows(r0, r1, prm.N, prm.rmax, prm.err, g == 0 && tid == 0);
    if (R == 0) return;
    const int Rb = r1 - r0;
    const int64_t L = prm.seq_lens[b];
    const int P = prm.P, MP = prm.MP;
    constexpr int NB = D / 16;                              // blocks per token

    // ---- phase 1: quantise the new tokens' blocks (K then V) --------------------------
    for (int task = tid; task < 2 * R * NB; task += blockDim.x) {
        const bool is_v = task >= R * NB;
        const int w = is_v ? task - R * NB : task;
        const int j = w / NB, blk = w - j * NB;
        const int64_t pos = L - Rb + j;
        if (pos >= 0 && pos / P < MP) {
            const int32_t phys = prm.page_table[(int64_t)b * MP + pos / P];
            if (phys >= 0 && (int64_t)phys < prm.NP) {
                const uint16_t *src = (is_v ? prm.new_v : prm.new_k) + ((int64_t)(r0 + j) * prm.Hkv + g) * D + blk * 16;
                const uint4 lo = *reinterpret_cast<const uint4 *>(src);
                const uint4 hi = *reinterpret_cast<const uint4 *>(src + 8);
                const uint32_t u[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                float x[16];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    x[2 * i] = bf16lo(u[i]);
                    x[2 * i + 1] = bf16hi(u[i]);
                }
                float amax = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
                const float global = is_v ? prm.v_global : prm.k_global;
                const uint32_t sc = e4m3_encode((amax / 6.0f) / global);
                const float s = e4m3_value(sc) * global;
                uint32_t w0 = 0u, w1 = 0u;
                if (s != 0.0f) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) w0 |= e2m1_encode(x[i] / s) << (4 * i);
#pragma unroll
                    for (int i = 0; i < 8; ++i) w1 |= e2m1_encode(x[8 + i] / s) << (4 * i);
                }
                const int64_t tok = ((int64_t)phys * prm.Hkv + g) * P + pos % P;
                uint8_t *codes = (is_v ? prm.v_codes : prm.k_codes) + tok * (D / 2) + blk * 8;
                *reinterpret_cast<uint2 *>(codes) = make_uint2(w0, w1);
                (is_v ? prm.v_scales : prm.k_scales)[tok * (D / 16) + blk] = (uint8_t)sc;
            } else if (phys != -1) {
                set_error(prm.err, QSA_DEVERR_PAGE_ID);
            }
        } else if (g == 0 && blk == 0 && !is_v) {
            set_error(prm.err, QSA_DEVERR_SEQ_LEN);
        }
    }
    __syncthreads();               // the new slots are visible to the whole workgroup

    // ---- phase 2: index keys of the touched pages --------------------------------------
    const int64_t first_pos = L - Rb > 0 ? L - Rb : 0;
    const int64_t last_pos = L - Rb + R - 1;
    if (last_pos < 0) return;
    const int64_t p_lo = first_pos / P, p_hi = last_pos / P;      // at most 2 pages for R <= 4 <= P
    for (int task = tid; task < (int)(p_hi - p_lo + 1) * D; task += blockDim.x) {
        const int64_t page = p_lo + task / D;
        const int i = task % D;
        if (page >= MP) continue;
        const int32_t phys = prm.page_table[(int64_t)b * MP + page];
        if (phys < 0 || (int64_t)phys >= prm.NP) continue;
        const int64_t n = L - page * P < P ? L - page * P : P;
        const int64_t head = (int64_t)phys * prm.Hkv + g;
        float S = 0.0f;
        for (int64_t t = 0; t < n; ++t) {
            const int64_t tok = head * P + t;
            const uint32_t byte = prm.k_codes[tok * (D / 2) + i / 2];
            const uint32_t c = (i & 1) ? (byte >> 4) : (byte & 15u);
            const float v = (e2m1_value(c) * e4m3_value(prm.k_scales[tok * (D / 16) + i / 16])) * prm.k_global;
            S = S + v;
        }
        const float mean = S / (float)n;
        const uint32_t u = __float_as_uint(mean);
        prm.index_keys[head * D + i] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    }
}

hipError_t launch_kv_store(const StoreParams &prm, int D, int B, hipStream_t stream)
{
    dim3 grid(B, prm.Hkv);
    if (D == 64)
        kv_store_kernel<64><<<grid, 256, 0, stream>>>(prm);
    else
        kv_store_kernel<128><<<grid, 256, 0, stream>>>(prm);
    return hipGetLastError();
}

}  // namespace qsa
