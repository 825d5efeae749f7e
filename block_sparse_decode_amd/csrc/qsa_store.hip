// qsa_store.hip -- the KV-store prologue of a decode / verify step: this step's new K and V
// tokens quantised to NVFP4 into their page slots, and the index keys of the pages that
// received them recomputed.
//
// Method: TensorRT-LLM PR #20276, Performance > What runs on the fast paths (the decode
// prologue covers index store and compression); PR #20937, Description > What changes (the
// prologue that writes a decode step's NVFP4 KV, fused); PR #20276, Features, NVFP4 KV cache row (e2m1 codes
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
// Design: one workgroup per (request, KV head); R <= 4 <= P, so the new tokens touch at
// most two pages. Every global load is issued at the start: each thread's share of the new
// rows (four elements of one 16-element block of K or V) and of the touched pages' stored K
// (16-byte code loads, 4-byte scale loads, into LDS). Then four lanes per block: amax over
// the quad by two xor shuffles, the scale, and four codes by threshold compares (the E2M1
// midpoints, with the tie direction of each). A code pair goes to its page slot in HBM and,
// for K, over the old slot in the LDS copy. Last, one thread per (touched page, element)
// sums the page's dequantised K from LDS over its valid tokens and writes the key. No value
// the kernel writes to HBM is read back. Contraction is off in this file so that every fp32
// sum and product is the rounded operation the definition states.
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

// E2M1 code nearest to an fp32 value, ties to the even code, magnitude at most 6: the
// magnitude code counts the midpoints of the grid {0, .5, 1, 1.5, 2, 3, 4, 6} that |y| passes,
// a midpoint counting when |y| lies above it, or on it when the code above it is even.
// NaN gives +0.
__device__ __forceinline__ uint32_t e2m1_encode(float y)
{
    const float a = fabsf(y);
    const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return mag | ((y < 0.0f && mag != 0u) ? 8u : 0u);
}

constexpr int kStoreMaxPage = 128;      // largest page size the store supports
constexpr int kStorePages = 2;          // pages R <= 4 new tokens can touch when P >= 64

template <int D>
__global__ __launch_bounds__(256) void kv_store_kernel(StoreParams prm)
{
    constexpr int CB = D / 2, SB = D / 16;                  // code / scale bytes per token
    constexpr int NB = D / 16;                              // blocks per token
    // one quad of lanes per new block of K or V: 2 * R * NB quads fit the 256 lanes for the
    // at most 4 rows per request that the host admits
    static_assert(2 * 4 * NB * 4 <= 256, "one pass of quads covers the new blocks");
    __shared__ __align__(16) uint8_t kc_lds[kStorePages][kStoreMaxPage * CB];
    __shared__ __align__(16) uint8_t ks_lds[kStorePages][kStoreMaxPage * SB];

    const int b = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    const int r0 = prm.row_offsets[b], r1 = prm.row_offsets[b + 1];
    const int R = clip_rows(r0, r1, prm.N, prm.rmax, prm.err, g == 0 && tid == 0);
    if (R == 0) return;
    const int Rb = r1 - r0;
    const int64_t L = prm.seq_lens[b];
    const int P = prm.P, MP = prm.MP;
    const int64_t first_pos = L - Rb > 0 ? L - Rb : 0;
    const int64_t last_pos = L - Rb + R - 1;
    const int64_t p_lo = first_pos / P;

    // this thread's quarter of one new block: K blocks of rows 0..R-1, then V blocks
    const int task = tid >> 2, quarter = tid & 3;
    const bool has_task = task < 2 * R * NB;                // whole quads: 2 R NB 4 <= 256
    const bool is_v = task >= R * NB;
    const int w = is_v ? task - R * NB : task;
    const int j = w / NB, blk = w - j * NB;
    const int64_t pos = L - Rb + j;
    int32_t phys = -1;
    uint2 raw = make_uint2(0u, 0u);
    if (has_task) {
        if (pos >= 0 && pos / P < MP) {
            phys = prm.page_table[(int64_t)b * MP + pos / P];
            if (phys >= 0 && (int64_t)phys < prm.NP) {
                const uint16_t *src = (is_v ? prm.new_v : prm.new_k) + ((int64_t)(r0 + j) * prm.Hkv + g) * D +
                                      blk * 16 + quarter * 4;
                raw = *reinterpret_cast<const uint2 *>(src);
            } else {
                if (phys != -1 && quarter == 0) set_error(prm.err, QSA_DEVERR_PAGE_ID);
                phys = -1;
            }
        } else if (g == 0 && blk == 0 && !is_v && quarter == 0) {
            set_error(prm.err, QSA_DEVERR_SEQ_LEN);
        }
    }

    // the touched pages: physical id (or -1 when the key is not rewritten) and valid tokens
    int32_t phys_pg[kStorePages];
    int n_pg[kStorePages];
#pragma unroll
    for (int k = 0; k < kStorePages; ++k) {
        const int64_t page = p_lo + k;
        phys_pg[k] = -1;
        n_pg[k] = 0;
        if (last_pos >= 0 && page * P <= last_pos && page < MP) {
            const int32_t ph = prm.page_table[(int64_t)b * MP + page];
            if (ph >= 0 && (int64_t)ph < prm.NP) {
                phys_pg[k] = ph;
                n_pg[k] = (int)(L - page * P < P ? L - page * P : P);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kStorePages; ++k) {
        if (phys_pg[k] < 0) continue;
        const int64_t tok0 = ((int64_t)phys_pg[k] * prm.Hkv + g) * P;
        const uint4 *cs = reinterpret_cast<const uint4 *>(prm.k_codes + tok0 * CB);
        uint4 *cd = reinterpret_cast<uint4 *>(kc_lds[k]);
        for (int x = tid; x < n_pg[k] * (CB / 16); x += blockDim.x) cd[x] = cs[x];
        const uint32_t *ss = reinterpret_cast<const uint32_t *>(prm.k_scales + tok0 * SB);
        uint32_t *sd = reinterpret_cast<uint32_t *>(ks_lds[k]);
        for (int x = tid; x < n_pg[k] * (SB / 4); x += blockDim.x) sd[x] = ss[x];
    }

    // ---- quantise: amax over the quad, scale, four codes -------------------------------
    const float x0 = bf16lo(raw.x), x1 = bf16hi(raw.x), x2 = bf16lo(raw.y), x3 = bf16hi(raw.y);
    float amax = fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3)));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const float global = is_v ? prm.v_global : prm.k_global;
    const uint32_t sc = e4m3_encode((amax / 6.0f) / global);
    const float s = e4m3_value(sc) * global;
    uint32_t pair = 0u;                                     // four nibbles, element 4q in the lowest
    if (s != 0.0f)
        pair = e2m1_encode(x0 / s) | (e2m1_encode(x1 / s) << 4) | (e2m1_encode(x2 / s) << 8) |
               (e2m1_encode(x3 / s) << 12);
    __syncthreads();                                        // the LDS copy of the stored K is whole

    if (phys >= 0) {
        const int slot = (int)(pos % P);
        const int64_t tok = ((int64_t)phys * prm.Hkv + g) * P + slot;
        uint8_t *codes = (is_v ? prm.v_codes : prm.k_codes) + tok * CB + blk * 8 + quarter * 2;
        *reinterpret_cast<uint16_t *>(codes) = (uint16_t)pair;
        if (quarter == 0) (is_v ? prm.v_scales : prm.k_scales)[tok * SB + blk] = (uint8_t)sc;
        if (!is_v) {
            const int k = (int)(pos / P - p_lo);            // 0 or 1: pos lies in [first_pos, last_pos]
            *reinterpret_cast<uint16_t *>(&kc_lds[k][slot * CB + blk * 8 + quarter * 2]) = (uint16_t)pair;
            if (quarter == 0) ks_lds[k][slot * SB + blk] = (uint8_t)sc;
        }
    }
    __syncthreads();

    // ---- index keys of the touched pages, from LDS -------------------------------------
    for (int t2 = tid; t2 < kStorePages * D; t2 += blockDim.x) {
        const int k = t2 / D, i = t2 % D;
        const int32_t ph = k == 0 ? phys_pg[0] : phys_pg[1];
        if (ph < 0) continue;
        const int n = k == 0 ? n_pg[0] : n_pg[1];
        const uint8_t *cl = kc_lds[k] + i / 2;
        const uint8_t *sl = ks_lds[k] + i / 16;
        const int sel = i & 1;
        const float kg = prm.k_global;
        float S = 0.0f;
        for (int t = 0; t < n; ++t) {
            // exact e2m1 and e4m3 values (hardware converts with a unit scale)
            const float e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((uint32_t)cl[t * CB], 1.0f, 0)[sel];
            const float sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)sl[t * SB], 1.0f, false)[0];
            S = S + (e * sv) * kg;
        }
        const float mean = S / (float)n;
        const uint32_t u = __float_as_uint(mean);
        prm.index_keys[((int64_t)ph * prm.Hkv + g) * D + i] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
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
