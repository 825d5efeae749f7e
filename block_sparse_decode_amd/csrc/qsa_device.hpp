// qsa_device.hpp -- device helpers shared by the gfx950 kernels of libqsa.
//
// Formats (OCP specs): e2m1 elements (1 sign, 2 exponent bits with bias 1, 1 mantissa bit),
// E4M3FN block scales (bias 7, NaN at S.1111.111, no infinities), bf16 queries and keys.
// The pages' NVFP4 KV cache keeps the e2m1 elements as uint8 codes beside e4m3 block scales
// (TensorRT-LLM PR #20276, Features, NVFP4 KV cache row).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

typedef _Float16 half_t;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two E4M3FN scale bytes (the low two bytes of `bytes`) -> two f16 values, exactly.
// gfx950's scaled fp8 convert applies only its scale operand's exponent, so with scale 1.0
// it is a plain OCP E4M3FN decode (NaN included). Every E4M3FN value, from the 2^-9
// subnormal up to 448, is exact in f16.
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t bytes)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 1.0f, false);
}

// Eight e2m1 codes (one dword; element 2i in the low nibble of byte i) times one e4m3
// block scale `s` (already in f16) -> eight f16 values, exactly.
// The hardware fp4 convert also takes its scale operand's exponent only, so it runs with
// scale 1.0 and returns the exact e2m1 values. The block scale is then one packed f16
// multiply per pair. An e2m1 value (<= 2 significant bits) times an e4m3 value
// (<= 4 bits) needs at most 6 bits and lies in [2^-10, 2688], so the product is exact
// in f16.
__device__ __forceinline__ f16x8 nvfp4_dequant8(uint32_t codes, half_t s)
{
    const f16x2 ss = {s, s};
    f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss;
    f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss;
    f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss;
    f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss;
    return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3),
                                   __builtin_shufflevector(c, d, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key), with -0 == +0.
__device__ __forceinline__ uint32_t float_order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void set_error(uint32_t *err, uint32_t bit)
{
    if (err) atomicOr(err, bit);
}

// Row geometry of an MTP verify batch: row j of a request with R rows and L_b tokens
// sees L_b - (R - 1 - j) tokens (clipped at 0) and ceil(L / P) pages (clipped at MP);
// P = 2^log2P.
struct RowGeom {
    int64_t len;
    int pages;
};

__device__ __forceinline__ RowGeom row_geom(int64_t seq_len, int R, int j, int log2P, int MP)
{
    RowGeom g;
    int64_t L = seq_len - (int64_t)(R - 1 - j);
    if (L < 0) L = 0;
    const int64_t n = (L + (1 << log2P) - 1) >> log2P;
    g.len = L;
    g.pages = (int)(n < MP ? n : MP);
    return g;
}

// Rows [r0, r0 + R) of one request, clipped to [0, N) and to at most rmax rows. A clip
// means row_offsets broke its contract; the caller learns it through the error word.
__device__ __forceinline__ int clip_rows(int r0, int r1, int N, int rmax, uint32_t *err, bool report)
{
    int R = r1 - r0;
    bool bad = r0 < 0 || R < 0 || r1 > N || R > rmax;
    if (r0 < 0 || R <= 0) R = 0;
    else {
        if (r0 + R > N) R = N - r0 > 0 ? N - r0 : 0;
        if (R > rmax) R = rmax;
    }
    if (bad && report) set_error(err, QSA_DEVERR_ROWS);
    return R;
}

// Wave-wide max over the lanes that share a 16-lane column slot (xor 16, xor 32).
__device__ __forceinline__ float max_across_groups(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), on DPP lane moves:
// a sliding sum of 4 lanes (row_shr 1, 2, 3), then row_shr 4 and 8 within each 16-lane row,
// then row_bcast 15 and 31 carry the row totals forward. Lanes outside a move add 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x)
{
    uint32_t y = x;
    y += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
    y += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
    y += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x113, 0xF, 0xF, true);   // row_shr:3
    y += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)y, 0x114, 0xF, 0xE, true);   // row_shr:4, lanes 4..15
    y += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)y, 0x118, 0xF, 0xC, true);   // row_shr:8, lanes 8..15
    y += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)y, 0x142, 0xA, 0xF, true);   // row_bcast:15, rows 1, 3
    y += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)y, 0x143, 0xC, 0xF, true);   // row_bcast:31, rows 2, 3
    return y;
}

}  // namespace qsa
