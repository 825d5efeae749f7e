// qsa_internal.hpp -- launch parameter blocks shared by the host API and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <assert.h>
#include <stdint.h>

#include "qsa.h"
#include "qsa_fastdiv.hpp"

namespace qsa {

// n / f.d for 0 <= n < 2^31 (f taken by value, so that a kernel argument's copy is not
// addressed)
__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) { return (__umulhi(n, f.m) + n) >> f.l; }

struct IndexParams {
    const int32_t *page_table;
    const int32_t *seq_lens;
    const int32_t *row_offsets;
    const uint16_t *keys;
    const uint32_t *q32;      // bf16 pairs
    float *scores;
    uint32_t *err;
    int64_t NP;
    int N, MP, P, log2P, W, Hq, Hkv, rmax;
    float sm_scale;
    int uniform_rows;         // N == B * rmax: request b's rows are [b * rmax, (b + 1) * rmax)
};

struct SelectParams {
    const int32_t *seq_lens;
    const int32_t *row_offsets;
    const float *scores;
    int32_t *selected;
    uint32_t *err;
    int N, MP, P, log2P, k, W, rmax;
};

struct DecodeParams {
    const int32_t *page_table;
    const int32_t *seq_lens;
    const int32_t *row_offsets;
    const uint8_t *k_codes;
    const uint8_t *k_scales;
    const uint8_t *v_codes;
    const uint8_t *v_scales;
    const uint16_t *q;
    int32_t *selected;        // input, or with the selection fused in: output [N][k + W]
    const float *scores;      // selection fused in only: [N][MP]
    uint16_t *out;
    float *lse;
    float *part;              // [tiles][S][decode_part_floats(D)] partials of split tiles (S > 1)
    uint32_t *counters;       // [tiles] splits finished per tile; zero between calls (S > 1)
    uint32_t *err;
    int64_t NP;
    int N, MP, P, log2P, KW, Hq, Hkv, rmax, splits, col_tiles, tiles;
    int tile_cols;            // query columns (rows x q heads of one KV head) per tile, <= 16
    FastDiv div_splits, div_ctiles, div_htiles, div_group, div_kw;   // S, col_tiles, Hkv * col_tiles, Hq / Hkv, k + W
    int k, W;                 // selection fused in only
    float qk_scale_log2;      // sm_scale * k_global * log2(e)
    float v_global;
    const uint16_t *gate;     // optional bf16 [N][Hq][d]: out = o * sigmoid(gate)
    int kv_format;            // QSA_KV_NVFP4 or QSA_KV_FP8
    int uniform_rows;         // N == B * rmax: request b's rows are [b * rmax, (b + 1) * rmax)
    int one_row_tiles;        // every tile holds columns of one row only
};

struct StoreParams {
    const int32_t *page_table;
    const int32_t *seq_lens;
    const int32_t *row_offsets;
    const uint16_t *new_k;    // bf16 [N][Hkv][d]
    const uint16_t *new_v;
    uint8_t *k_codes;
    uint8_t *k_scales;
    uint8_t *v_codes;
    uint8_t *v_scales;
    uint16_t *index_keys;
    uint32_t *err;
    int64_t NP;
    int N, MP, P, Hkv, rmax;
    float k_global, v_global;
};

struct DequantParams {
    const uint8_t *codes;
    const uint8_t *scales;
    const int32_t *pages;
    float *out;
    int64_t NP;
    int n, Hkv, P;
    float global;
};

hipError_t launch_index_scores(const IndexParams &prm, int D, int B, hipStream_t stream);
hipError_t launch_select_topk(const SelectParams &prm, int B, hipStream_t stream);
hipError_t launch_sparse_decode(const DecodeParams &prm, int D, hipStream_t stream);
// the selection of each tile's rows computed from `scores` inside the attention kernel's
// prologue (MP <= 1024); `selected` is written as qsa_select_topk writes it
hipError_t launch_select_sparse_decode(const DecodeParams &prm, int D, hipStream_t stream);
hipError_t launch_dequant_pages(const DequantParams &prm, int D, hipStream_t stream);
// n uint32 words at p set to zero by a small fill kernel (no memset node in captured graphs)
hipError_t launch_clear_words(uint32_t *p, int n, hipStream_t stream);

// host side of the attention calls (qsa_api.hip): validation, launch plan and launches;
// clear_counters zeroes the workspace's completion counters first
qsa_status decode_call(const qsa_shape *sh, const qsa_paged *pg, const uint16_t *q, const float *scores,
                       int32_t *selected, uint16_t *out, float *lse, const uint16_t *gate, int32_t num_splits,
                       void *workspace, size_t workspace_bytes, void *stream, bool clear_counters);
hipError_t launch_kv_store(const StoreParams &prm, int D, int B, hipStream_t stream);

// ---- rollback ---------------------------------------------------------------------------
struct PlaneDesc {
    char *base;
    int64_t page_stride, slot_stride, seg_stride;
    int64_t num_pages;
    int64_t stash_off;          // byte offset of this plane's rows in the stash
    int32_t seg_words;          // seg_bytes / 4
    int32_t nseg;
    int32_t num_slots;
    int32_t pad;
};

struct RollbackParams {
    PlaneDesc planes[QSA_MAX_PLANES];
    const int32_t *pages;
    const int32_t *within;
    const int32_t *rejected;    // restore only
    char *stash;
    uint32_t *err;
    int32_t nrows;
};

struct SlotParams {
    const int32_t *page_table;
    const int32_t *seq_lens;
    const int32_t *row_offsets;
    int32_t *pages;
    int32_t *within;
    uint32_t *err;
    int64_t NP;
    int32_t N, MP, P, rmax;
};

hipError_t launch_rollback(const RollbackParams &prm, int num_planes, bool restore, hipStream_t stream);
hipError_t launch_step_slots(const SlotParams &prm, int B, hipStream_t stream);

// number of waves per decode workgroup
constexpr int kDecodeWaves = 8;

// Waves per workgroup of an attention launch. An 8-wave one-row workgroup takes half a CU
// (its V staging fills half the LDS), so a launch of more than two work items per CU runs
// in rounds, the last of them part-filled. One-row tiles then take 4-wave workgroups, three
// of which fit a CU, and the items run together in fewer rounds.
constexpr int kDecodeCUs = 256;
constexpr int decode_waves(int one_row_tiles, int tiles, int splits)
{
    return one_row_tiles && (int64_t)tiles * splits > 2 * kDecodeCUs ? 4 : kDecodeWaves;
}

// XCDs of the chip; decode workgroups are numbered so that each XCD takes a contiguous run of
// work items (the grid is rounded up to a multiple of this)
constexpr int kXcdCount = 8;

// Score columns per lane of the selection fused into the attention launch: the fewest that
// cover the table (each bit-search step costs a compare and a popcount per column); 0 when
// the table is too wide and the launch runs the separate selection kernel first.
constexpr int fused_select_cols(int MP) { return MP <= 128 ? 2 : MP <= 256 ? 4 : MP <= 512 ? 8 : MP <= 1024 ? 16 : 0; }

// A split's partial result for one tile (16 query columns): the unnormalised O^T
// accumulators of the d/16 output tiles and the ones tile (the softmax denominator), laid
// out [tile][element 0..3][lane], then the column max (log2 units) per lane.
constexpr int decode_part_floats(int D) { return (D / 16 + 1) * 64 * 4 + 64; }

}  // namespace qsa
