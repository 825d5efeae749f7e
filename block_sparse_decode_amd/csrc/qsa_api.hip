// qsa_api.hip -- the C ABI of libqsa (declared in include/qsa.h): host-side validation,
// launch-shape choice and kernel launches. No allocation, no synchronisation, no global state.
#include <cfloat>
#include <cmath>
#include <math.h>
#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "qsa_internal.hpp"

using namespace qsa;

namespace {

constexpr int kMaxRows = 1024;       // rows per request: decode, MTP verify, context and mixed steps
constexpr int kStoreMaxRows = 4;     // rows per request the KV store takes
constexpr int kTileMaxRows = 4;      // rows per attention tile (row-mask byte, union bound)
constexpr int kMaxPages = 4096;
constexpr int kMaxKW = 256;
constexpr int kMaxSplits = 64;
constexpr int64_t kCounterSlots = 8192;                 // split tiles per call
constexpr size_t kCounterBytes = kCounterSlots * sizeof(uint32_t);

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

qsa_status check_shape(const qsa_shape *sh)
{
    if (!sh) return QSA_ERR_INVALID_ARG;
    if (sh->num_requests < 0 || sh->num_rows < 0 || sh->num_q_heads < 1 || sh->num_kv_heads < 1 ||
        sh->num_q_heads % sh->num_kv_heads != 0 || sh->max_pages < 1 || sh->num_phys_pages < 0 ||
        sh->topk < 0 || sh->window < 0 || sh->max_rows_per_request < 1 || !isfinite(sh->sm_scale))
        return QSA_ERR_INVALID_ARG;
    if (sh->max_rows_per_request > kMaxRows) return QSA_ERR_UNSUPPORTED;
    if (sh->head_dim != 64 && sh->head_dim != 128) return QSA_ERR_UNSUPPORTED;
    if (sh->page_size != 64 && sh->page_size != 128) return QSA_ERR_UNSUPPORTED;
    if (sh->max_pages > kMaxPages) return QSA_ERR_UNSUPPORTED;
    if ((int64_t)sh->topk + sh->window > kMaxKW) return QSA_ERR_UNSUPPORTED;
    if (sh->num_requests > 65535 || sh->num_kv_heads > 65535) return QSA_ERR_UNSUPPORTED;
    if (sh->num_rows > (int64_t)sh->num_requests * sh->max_rows_per_request) return QSA_ERR_INVALID_ARG;
    if (sh->kv_format != QSA_KV_NVFP4 && sh->kv_format != QSA_KV_FP8) return QSA_ERR_INVALID_ARG;
    return QSA_OK;
}

qsa_status check_rows_ptrs(const qsa_paged *pg)
{
    if (!pg || !pg->seq_lens || !pg->row_offsets) return QSA_ERR_INVALID_ARG;
    if (!aligned16(pg->seq_lens) || !aligned16(pg->row_offsets)) return QSA_ERR_INVALID_ARG;
    if (pg->error_word && ((uintptr_t)pg->error_word & 3u)) return QSA_ERR_INVALID_ARG;
    return QSA_OK;
}

constexpr int kCUs = 256;
// A tile's prologue (row range, selection, union) in units of one page's loop work: the
// 32K verify workload's fused prologue (about 4.6 us) against its loop (about 11 us for a
// row's 34 pages).
constexpr double kTileProloguePages = 14.0;

// Query columns per tile. A request's columns for one KV head are its R rows x G q heads
// (row-major); a tile is a run of at most 16 of them (one MFMA N tile), and every page
// that any of the tile's rows selected is dequantised once for the whole tile. Tiles hold
// whole rows when G <= 16.
//
// Rows per tile, r, trade that sharing against balance. A tile's cost is taken as its
// expected union of pages plus a fixed prologue, and a launch of T tiles as ceil(T / CUs)
// times that: tiles are counted in rounds of one per CU, since a CU that holds two tiles
// finishes when both have. The union of r rows, each selecting s = k + W of a request's n
// pages (n taken as the table width MP), is n (1 - (1 - s/n)^r) when the selections are
// independent: verify rows of a long request share only their window and a few pages,
// the neighbouring rows of a context step over a short one most of theirs. A larger r is
// considered only while it keeps a tile per CU; below that the parallelism has to come
// from splits (auto_splits), whose merge a single row per tile avoids best. Measured
// (MI355X, fused launch): 48 requests x 4 verify rows over 1024-page tables, one row per
// tile 53.8 us against 56.0 us at two; 4 requests x 256 context rows over 128 pages, two
// rows per tile 140 us against 158 us at one.
int tile_cols(const qsa_shape *sh)
{
    const int G = sh->num_q_heads / sh->num_kv_heads;
    if (G >= 16) return 16;
    const int rcap = std::max(1, std::min({sh->max_rows_per_request, 16 / G, kTileMaxRows}));
    auto tiles = [&](int r) {
        return (int64_t)sh->num_requests * sh->num_kv_heads * ((sh->max_rows_per_request + r - 1) / r);
    };
    const double n = std::max(1, sh->max_pages);
    const double sel = std::min<double>(sh->topk + sh->window, n);
    int best = 1;
    double best_cost = 0.0;
    for (int r = 1; r <= rcap; ++r) {
        const int64_t T = tiles(r);
        if (r > 1 && T < kCUs) break;
        const double uni = n * (1.0 - std::pow(1.0 - sel / n, (double)r));
        const double cost = (double)((T + kCUs - 1) / kCUs) * (uni + kTileProloguePages);
        if (r == 1 || cost < best_cost) {
            best = r;
            best_cost = cost;
        }
    }
    return best * G;
}

int col_tiles(const qsa_shape *sh)
{
    const int cols = sh->max_rows_per_request * (sh->num_q_heads / sh->num_kv_heads);
    const int tw = tile_cols(sh);
    return (cols + tw - 1) / tw;
}

// Splits per (request, KV head, column tile) when the caller leaves the choice to the
// library: about one workgroup (8 waves) per CU over the 256 CUs, without splits so thin
// that a wave gets less than half a page of the expected union. (Two workgroups fit per CU;
// fewer, longer workgroups measured faster than one full round of short ones, because each
// workgroup pays the union build and each split adds partials to merge.)
int auto_splits(const qsa_shape *sh)
{
    const int64_t base = (int64_t)sh->num_requests * sh->num_kv_heads * col_tiles(sh);
    if (base <= 0) return 1;
    const int G = sh->num_q_heads / sh->num_kv_heads;
    const int64_t rows_per_tile = std::max<int64_t>(1, std::min<int64_t>(sh->max_rows_per_request, tile_cols(sh) / G));
    const int64_t union_est = std::min<int64_t>(rows_per_tile * (sh->topk + sh->window), sh->max_pages);
    int64_t s = (kCUs + base - 1) / base;
    const int64_t cap = std::max<int64_t>(1, 2 * union_est / kDecodeWaves);
    s = std::min(s, cap);
    s = std::max<int64_t>(1, std::min<int64_t>(s, kMaxSplits));
    return (int)s;
}

// Every tile holds columns of one row only: one row per tile, or 16-column tiles of rows of a
// multiple of 16 q heads.
bool one_row_tiles(const qsa_shape *sh)
{
    const int G = sh->num_q_heads / sh->num_kv_heads;
    return G <= 16 ? tile_cols(sh) == G : G % 16 == 0;
}

int64_t decode_tiles(const qsa_shape *sh)
{
    return (int64_t)sh->num_requests * sh->num_kv_heads * col_tiles(sh);
}

// Splits per tile: the caller's count (clamped to kMaxSplits) or the library's choice. A split
// tile needs a completion counter, and the counters live in a region of fixed size at the
// start of the workspace (kCounterSlots words), so a batch with more tiles than that runs one
// split per tile. Splitting pays only when tiles are fewer than CUs, so the automatic choice
// never reaches that bound.
int resolve_splits(const qsa_shape *sh, int32_t num_splits)
{
    const int s = num_splits <= 0 ? auto_splits(sh) : (num_splits > kMaxSplits ? kMaxSplits : num_splits);
    return decode_tiles(sh) > kCounterSlots ? 1 : s;
}

// Workspace of a split decode: the counter region first, at a fixed size that does not depend
// on the shape, then the partials of every (tile, split). A workspace therefore keeps its
// counters where every later call looks for them, whatever that call's batch or split count,
// and no call's partials ever overlap a counter.
size_t decode_ws_bytes(const qsa_shape *sh, int splits)
{
    if (splits <= 1) return 0;
    return kCounterBytes + (size_t)decode_tiles(sh) * splits * decode_part_floats(sh->head_dim) * sizeof(float);
}

}  // namespace

extern "C" {

int32_t qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char *qsa_status_string(qsa_status st)
{
    switch (st) {
    case QSA_OK: return "ok";
    case QSA_ERR_INVALID_ARG: return "invalid argument";
    case QSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case QSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QSA_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

qsa_status qsa_index_scores(const qsa_shape *sh, const qsa_paged *pg, const uint16_t *q, float *scores,
                            void *stream)
{
    qsa_status st = check_shape(sh);
    if (st != QSA_OK) return st;
    if ((st = check_rows_ptrs(pg)) != QSA_OK) return st;
    if (sh->num_rows == 0 || sh->num_requests == 0) return QSA_OK;
    if (!q || !scores || !pg->page_table || !pg->index_keys) return QSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(scores) || !aligned16(pg->page_table) || !aligned16(pg->index_keys))
        return QSA_ERR_INVALID_ARG;
    IndexParams prm;
    prm.page_table = pg->page_table;
    prm.seq_lens = pg->seq_lens;
    prm.row_offsets = pg->row_offsets;
    prm.keys = pg->index_keys;
    prm.q32 = reinterpret_cast<const uint32_t *>(q);
    prm.scores = scores;
    prm.err = pg->error_word;
    prm.NP = sh->num_phys_pages;
    prm.N = sh->num_rows;
    prm.MP = sh->max_pages;
    prm.P = sh->page_size;
    prm.log2P = sh->page_size == 64 ? 6 : 7;
    prm.W = sh->window;
    prm.Hq = sh->num_q_heads;
    prm.Hkv = sh->num_kv_heads;
    prm.rmax = sh->max_rows_per_request;
    prm.sm_scale = sh->sm_scale;
    prm.uniform_rows = (int64_t)sh->num_rows == (int64_t)sh->num_requests * sh->max_rows_per_request;
    hipError_t e = launch_index_scores(prm, sh->head_dim, sh->num_requests, (hipStream_t)stream);
    return e == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

qsa_status qsa_select_topk(const qsa_shape *sh, const qsa_paged *pg, const float *scores, int32_t *selected,
                           void *stream)
{
    qsa_status st = check_shape(sh);
    if (st != QSA_OK) return st;
    if ((st = check_rows_ptrs(pg)) != QSA_OK) return st;
    if (sh->num_rows == 0 || sh->num_requests == 0 || sh->topk + sh->window == 0) return QSA_OK;
    if (!scores || !selected || !aligned16(scores) || !aligned16(selected)) return QSA_ERR_INVALID_ARG;
    SelectParams prm;
    prm.seq_lens = pg->seq_lens;
    prm.row_offsets = pg->row_offsets;
    prm.scores = scores;
    prm.selected = selected;
    prm.err = pg->error_word;
    prm.N = sh->num_rows;
    prm.MP = sh->max_pages;
    prm.P = sh->page_size;
    prm.log2P = sh->page_size == 64 ? 6 : 7;
    prm.k = sh->topk;
    prm.W = sh->window;
    prm.rmax = sh->max_rows_per_request;
    hipError_t e = launch_select_topk(prm, sh->num_requests, (hipStream_t)stream);
    return e == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

size_t qsa_workspace_bytes(const qsa_shape *sh, int32_t num_splits)
{
    if (check_shape(sh) != QSA_OK) return 0;
    return decode_ws_bytes(sh, resolve_splits(sh, num_splits));
}

qsa_status qsa_plan_decode(const qsa_shape *sh, int32_t num_splits, int32_t fused, qsa_decode_plan *plan)
{
    const qsa_status st = check_shape(sh);
    if (st != QSA_OK) return st;
    if (!plan || num_splits < 0) return QSA_ERR_INVALID_ARG;
    const int G = sh->num_q_heads / sh->num_kv_heads;
    const int splits = resolve_splits(sh, num_splits);
    plan->tile_cols = tile_cols(sh);
    plan->rows_per_tile = G <= 16 ? plan->tile_cols / G : 0;
    plan->col_tiles = col_tiles(sh);
    plan->splits = splits;
    plan->select_cols = (fused && sh->topk + sh->window > 0) ? fused_select_cols(sh->max_pages) : 0;
    const int64_t items = decode_tiles(sh) * splits;
    plan->waves = decode_waves(one_row_tiles(sh), (int)std::min<int64_t>(decode_tiles(sh), 1 << 30), splits);
    plan->workgroups = (items + kXcdCount - 1) / kXcdCount * kXcdCount;
    plan->workspace_bytes = decode_ws_bytes(sh, splits);
    return QSA_OK;
}

}  // extern "C"

namespace qsa {

// Shared by qsa_sparse_decode (scores == NULL: `selected` is an input),
// qsa_select_sparse_decode (the selection is computed from `scores` and written to `selected`)
// and qsa_select_sparse_decode_static (clear_counters: the workspace's completion counters are
// zeroed by a fill kernel before the attention launch, since its contents are not the caller's).
qsa_status decode_call(const qsa_shape *sh, const qsa_paged *pg, const uint16_t *q, const float *scores,
                       int32_t *selected, uint16_t *out, float *lse, const uint16_t *gate, int32_t num_splits,
                       void *workspace, size_t workspace_bytes, void *stream, bool clear_counters)
{
    qsa_status st = check_shape(sh);
    if (st != QSA_OK) return st;
    if ((st = check_rows_ptrs(pg)) != QSA_OK) return st;
    if (num_splits < 0) return QSA_ERR_INVALID_ARG;
    if (sh->num_rows == 0 || sh->num_requests == 0) return QSA_OK;
    const bool nvfp4 = sh->kv_format == QSA_KV_NVFP4;
    if (!q || !out || !pg->page_table || !pg->k_codes || !pg->v_codes) return QSA_ERR_INVALID_ARG;
    if (nvfp4 && (!pg->k_scales || !pg->v_scales || !aligned16(pg->k_scales) || !aligned16(pg->v_scales)))
        return QSA_ERR_INVALID_ARG;
    const bool fused = scores != nullptr;
    const int KW = sh->topk + sh->window;
    if (KW > 0 && !selected) return QSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(pg->page_table) || !aligned16(pg->k_codes) ||
        !aligned16(pg->v_codes) || (selected && !aligned16(selected)) || (lse && !aligned16(lse)) ||
        (fused && !aligned16(scores)) || (gate && !aligned16(gate)))
        return QSA_ERR_INVALID_ARG;
    if (!isfinite(pg->k_global) || !isfinite(pg->v_global)) return QSA_ERR_INVALID_ARG;
    // the logit scale sm_scale * k_global * log2(e) must be a positive normal fp32: the
    // kernel's lazy max compares raw logits against (max + margin) / scale
    const double qk = (double)sh->sm_scale * (double)pg->k_global * 1.4426950408889634;
    if (!(qk >= (double)FLT_MIN && qk <= (double)FLT_MAX)) return QSA_ERR_INVALID_ARG;
    const int splits = resolve_splits(sh, num_splits);
    const size_t need = decode_ws_bytes(sh, splits);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return QSA_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned16(workspace)) return QSA_ERR_INVALID_ARG;
    }
    DecodeParams prm;
    prm.page_table = pg->page_table;
    prm.seq_lens = pg->seq_lens;
    prm.row_offsets = pg->row_offsets;
    prm.k_codes = pg->k_codes;
    prm.k_scales = pg->k_scales;
    prm.v_codes = pg->v_codes;
    prm.v_scales = pg->v_scales;
    prm.q = q;
    prm.selected = selected;
    prm.scores = scores;
    prm.out = out;
    prm.lse = lse;
    prm.counters = need ? reinterpret_cast<uint32_t *>(workspace) : nullptr;
    prm.part = need ? reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + kCounterBytes)
                    : nullptr;
    prm.err = pg->error_word;
    prm.NP = sh->num_phys_pages;
    prm.N = sh->num_rows;
    prm.MP = sh->max_pages;
    prm.P = sh->page_size;
    prm.log2P = sh->page_size == 64 ? 6 : 7;
    prm.KW = KW;
    prm.k = sh->topk;
    prm.W = sh->window;
    prm.Hq = sh->num_q_heads;
    prm.Hkv = sh->num_kv_heads;
    prm.rmax = sh->max_rows_per_request;
    prm.splits = splits;
    prm.col_tiles = col_tiles(sh);
    prm.tile_cols = tile_cols(sh);
    if (decode_tiles(sh) * splits > (int64_t)1 << 30) return QSA_ERR_UNSUPPORTED;
    prm.tiles = (int)decode_tiles(sh);
    prm.div_splits = FastDiv::make((uint32_t)splits);
    prm.div_ctiles = FastDiv::make((uint32_t)prm.col_tiles);
    prm.div_htiles = FastDiv::make((uint32_t)(prm.Hkv * prm.col_tiles));
    prm.div_group = FastDiv::make((uint32_t)(prm.Hq / prm.Hkv));
    prm.div_kw = FastDiv::make((uint32_t)(KW > 0 ? KW : 1));
    prm.qk_scale_log2 = (float)qk;
    prm.v_global = pg->v_global;
    prm.gate = gate;
    prm.kv_format = sh->kv_format;
    prm.uniform_rows = (int64_t)sh->num_rows == (int64_t)sh->num_requests * sh->max_rows_per_request;
    prm.one_row_tiles = one_row_tiles(sh);
    hipError_t e = hipSuccess;
    if (clear_counters && need > 0) {
        e = launch_clear_words(prm.counters, prm.tiles, (hipStream_t)stream);
        if (e != hipSuccess) return QSA_ERR_HIP;
    }
    if (!fused || KW == 0) {
        e = launch_sparse_decode(prm, sh->head_dim, (hipStream_t)stream);
    } else if (sh->max_pages <= 1024) {
        e = launch_select_sparse_decode(prm, sh->head_dim, (hipStream_t)stream);
    } else {
        // wide score tables: the separate selection kernel, then the attention
        SelectParams sp;
        sp.seq_lens = pg->seq_lens;
        sp.row_offsets = pg->row_offsets;
        sp.scores = scores;
        sp.selected = selected;
        sp.err = pg->error_word;
        sp.N = sh->num_rows;
        sp.MP = sh->max_pages;
        sp.P = sh->page_size;
        sp.log2P = prm.log2P;
        sp.k = sh->topk;
        sp.W = sh->window;
        sp.rmax = sh->max_rows_per_request;
        e = launch_select_topk(sp, sh->num_requests, (hipStream_t)stream);
        if (e == hipSuccess) e = launch_sparse_decode(prm, sh->head_dim, (hipStream_t)stream);
    }
    return e == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

}  // namespace qsa

extern "C" {

qsa_status qsa_sparse_decode(const qsa_shape *sh, const qsa_paged *pg, const uint16_t *q, const int32_t *selected,
                             uint16_t *out, float *lse, const uint16_t *gate, int32_t num_splits, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    return decode_call(sh, pg, q, nullptr, const_cast<int32_t *>(selected), out, lse, gate, num_splits, workspace,
                       workspace_bytes, stream, false);
}

qsa_status qsa_select_sparse_decode(const qsa_shape *sh, const qsa_paged *pg, const uint16_t *q, const float *scores,
                                    int32_t *selected, uint16_t *out, float *lse, const uint16_t *gate,
                                    int32_t num_splits, void *workspace, size_t workspace_bytes, void *stream)
{
    if (sh && pg && sh->topk + sh->window > 0 && !scores && sh->num_rows > 0 && sh->num_requests > 0)
        return QSA_ERR_INVALID_ARG;
    return decode_call(sh, pg, q, scores, selected, out, lse, gate, num_splits, workspace, workspace_bytes, stream,
                       false);
}

qsa_status qsa_kv_store(const qsa_shape *sh, const qsa_paged *pg, const uint16_t *new_k, const uint16_t *new_v,
                        void *stream)
{
    qsa_status st = check_shape(sh);
    if (st != QSA_OK) return st;
    if (sh->kv_format != QSA_KV_NVFP4 || sh->max_rows_per_request > kStoreMaxRows) return QSA_ERR_UNSUPPORTED;
    if ((st = check_rows_ptrs(pg)) != QSA_OK) return st;
    if (sh->num_rows == 0 || sh->num_requests == 0) return QSA_OK;
    if (!new_k || !new_v || !pg->page_table || !pg->k_codes || !pg->k_scales || !pg->v_codes || !pg->v_scales ||
        !pg->index_keys)
        return QSA_ERR_INVALID_ARG;
    if (!aligned16(new_k) || !aligned16(new_v) || !aligned16(pg->page_table) || !aligned16(pg->k_codes) ||
        !aligned16(pg->k_scales) || !aligned16(pg->v_codes) || !aligned16(pg->v_scales) || !aligned16(pg->index_keys))
        return QSA_ERR_INVALID_ARG;
    if (!isfinite(pg->k_global) || !isfinite(pg->v_global) || !(pg->k_global > 0.0f) || !(pg->v_global > 0.0f))
        return QSA_ERR_INVALID_ARG;
    StoreParams prm;
    prm.page_table = pg->page_table;
    prm.seq_lens = pg->seq_lens;
    prm.row_offsets = pg->row_offsets;
    prm.new_k = new_k;
    prm.new_v = new_v;
    // the planes are written through the same pointers the other calls read
    prm.k_codes = const_cast<uint8_t *>(pg->k_codes);
    prm.k_scales = const_cast<uint8_t *>(pg->k_scales);
    prm.v_codes = const_cast<uint8_t *>(pg->v_codes);
    prm.v_scales = const_cast<uint8_t *>(pg->v_scales);
    prm.index_keys = const_cast<uint16_t *>(pg->index_keys);
    prm.err = pg->error_word;
    prm.NP = sh->num_phys_pages;
    prm.N = sh->num_rows;
    prm.MP = sh->max_pages;
    prm.P = sh->page_size;
    prm.Hkv = sh->num_kv_heads;
    prm.rmax = sh->max_rows_per_request;
    prm.k_global = pg->k_global;
    prm.v_global = pg->v_global;
    hipError_t e = launch_kv_store(prm, sh->head_dim, sh->num_requests, (hipStream_t)stream);
    return e == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

qsa_status qsa_nvfp4_dequant_pages(const qsa_shape *sh, const uint8_t *codes, const uint8_t *scales,
                                   float global_scale, const int32_t *pages, int32_t num_pages, float *out,
                                   void *stream)
{
    if (!sh) return QSA_ERR_INVALID_ARG;
    if (sh->num_kv_heads < 1 || sh->num_phys_pages < 0 || num_pages < 0 || !isfinite(global_scale))
        return QSA_ERR_INVALID_ARG;
    if (sh->head_dim != 64 && sh->head_dim != 128) return QSA_ERR_UNSUPPORTED;
    if (sh->page_size != 64 && sh->page_size != 128) return QSA_ERR_UNSUPPORTED;
    if (num_pages == 0) return QSA_OK;
    if (!codes || !scales || !pages || !out) return QSA_ERR_INVALID_ARG;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(pages) || !aligned16(out)) return QSA_ERR_INVALID_ARG;
    DequantParams prm;
    prm.codes = codes;
    prm.scales = scales;
    prm.pages = pages;
    prm.out = out;
    prm.NP = sh->num_phys_pages;
    prm.n = num_pages;
    prm.Hkv = sh->num_kv_heads;
    prm.P = sh->page_size;
    prm.global = global_scale;
    hipError_t e = launch_dequant_pages(prm, sh->head_dim, (hipStream_t)stream);
    return e == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

}  // extern "C"

namespace {

bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

// Validates the plane descriptors and fills the device descriptors with the stash offsets;
// returns the stash size, or 0 (with ok = false) when anything is invalid.
size_t plan_planes(const qsa_plane *planes, int32_t n, int32_t nrows, PlaneDesc *out, bool &ok)
{
    ok = false;
    if (!planes || n < 1 || n > QSA_MAX_PLANES || nrows < 0) return 0;
    unsigned __int128 off = 0;
    for (int k = 0; k < n; ++k) {
        const qsa_plane &p = planes[k];
        if (!p.base || !aligned4(p.base) || p.plane_bytes <= 0 || p.page_stride < 0 || p.slot_stride < 0 ||
            p.seg_stride < 0 || p.seg_bytes <= 0 || p.nseg < 1 || p.num_pages < 0 || p.num_slots < 1)
            return 0;
        if ((p.page_stride | p.slot_stride | p.seg_stride | (int64_t)p.seg_bytes) & 3) return 0;
        if (p.num_pages > 0) {
            // the last byte any (page, slot, segment) can address must lie inside the plane
            const unsigned __int128 last = (unsigned __int128)(p.num_pages - 1) * (uint64_t)p.page_stride +
                                           (unsigned __int128)(p.num_slots - 1) * (uint64_t)p.slot_stride +
                                           (unsigned __int128)(p.nseg - 1) * (uint64_t)p.seg_stride +
                                           (uint64_t)p.seg_bytes;
            if (last > (unsigned __int128)p.plane_bytes) return 0;
        }
        const unsigned __int128 row = (unsigned __int128)p.nseg * (uint64_t)p.seg_bytes;
        if (row / 4 > (1u << 24)) return 0;         // a row of at most 64 MiB
        if (out) {
            out[k].base = reinterpret_cast<char *>(p.base);
            out[k].page_stride = p.page_stride;
            out[k].slot_stride = p.slot_stride;
            out[k].seg_stride = p.seg_stride;
            out[k].num_pages = p.num_pages;
            out[k].stash_off = (int64_t)off;
            out[k].seg_words = p.seg_bytes / 4;
            out[k].nseg = p.nseg;
            out[k].num_slots = p.num_slots;
            out[k].pad = 0;
        }
        off += (row * (uint64_t)nrows + 15) / 16 * 16;
        if (off > ((unsigned __int128)1 << 62)) return 0;
    }
    ok = true;
    return (size_t)off;
}

qsa_status rollback_call(const qsa_plane *planes, int32_t num_planes, const int32_t *pages, const int32_t *within,
                         const int32_t *rejected, int32_t num_rows, const void *stash, size_t stash_bytes,
                         uint32_t *error_word, void *stream, bool restore)
{
    RollbackParams prm;
    bool ok = false;
    const size_t need = plan_planes(planes, num_planes, num_rows, prm.planes, ok);
    if (!ok) return QSA_ERR_INVALID_ARG;
    if (error_word && !aligned4(error_word)) return QSA_ERR_INVALID_ARG;
    if (num_rows == 0) return QSA_OK;
    if (!pages || !within || !aligned4(pages) || !aligned4(within)) return QSA_ERR_INVALID_ARG;
    if (restore && (!rejected || !aligned4(rejected))) return QSA_ERR_INVALID_ARG;
    if (!stash || !aligned16(stash)) return QSA_ERR_INVALID_ARG;
    if (stash_bytes < need) return QSA_ERR_WORKSPACE_TOO_SMALL;
    prm.pages = pages;
    prm.within = within;
    prm.rejected = rejected;
    prm.stash = reinterpret_cast<char *>(const_cast<void *>(stash));
    prm.err = error_word;
    prm.nrows = num_rows;
    const hipError_t e = launch_rollback(prm, num_planes, restore, (hipStream_t)stream);
    return e == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

}  // namespace

extern "C" {

size_t qsa_rollback_stash_bytes(const qsa_plane *planes, int32_t num_planes, int32_t num_rows)
{
    bool ok = false;
    const size_t n = plan_planes(planes, num_planes, num_rows, nullptr, ok);
    return ok ? n : 0;
}

qsa_status qsa_rollback_gather(const qsa_plane *planes, int32_t num_planes, const int32_t *pages,
                               const int32_t *within, int32_t num_rows, void *stash, size_t stash_bytes,
                               uint32_t *error_word, void *stream)
{
    return rollback_call(planes, num_planes, pages, within, nullptr, num_rows, stash, stash_bytes, error_word,
                         stream, false);
}

qsa_status qsa_rollback_restore(const qsa_plane *planes, int32_t num_planes, const int32_t *pages,
                                const int32_t *within, const int32_t *rejected, int32_t num_rows,
                                const void *stash, size_t stash_bytes, uint32_t *error_word, void *stream)
{
    return rollback_call(planes, num_planes, pages, within, rejected, num_rows, stash, stash_bytes, error_word,
                         stream, true);
}

qsa_status qsa_step_slots(const qsa_shape *sh, const qsa_paged *pg, int32_t *pages, int32_t *within,
                          void *stream)
{
    qsa_status st = check_shape(sh);
    if (st != QSA_OK) return st;
    if ((st = check_rows_ptrs(pg)) != QSA_OK) return st;
    if (sh->num_rows == 0 || sh->num_requests == 0) return QSA_OK;
    if (!pg->page_table || !aligned16(pg->page_table) || !pages || !within || !aligned4(pages) ||
        !aligned4(within))
        return QSA_ERR_INVALID_ARG;
    SlotParams prm;
    prm.page_table = pg->page_table;
    prm.seq_lens = pg->seq_lens;
    prm.row_offsets = pg->row_offsets;
    prm.pages = pages;
    prm.within = within;
    prm.err = pg->error_word;
    prm.NP = sh->num_phys_pages;
    prm.N = sh->num_rows;
    prm.MP = sh->max_pages;
    prm.P = sh->page_size;
    prm.rmax = sh->max_rows_per_request;
    const hipError_t e = launch_step_slots(prm, sh->num_requests, (hipStream_t)stream);
    return e == hipSuccess ? QSA_OK : QSA_ERR_HIP;
}

}  // extern "C"
