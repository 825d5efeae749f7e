/*
 * qsa.h -- C ABI of the query-sparse NVFP4 decode / verify attention library (libqsa.so).
 *
 * The method (TensorRT-LLM PR #20276, "What runs on the fast paths"; PR #20937,
 * Description > What changes) runs one attention layer of a decode, MTP-verify, context or
 * mixed step over a paged KV cache in three calls:
 *
 *   1. qsa_index_scores  -- score every page of every query row against its index key;
 *   2. qsa_select_topk   -- canonical top-k pages plus a local window per row;
 *   3. qsa_sparse_decode -- split-KV softmax attention over the selected pages, with an
 *                           LSE merge of the splits (optionally gated);
 *
 * or in two, with qsa_select_sparse_decode doing 2 and 3 in one launch. Around the step:
 * qsa_kv_store writes the step's new tokens into the cache and the touched pages' index
 * keys; qsa_rollback_gather / qsa_rollback_restore save and restore the plane rows of
 * rejected draft rows (qsa_step_slots gives each row's page and slot).
 *
 * Conventions shared by every call
 *   - Tensor arguments are DEVICE pointers owned by the caller. The library never
 *     allocates, frees or reads device memory from the host, and it never synchronises.
 *     Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *   - Tensor pointers must be aligned to 16 bytes unless a call states otherwise.
 *   - Host-checkable argument errors return a status before any launch. Nothing is
 *     written then. The library never aborts or throws.
 *   - The library keeps no mutable global state. Calls on different streams may run
 *     concurrently as long as their output buffers are distinct.
 *   - Data-dependent preconditions (page ids, lengths) cannot be checked on the host
 *     without a sync. Device code handles a violation as stated per call, and if
 *     `paged->error_word` is non-NULL it ORs one of the QSA_DEVERR_* bits into it.
 *
 * Notation: B requests, N = row_offsets[B] query rows, Hq query heads, Hkv KV heads
 * (G = Hq / Hkv), d head dim, P tokens per page, MP page-table stride, NP physical pages,
 * k top-k, W window pages.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 2

typedef enum qsa_status {
    QSA_OK = 0,
    QSA_ERR_INVALID_ARG = 1,          /* NULL required pointer, negative or inconsistent size */
    QSA_ERR_UNSUPPORTED = 2,          /* a size outside what the kernels are built for */
    QSA_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < qsa_workspace_bytes(...) */
    QSA_ERR_HIP = 4                   /* the HIP runtime reported an error at launch */
} qsa_status;

/* Bits OR-ed into *error_word by device code (sticky until the caller clears them). */
#define QSA_DEVERR_PAGE_ID    0x1u   /* a page-table entry outside [-1, NP): treated as -1 */
#define QSA_DEVERR_SEQ_LEN    0x2u   /* seq_lens[b] < rows of b, or > MP * P: rows clipped */
#define QSA_DEVERR_ROWS       0x4u   /* row_offsets not non-decreasing, or a request with > max rows */
#define QSA_DEVERR_Q_RANGE    0x8u   /* a q element that is not finite (NaN or +-inf) */
#define QSA_DEVERR_SELECTED   0x10u  /* a selected entry outside [-1, MP): ignored */
#define QSA_DEVERR_SLOT       0x20u  /* a rollback row's slot outside [0, num_slots): skipped */

/* Sizes of one call. Host memory, read during the call only. */
typedef struct qsa_shape {
    int32_t num_requests;          /* B >= 0 */
    int32_t num_rows;              /* N = row_offsets[B] >= 0 (the caller knows it) */
    int32_t max_rows_per_request;  /* 1..1024: upper bound on row_offsets[b+1] - row_offsets[b]
                                      (1 decode, 2..4 MTP verify, more: a context or mixed step;
                                      qsa_kv_store takes 1..4) */
    int32_t num_q_heads;           /* Hq >= 1, a multiple of Hkv */
    int32_t num_kv_heads;          /* Hkv >= 1 */
    int32_t head_dim;              /* d: 64 or 128 */
    int32_t page_size;             /* P: 64 or 128 tokens */
    int32_t max_pages;             /* MP: page-table row stride, 1..4096 */
    int64_t num_phys_pages;        /* NP >= 0: pages in each pool plane */
    int32_t topk;                  /* k >= 0 */
    int32_t window;                /* W >= 0, k + W <= 256 */
    float   sm_scale;              /* softmax scale, normally (float)(1 / sqrt(d)) */
    int32_t kv_format;             /* QSA_KV_NVFP4 (0) or QSA_KV_FP8 (1): the K/V pools' format */
} qsa_shape;

/* K/V pool formats (qsa_shape.kv_format). NVFP4: the layout of qsa_paged below. FP8 (PR
   #20937, the FP8 KV cache of its tested configurations, unit scales): k_codes / v_codes
   are uint8 [NP][Hkv][P][d], one OCP E4M3FN byte per element, K = e4m3 * k_global; the
   scale planes are not read (may be NULL). Only the attention calls take FP8 pools. */
#define QSA_KV_NVFP4 0
#define QSA_KV_FP8   1

/*
 * The paged KV cache. One physical page index addresses every plane (PR #20276, Features,
 * NVFP4 KV cache: codes and scales share the page numbering). Device memory.
 *   page_table  int32 [B][MP]           logical page -> physical page, -1 = no page
 *   seq_lens    int32 [B]               tokens of request b, including this step's rows
 *   row_offsets int32 [B+1]             rows of request b are [row_offsets[b], row_offsets[b+1])
 *   k_codes     uint8 [NP][Hkv][P][d/2] e2m1 codes, element 2i in the low nibble of byte i
 *   k_scales    uint8 [NP][Hkv][P][d/16] OCP E4M3FN scale of elements [16j, 16j+16)
 *   v_codes, v_scales                   as for K
 *   index_keys  bf16  [NP][Hkv][d]      per-page index key (only qsa_index_scores reads it)
 *   k_global, v_global                  fp32 per-tensor scales: K = e2m1 * e4m3 * k_global
 *   error_word  uint32 (device), optional: QSA_DEVERR_* bits are OR-ed into it
 */
typedef struct qsa_paged {
    const int32_t  *page_table;
    const int32_t  *seq_lens;
    const int32_t  *row_offsets;
    const uint8_t  *k_codes;
    const uint8_t  *k_scales;
    const uint8_t  *v_codes;
    const uint8_t  *v_scales;
    const uint16_t *index_keys;
    float           k_global;
    float           v_global;
    uint32_t       *error_word;
} qsa_paged;

/*
 * Index scores (PR #20276, "What runs on the fast paths": index store and compression,
 * then index scores; PR #20937, MTP > Verify: request-tiled index scores).
 *   q       bf16 [N][Hq][d]   (device)
 *   scores  fp32 [N][MP]      (device, written in full)
 * Row j of request b (R_b rows) sees L = seq_lens[b] - (R_b - 1 - j) tokens and
 * n = min(ceil(L / P), MP) pages. For every candidate column p < n - W whose page-table
 * entry is valid:
 *   scores[row][p] = fl32(sm_scale * max_h dot_h),
 *   dot_h = sum_{i ascending} q[row][h][i] * index_keys[phys][h / G][i],
 * with the sum in fp32, rounded after each addition. A zero score is stored as +0.
 * Every other column is -inf. The result is bitwise reproducible.
 * Reads page_table, seq_lens, row_offsets, index_keys.
 */
qsa_status qsa_index_scores(const qsa_shape *shape, const qsa_paged *paged,
                            const uint16_t *q, float *scores, void *stream);

/*
 * Canonical top-k selection plus local window (PR #20276, Features, "Canonical QSA
 * selection" row, and Decisions worth knowing). A row's result depends on its scores, W and
 * k only: candidates scoring above the k-th largest value are kept, equal scores are ranked
 * by descending page index, and the launch order never changes the result.
 *   scores    fp32  [N][MP]     (device)
 *   selected  int32 [N][k + W]  (device, written in full)
 * Per row (n as above): the window is pages [max(0, n - W), n). Candidates are columns
 * p < n - W whose score is neither NaN nor -inf. The row keeps the first min(k, |C|)
 * candidates by (score descending, page index descending), -0 equal to +0, adds the
 * window, and stores them in ascending order followed by -1 padding. Bitwise deterministic.
 * Reads seq_lens and row_offsets (not the page table and not the pools).
 */
qsa_status qsa_select_topk(const qsa_shape *shape, const qsa_paged *paged,
                           const float *scores, int32_t *selected, void *stream);

/*
 * Workspace needed by qsa_sparse_decode for `num_splits` (0 = the library's choice for
 * this shape). Returns 0 when the call needs none (one split). Also 0 for an invalid shape.
 * The workspace holds a region of completion counters of fixed size (32 KiB, one counter per
 * split tile, at most 8192 tiles: a batch with more tiles runs one split per tile), then each
 * split's partial result. The counters must be zero when a call starts: fill a new workspace
 * with zeros once (e.g. hipMemsetAsync) before its first use. Every call leaves them zero
 * again, and their place does not depend on the shape, so a workspace can be reused by later
 * calls of any batch, shape or split count (as long as it is large enough) with no further
 * clearing (also inside captured graphs). Two calls that may overlap in time must not share
 * a workspace.
 */
size_t qsa_workspace_bytes(const qsa_shape *shape, int32_t num_splits);

/*
 * The launch the attention calls make for this shape (host only; nothing is launched).
 * A tile is a run of at most 16 of one request's query columns (its rows x the G q heads of
 * one KV head, row-major); every page any of its rows selected is read once for the tile
 * (PR #20276, Performance > What runs on the fast paths: rows of a request share their K/V
 * page reads). `fused` != 0 describes qsa_select_sparse_decode, 0 qsa_sparse_decode.
 *   tile_cols       query columns per tile (1..16)
 *   rows_per_tile   whole rows per tile (tile_cols / G) when G <= 16; 0 when tiles cut rows
 *   col_tiles       tiles per (request, KV head)
 *   splits          KV splits per tile (as qsa_sparse_decode resolves num_splits)
 *   select_cols     score columns per lane of the fused selection (2, 4, 8 or 16), 0 when
 *                   not fused or when max_pages > 1024 (a separate selection launch runs first)
 *   waves           waves per attention workgroup: 8, or 4 when the tiles hold one row each
 *                   and tiles x splits exceed two per CU (three 4-wave workgroups fit a CU,
 *                   two 8-wave ones)
 *   workgroups      attention workgroups launched
 *   workspace_bytes qsa_workspace_bytes(shape, num_splits)
 * QSA_ERR_INVALID_ARG for a NULL plan, negative num_splits or an invalid shape.
 */
typedef struct qsa_decode_plan {
    int32_t tile_cols;
    int32_t rows_per_tile;
    int32_t col_tiles;
    int32_t splits;
    int32_t select_cols;
    int32_t waves;
    int64_t workgroups;
    size_t  workspace_bytes;
} qsa_decode_plan;

qsa_status qsa_plan_decode(const qsa_shape *shape, int32_t num_splits, int32_t fused, qsa_decode_plan *plan);

/*
 * Split-KV sparse GQA attention over the selected pages, with an LSE merge (PR #20937,
 * What changes: the decode kernel splits the pages and merges the partial results, with a
 * cheaper form for one split; verify rows are grouped by request and merged per row).
 *   q          bf16  [N][Hq][d]     (device)
 *   selected   int32 [N][k + W]     (device; entries outside [0, MP) are ignored, and
 *                                    a page listed twice counts once)
 *   out        bf16  [N][Hq][d]     (device, written in full, RNE)
 *   lse        fp32  [N][Hq]        (device, optional: natural-log sum of exp of the logits)
 *   gate       bf16  [N][Hq][d]     (device, optional, 16-byte aligned: the gated epilogue of
 *                                    PR #20937's verify kernel, out = bf16(o * sigmoid(gate)),
 *                                    o the attention in fp32; lse is not gated)
 *   num_splits 0 = the library's choice; > 0 forces that many KV splits per
 *              (request, KV head), clamped to 64
 *   workspace  device scratch of at least qsa_workspace_bytes(shape, num_splits) bytes,
 *              zero-filled before its first use (see qsa_workspace_bytes)
 * For row j of request b and q head h, the tokens attended are
 *   T = {(p, t): p listed in the row, page_table[b][p] valid, t < P, p * P + t < L}.
 * The output is softmax(sm_scale * k_global * q . K_raw) @ (v_global * V_raw) over T, where
 * K_raw and V_raw are e2m1 * e4m3 (NVFP4) or e4m3 (FP8). An empty T gives out = 0 and lse = -inf. Each request's
 * rows share one read of the union of their selected pages. fp32 accumulation; the q and
 * P operands of the MFMA tiles are f16: each query column's q is scaled by an exact power of
 * two into the f16 range (its largest element in [2^14, 2^15)) and its logits are scaled
 * back, so q of any finite bf16 magnitude is taken as is.
 * Deterministic for a fixed num_splits. sm_scale * k_global * log2(e) must be a positive
 * normal fp32 and v_global finite; otherwise QSA_ERR_INVALID_ARG.
 */
qsa_status qsa_sparse_decode(const qsa_shape *shape, const qsa_paged *paged,
                             const uint16_t *q, const int32_t *selected,
                             uint16_t *out, float *lse, const uint16_t *gate, int32_t num_splits,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * The selection fused into the attention (PR #20276, Performance > What runs on the fast
 * paths: the block top-k runs in the same kernel that turns blocks into tokens; Decisions worth knowing: the
 * fast path produces the canonical rows from one launch). Takes the index scores instead
 * of the selection rows and writes both results: `selected` exactly as qsa_select_topk
 * writes it and `out` / `lse` exactly as qsa_sparse_decode computes them from it, in one
 * launch (two when max_pages > 1024). Arguments as for those calls; `scores` fp32 [N][MP]
 * (device, read only), `selected` int32 [N][k + W] (device, written in full), workspace
 * as for qsa_sparse_decode.
 */
qsa_status qsa_select_sparse_decode(const qsa_shape *shape, const qsa_paged *paged,
                                    const uint16_t *q, const float *scores, int32_t *selected,
                                    uint16_t *out, float *lse, const uint16_t *gate, int32_t num_splits,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. qsa_select_sparse_decode without the
 * workspace arguments: when the launch splits tiles, its counters and split partials live in
 * an 8 MiB device array that the library holds on each GPU it runs on until the process
 * ends (the call itself allocates nothing). Each call clears the counters it uses with a
 * small fill kernel on `stream` before the attention launch. A shape whose split workspace
 * (qsa_workspace_bytes(shape, num_splits)) exceeds 8 MiB returns QSA_ERR_WORKSPACE_TOO_SMALL
 * before any launch; pass num_splits = 1 (no workspace) or use qsa_select_sparse_decode.
 * Every call on one GPU shares that GPU's array: calls that may overlap in time on one GPU
 * (different streams, or graphs replayed concurrently) race and give wrong results. Other
 * arguments, results and errors as for qsa_select_sparse_decode.
 */
qsa_status qsa_select_sparse_decode_static(const qsa_shape *shape, const qsa_paged *paged,
                                           const uint16_t *q, const float *scores, int32_t *selected,
                                           uint16_t *out, float *lse, const uint16_t *gate,
                                           int32_t num_splits, void *stream);

/*
 * The KV-store prologue of a step (PR #20276, Performance > What runs on the fast paths:
 * the decode prologue's index store and compression; PR #20937, What changes: the prologue
 * that writes the NVFP4 KV of a decode step, fused). Writes this step's new tokens into the paged cache and
 * recomputes the index keys of the pages that received them.
 *   new_k, new_v  bf16 [N][Hkv][d]  (device): row j of request b (R_b rows) is the token at
 *                 position seq_lens[b] - R_b + j, i.e. page (pos / P), slot (pos % P)
 * For each new token and KV head, per block of 16 elements x (K with k_global, V with
 * v_global): scale = the E4M3 code nearest to fl32(fl32(amax|x| / 6) / global), ties to the
 * even code, at most 448; code_i = the E2M1 code nearest to fl32(x_i / (e4m3(scale) *
 * global)), ties to the even code, magnitude at most 6 (+0 when it rounds to zero; all 0 when
 * the scale is 0). Then for each page that received a token and each KV head:
 *   index_keys[phys][h][i] = bf16_RNE(fl32(S_i / n)),
 * S_i the fp32 sum, in ascending token order, of the page's stored K (e2m1 * e4m3 * k_global)
 * over its n = min(P, seq_lens[b] - page * P) valid tokens.
 * WRITES through paged->k_codes, k_scales, v_codes, v_scales and index_keys (the caller's
 * device memory; the const in qsa_paged is for the read-only calls). A new token whose page
 * entry is -1 is skipped; one outside [-1, NP) is skipped and sets QSA_DEVERR_PAGE_ID;
 * a position below 0 or at or past max_pages * P (seq_lens[b] < R_b, or too long) is skipped
 * and sets QSA_DEVERR_SEQ_LEN. Pages that receive tokens must not be shared between requests
 * of one call. k_global and v_global must be positive and finite (else QSA_ERR_INVALID_ARG).
 */
qsa_status qsa_kv_store(const qsa_shape *shape, const qsa_paged *paged,
                        const uint16_t *new_k, const uint16_t *new_v, void *stream);

/*
 * Index-plane rollback (PR #20937, Description > What changes > Rollback and PLE: the index
 * planes' writes of rejected rows undone in one batch, by a gather and a restore operation). Before a
 * verify step stores its draft rows, qsa_rollback_gather saves the plane rows those rows
 * will overwrite; after acceptance, qsa_rollback_restore writes the saved bytes back for the
 * rejected rows. Kept rows, and every other byte, stay as the step left them.
 *
 * A plane is caller-owned device memory. Row r of a plane (for step row r) is the nseg
 * segments of seg_bytes bytes at
 *     base + pages[r] * page_stride + within[r] * slot_stride + s * seg_stride,  s < nseg
 * (slot_stride 0: one row per page, such as the index keys). Every row that pages in
 * [0, num_pages) and slots in [0, num_slots) can address must lie in [base, base +
 * plane_bytes), base and all strides and seg_bytes must be multiples of 4; else the call
 * returns QSA_ERR_INVALID_ARG. For the paged cache of this library the planes are
 * k_codes / k_scales / v_codes / v_scales (page_stride Hkv*P*b, slot_stride b, seg_stride
 * P*b, seg_bytes b, nseg Hkv, with b the bytes per token and head) and index_keys
 * (page_stride Hkv*d*2, slot_stride 0, seg_stride d*2, seg_bytes d*2, nseg Hkv).
 */
typedef struct {
    void *base;                /* device */
    int64_t plane_bytes;
    int64_t page_stride;
    int64_t slot_stride;
    int64_t seg_stride;
    int32_t seg_bytes;
    int32_t nseg;
    int64_t num_pages;
    int32_t num_slots;
    int32_t reserved;          /* 0 */
} qsa_plane;

#define QSA_MAX_PLANES 16

/*
 * Stash size for num_rows rows of these planes: plane k's rows are stored contiguously,
 * row r at offset_k + r * row_bytes_k (row_bytes = nseg * seg_bytes), with offset_k the sum
 * over earlier planes of num_rows * row_bytes rounded up to 16 bytes. 0 for invalid input.
 */
size_t qsa_rollback_stash_bytes(const qsa_plane *planes, int32_t num_planes, int32_t num_rows);

/*
 * The (physical page, slot) that each row of a verify step occupies in the paged cache,
 * the placement qsa_kv_store uses: row j of request b (R_b rows, length L) is the token at
 * position L - R_b + j. pages[r] = page_table[b][pos / P] (or -1 when pos < 0, pos / P >=
 * max_pages, or the entry is invalid; an entry outside [-1, NP) sets QSA_DEVERR_PAGE_ID),
 * within[r] = pos % P (0 when the page is -1). pages, within: int32 [N] (device, written).
 */
qsa_status qsa_step_slots(const qsa_shape *shape, const qsa_paged *paged, int32_t *pages,
                          int32_t *within, void *stream);

/*
 * stash[plane k][row r] = row r of plane k, for every row whose page is in [0, num_pages)
 * and slot in [0, num_slots). A row with page -1 is skipped; any other page or slot out of
 * range is skipped and sets QSA_DEVERR_PAGE_ID / QSA_DEVERR_SLOT in error_word (optional).
 * Skipped rows leave their stash bytes unchanged.
 *   pages, within  int32 [num_rows] (device)
 *   stash          device, at least qsa_rollback_stash_bytes bytes, 16-byte aligned
 */
qsa_status qsa_rollback_gather(const qsa_plane *planes, int32_t num_planes, const int32_t *pages,
                               const int32_t *within, int32_t num_rows, void *stash,
                               size_t stash_bytes, uint32_t *error_word, void *stream);

/*
 * Row r of plane k = stash[k][r] for every row with rejected[r] != 0 (rows skipped as in
 * qsa_rollback_gather). rejected: int32 [num_rows] (device). Rows of distinct (page, slot)
 * per plane are written independently; rows that address the same bytes (two step rows in
 * one page of a per-page plane) must carry the same stashed bytes, which a gather of the
 * same rows guarantees.
 */
qsa_status qsa_rollback_restore(const qsa_plane *planes, int32_t num_planes, const int32_t *pages,
                                const int32_t *within, const int32_t *rejected, int32_t num_rows,
                                const void *stash, size_t stash_bytes, uint32_t *error_word,
                                void *stream);

/*
 * Parity hook: NVFP4 dequantisation of whole pages through the same device decode that
 * qsa_sparse_decode uses (the counterpart of the pages' NVFP4 page -> bf16 conversion,
 * PR #20937, qsa_nvfp4_pages_to_bf16).
 *   codes  uint8 [NP][Hkv][P][d/2], scales uint8 [NP][Hkv][P][d/16]   (device)
 *   pages  int32 [num_pages] physical page ids (device; an id outside [0, NP) gives NaN rows)
 *   out    fp32  [num_pages][Hkv][P][d] = fl32(e2m1 * e4m3 * global)  (device)
 * Uses shape->num_kv_heads, head_dim, page_size and num_phys_pages.
 */
qsa_status qsa_nvfp4_dequant_pages(const qsa_shape *shape, const uint8_t *codes,
                                   const uint8_t *scales, float global_scale,
                                   const int32_t *pages, int32_t num_pages, float *out,
                                   void *stream);

/* Static description of a status code. Never NULL. */
const char *qsa_status_string(qsa_status status);

/* QSA_ABI_VERSION of the loaded library. */
int32_t qsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
