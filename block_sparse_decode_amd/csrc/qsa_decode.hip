// qsa_decode.hip -- split-KV sparse GQA attention over NVFP4 (or FP8) pages, with LSE merge.
//
// Method: TensorRT-LLM PR #20937, Description > What changes: the NVFP4 sparse GQA decode
// splits a tile's pages over workgroups and merges their partial softmax results, with a
// cheaper form when one split suffices; verify rows are grouped by request and merged per row,
// with an optional gate on the output; context and mixed steps run as tiles of rows.
// PR #20276, "What runs on the fast paths": the rows of one request that share K/V pages read
// them together.
//
// Work item: a tile is (request b, KV head g, a run of at most 16 of the request's R x G
// query columns, whole rows when G <= 16); each tile is split S ways, one workgroup per
// (tile, split): 8 waves, or 4 for one-row tiles when there are more than two work items per
// CU (three such workgroups fit a CU, so the launch runs in one round). The host picks the
// rows per tile and S (see tile_cols and auto_splits in qsa_api.hip): rows are grouped only
// while that still leaves a tile per CU, since splitting a tile's pages instead costs a merge.
//  1. The tile's rows (at most 4 causal rows: verify rows, or a run of a context step's
//     rows) each list their selected pages (computed here from the scores, one wave per
//     row, when the selection is fused in). The workgroup builds the union of those pages in
//     ascending order, each with a row bitmask, in LDS, and drops entries whose page-table
//     entry is -1. Each page of the union is read once for all the tile's rows. A one-row
//     tile with the selection fused in has its selecting wave publish the union directly
//     (in a 4-wave launch after loading only the row's visible score columns).
//  2. The union's 32-token sub-chunks are numbered page-major. Split s takes a contiguous
//     range of them and its waves deal that range round-robin, so waves differ by at most
//     one sub-chunk. Each wave runs an online softmax over its sub-chunks:
//       S^T = K Q^T   (16x16x32 f16 MFMA; A = K dequantised straight from the global loads,
//                      B = the tile's q columns, from LDS)
//       O^T += V^T P^T (A = V^T read from LDS with ds_read_b64_tr_b16, B = P from the
//                      S^T accumulators, so P never leaves registers)
//     Each lane's column masks tokens past its row's length (causal verify rows) and pages
//     its row did not select.
//  3. The waves merge in a fixed order: each wave publishes the output tiles the others
//     own, and after one barrier wave w sums output tile w over the waves. With one split
//     the workgroup writes the final bf16 output and the LSE (the lean one-split form).
//     Otherwise it writes its partial and bumps the tile's counter; the tile's last split to
//     finish merges all S partials in ascending split order (so the result does not depend
//     on which split is last), writes the output and puts the counter back to zero for the
//     next call.
// Workgroups are dispatched round-robin over the 8 XCDs by linear id; the id -> (tile,
// split) map gives each XCD a contiguous run of (request, KV head, column tile, split)
// items, so a tile's splits, and the tiles of one request and KV head (whose rows share
// their window pages and often more), run on one XCD and share its L2.
// NVFP4 -> f16 and E4M3 -> f16 are exact (see nvfp4_dequant8, fp8x8_to_f16x8). With a gate the
// output is o * sigmoid(gate) before its one bf16 rounding. The global scales fold into the logit scale
// and the output.
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

// A traced build (-DQSA_TRACE) records, per wave of the first kTraceGroups workgroups of each
// launch, the 100 MHz real-time clock at the points of the kernel named in trace_points;
// qsa_trace_read copies them to the host. Lane 0 of each wave keeps its stamps in LDS and
// copies them to the global buffer when the wave leaves: a global store per stamp would
// count in the wave's vector-memory counter, and every later wait for a load would then
// also wait for the stores to be acknowledged. The normal build has neither the stamps nor
// the buffers.
#if defined(QSA_TRACE)
namespace qsa {
constexpr int kTraceGroups = 4096, kTracePoints = 16;
__device__ unsigned long long qsa_trace_stamps[kTraceGroups * 8 * kTracePoints];
__shared__ unsigned long long qsa_trace_lds[8][kTracePoints];
__device__ __forceinline__ void trace_clear()
{
    const unsigned t = threadIdx.x;
    if ((t & 63u) == 0u)
        for (int k = 0; k < kTracePoints; ++k) qsa_trace_lds[t >> 6][k] = 0ull;
}
__device__ __forceinline__ void trace_stamp(int k)
{
    const unsigned t = threadIdx.x;
    if ((t & 63u) == 0u) qsa_trace_lds[t >> 6][k] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void trace_flush()
{
    const unsigned t = threadIdx.x;
    if ((t & 63u) == 0u && blockIdx.x < (unsigned)kTraceGroups)
        for (int k = 0; k < kTracePoints; ++k)
            qsa_trace_stamps[((size_t)blockIdx.x * 8 + (t >> 6)) * kTracePoints + k] = qsa_trace_lds[t >> 6][k];
}
}  // namespace qsa
#define QSA_STAMP(k) qsa::trace_stamp(k)
#define QSA_TRACE_BEGIN() qsa::trace_clear()
#define QSA_TRACE_END() qsa::trace_flush()
#else
#define QSA_STAMP(k) ((void)0)
#define QSA_TRACE_BEGIN() ((void)0)
#define QSA_TRACE_END() ((void)0)
#endif
#define QSA_SELECT_STAMP(k) QSA_STAMP(k)

#include "qsa_select_row.hpp"

namespace qsa {

constexpr int kMaxUnion = 1024;     // rows (<= 4) x (k + W) (<= 256)
constexpr int kMaxPages = 4096;     // page-table stride MP
constexpr int kTileRows = 4;        // rows of a multi-row tile
constexpr int kXcds = kXcdCount;

__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Cache formats: NVFP4 (e2m1 codes, two per byte, plus one e4m3 scale per 16 elements) and
// FP8 (one e4m3 byte per element, unit scales).
constexpr int kNvfp4 = 0, kFp8 = 1;

template <int D, int F>
constexpr int code_bytes() { return F == kFp8 ? D : D / 2; }       // per token and KV head
template <int D, int F>
constexpr int scale_bytes() { return F == kFp8 ? 0 : D / 16; }

template <int D, int F>
struct RawTile;   // one lane's share of a 16-token M-tile: its d/4 consecutive elements

template <>
struct RawTile<128, kNvfp4> {
    uint4 codes;        // 32 e2m1 codes
    uint32_t scales;    // 2 e4m3 bytes in the low half
};

template <>
struct RawTile<64, kNvfp4> {
    uint2 codes;        // 16 e2m1 codes
    uint32_t scales;    // 1 e4m3 byte
};

template <>
struct RawTile<128, kFp8> {
    uint4 lo, hi;       // 32 e4m3 bytes
};

template <>
struct RawTile<64, kFp8> {
    uint4 lo;           // 16 e4m3 bytes
};

// `codes` / `scales`: the sub-chunk's first token (wave-uniform); `co` / `so`: this lane's
// byte offsets from there (token li of the M-tile, chunk gq), so each load is a uniform
// 64-bit base plus a 32-bit lane offset with no per-load vector address arithmetic.
template <int D, int F>
__device__ __forceinline__ RawTile<D, F> load_raw(const uint8_t *codes, const uint8_t *scales, uint32_t co, uint32_t so)
{
    RawTile<D, F> t;
    if constexpr (F == kFp8) {
        t.lo = *reinterpret_cast<const uint4 *>(codes + co);
        if constexpr (D == 128) t.hi = *reinterpret_cast<const uint4 *>(codes + co + 16);
    } else if constexpr (D == 128) {
        t.codes = *reinterpret_cast<const uint4 *>(codes + co);
        t.scales = *reinterpret_cast<const uint16_t *>(scales + so);
    } else {
        t.codes = *reinterpret_cast<const uint2 *>(codes + co);
        t.scales = scales[so];
    }
    return t;
}

template <int D>
__device__ __forceinline__ uint32_t raw_dword(const RawTile<D, kNvfp4> &t, int i)
{
    if constexpr (D == 128) {
        return i == 0 ? t.codes.x : i == 1 ? t.codes.y : i == 2 ? t.codes.z : t.codes.w;
    } else {
        return i == 0 ? t.codes.x : t.codes.y;
    }
}

// Eight e4m3 bytes (two dwords) -> eight f16 values, exactly (every E4M3FN value is an f16
// value); the scaled convert applies only its scale's exponent, so scale 1.0 is a plain decode.
__device__ __forceinline__ f16x8 fp8x8_to_f16x8(uint32_t a, uint32_t b)
{
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, false);
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, true);
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false);
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true);
    return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                   __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

// Dequantise a lane's 8-element group i (elements 8i..8i+7 of its d/4 chunk); for NVFP4 `sc`
// holds the chunk's block scales as f16 ({s0, s1} for d = 128, {s0, -} for d = 64).
template <int D, int F>
__device__ __forceinline__ f16x8 dequant_group(const RawTile<D, F> &t, f16x2 sc, int i)
{
    if constexpr (F == kFp8) {
        if constexpr (D == 128) {
            const uint4 &h = i < 2 ? t.lo : t.hi;
            return (i & 1) ? fp8x8_to_f16x8(h.z, h.w) : fp8x8_to_f16x8(h.x, h.y);
        } else {
            return (i & 1) ? fp8x8_to_f16x8(t.lo.z, t.lo.w) : fp8x8_to_f16x8(t.lo.x, t.lo.y);
        }
    } else {
        return nvfp4_dequant8(raw_dword<D>(t, i), (D == 128 && i >= 2) ? sc.y : sc.x);
    }
}

template <int D, int F>
__device__ __forceinline__ f16x2 tile_scales(const RawTile<D, F> &t)
{
    if constexpr (F == kFp8) {
        return (f16x2){(half_t)1.0f, (half_t)1.0f};
    } else {
        return e4m3x2_to_f16x2(t.scales);
    }
}

template <int D, int F>
__device__ __forceinline__ void load_unit(const DecodeParams &prm, int phys, int g, int c, uint32_t co, uint32_t so,
                                          RawTile<D, F> (&kr)[2], RawTile<D, F> (&vr)[2])
{
    constexpr int CB = code_bytes<D, F>(), SB = scale_bytes<D, F>();
    // the sub-chunk's first token in the pool (phys, g and c are wave-uniform)
    const int64_t tok = ((int64_t)phys * prm.Hkv + g) * prm.P + c * 32;
    const uint8_t *kc = prm.k_codes + tok * CB, *vc = prm.v_codes + tok * CB;
    const uint8_t *ks = SB ? prm.k_scales + tok * SB : nullptr, *vsc = SB ? prm.v_scales + tok * SB : nullptr;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const uint32_t cm = co + mt * 16 * CB, sm = so + mt * 16 * SB;
        kr[mt] = load_raw<D, F>(kc, ks, cm, sm);
        vr[mt] = load_raw<D, F>(vc, vsc, cm, sm);
    }
}

// V staging in LDS: row t (token) holds D f16 values as D/8 chunks of 16 bytes; chunk ch of
// row t is stored at chunk position ch ^ swz(t). Measured on gfx950 (LDS bank-conflict
// counters against two layouts), the 16-byte writes are served 8 lanes (one chunk of 8
// aligned consecutive rows) per cycle and the transposed 8-byte reads 32 lanes (8 aligned
// rows x chunks {2j, 2j + 1}) per cycle. swz(t) = (2t + t/4 mod 2) mod 16 takes 8 different
// values mod 8 on 8 aligned rows, and 8 different values of swz >> 1 mod 8 on them, so
// neither access conflicts (d = 128; at d = 64 two rows share a 256-byte line).
__device__ __forceinline__ int vswz(int row) { return ((row << 1) + ((row >> 2) & 1)) & 15; }

// A wave's position in its split's range of sub-chunks. Sub-chunk u is sub-chunk
// u mod (P/32) of union entry u / (P/32); sub-chunks that no row of the tile can see (past
// the longest row's length), and those of an entry without a valid physical page, are skipped.
struct UnitCursor {
    int u, c;
    uint32_t pm;
    int phys;
    bool have;
};

template <int NW>
__device__ __forceinline__ UnitCursor seek_unit(int u, int u_hi, int lc, const uint32_t *u_pm,
                                                const int32_t *u_phys)
{
    UnitCursor r;
    r.have = false;
    r.c = 0;
    r.pm = 0u;
    r.phys = 0;
    for (; u < u_hi; u += NW) {
        // the entry's physical page is read beside its page word, whether or not the unit
        // turns out visible: one LDS round trip instead of two
        const uint32_t pm = __builtin_amdgcn_readfirstlane(u_pm[u >> lc]);
        const int32_t ph = __builtin_amdgcn_readfirstlane(u_phys[u >> lc]);
        const int c = u & ((1 << lc) - 1);
        if (c < (int)(pm >> 24) && ph >= 0) {        // (an entry without a valid page holds -1)
            r.have = true;
            r.c = c;
            r.pm = pm;
            r.phys = ph;
            break;
        }
    }
    r.u = u;
    return r;
}

// SELC = 0: the rows' selections are an input. SELC = 2, 4, 8 or 16: they are computed here
// from the scores (select_row with that many columns per lane) and also written out.
// ONE: every tile holds columns of one row only (one-row tiles, or 16-column tiles of rows
// of a multiple of 16 q heads), which the host knows from the launch shape. That form has a
// shorter prologue of its own, and its instantiation carries none of the multi-row union
// build, which leaves the compiler more registers for the rest.
// Occupancy: LDS allows two workgroups per CU. The one-row form is allowed up to 256
// registers per lane but takes about 126, so two of its workgroups still fit a CU; the
// general form is held to 128.
template <int D, int SELC, int F, bool ONE, int NWV>
__global__ __launch_bounds__(NWV * 64, ONE ? (NWV == 4 ? 3 : 2) : 4) void sparse_decode_kernel(DecodeParams prm)
{
    constexpr int NW = NWV;
    constexpr int NT = NW * 64;
    constexpr int KS = D / 32;              // k-steps of S^T = K Q^T
    constexpr int DQ = D / 4;               // elements per lane group
    constexpr int NDT = D / 16;             // 16-row d tiles of O^T
    // A column's running max is raised only when a logit exceeds it by more than this
    // (log2 units), so most sub-chunks skip the rescale; P stays <= 2^8 in f16.
    constexpr float kLazy = 8.0f;
    static_assert(NDT * 64 * 16 <= 32 * D * 2, "a wave's O^T tiles must fit its V staging tile");
    static_assert(NW == kDecodeWaves || (ONE && NW == 4), "4-wave workgroups are built for one-row tiles only");
    static_assert(SELC <= 32, "a one-row tile's selection mask is kept in 32 bits");
    static_assert(D / 8 <= 16, "one V row holds at most 16 swizzled chunks");

    // One LDS area: the union build's scratch (row-mask bitmap, page-table row), then the
    // per-wave V staging tiles, then the wave merge slots.
    constexpr int kStageBytes = NW * 32 * D * 2;
    constexpr int kScratchBytes = 4 * (kMaxPages / 4 + kMaxPages);
    __shared__ __attribute__((aligned(16))) char lds_area[kStageBytes > kScratchBytes ? kStageBytes : kScratchBytes];
    half_t(*vsm)[32 * D] = reinterpret_cast<half_t(*)[32 * D]>(lds_area);
    __shared__ uint32_t u_pm[kMaxUnion];    // page | row mask << 16 | sub-chunks << 24
    __shared__ int32_t u_phys[kMaxUnion];
    __shared__ float ml_m[NW][16];         // per wave: column maxima (log2 units)
    __shared__ float ml_l[NW][16];         // per wave: softmax denominators
    __shared__ uint32_t scan_tmp[NT / 64 + 1];
    __shared__ f16x8 q_lds[KS][64];         // the tile's q operand, in MFMA B-operand lane order
    __shared__ int q_col_exp[16];           // per query column: its q operand is q * 2^-e

    // The kernel arguments the prologue needs, all in scalar registers before anything waits
    // on one: each first read of an argument's cache line misses the scalar cache at launch,
    // and reading them where they are first used would chain several such misses (one per
    // dependent step of the work-item arithmetic) before the first global load could issue.
    asm volatile("" ::"s"(prm.tiles), "s"(prm.splits), "s"(prm.div_splits.m), "s"(prm.div_splits.l),
                 "s"(prm.col_tiles), "s"(prm.Hkv), "s"(prm.div_htiles.m), "s"(prm.div_htiles.l),
                 "s"(prm.div_ctiles.m), "s"(prm.div_ctiles.l), "s"(prm.row_offsets), "s"(prm.seq_lens),
                 "s"(prm.uniform_rows), "s"(prm.rmax), "s"(prm.N), "s"(prm.tile_cols), "s"(prm.div_group.d),
                 "s"(prm.div_group.m), "s"(prm.div_group.l), "s"(prm.MP), "s"(prm.KW), "s"(prm.page_table));
    asm volatile("" ::"s"(SELC > 0 ? (const void *)prm.scores : (const void *)prm.selected), "s"(prm.q),
                 "s"(prm.Hq), "s"(prm.log2P), "s"(prm.k), "s"(prm.W), "s"(prm.NP), "s"(prm.P));
    // work item i = tile * S + split, tiles numbered (request, KV head, column tile); XCD x
    // (the dispatcher's linear id mod 8) takes the contiguous items [x * per, (x + 1) * per)
    const int S = prm.splits;
    // (tiles * S < 2^30, so the item arithmetic fits 32 bits; the divisors are the host's)
    const uint32_t n_items = (uint32_t)prm.tiles * (uint32_t)S;
    const uint32_t per = (n_items + kXcds - 1) / kXcds;
    const uint32_t wg = blockIdx.x;
    const uint32_t item = (wg % kXcds) * per + wg / kXcds;
    if (item >= n_items) return;
    QSA_TRACE_BEGIN();
    QSA_STAMP(0);
    const int tile = (int)fast_div(item, prm.div_splits), s = (int)item - tile * S;
    const int T = prm.col_tiles;
    const int HT = prm.Hkv * T;
    const int b = (int)fast_div((uint32_t)tile, prm.div_htiles);
    const int g = (int)fast_div((uint32_t)(tile - b * HT), prm.div_ctiles), ct = tile - b * HT - g * T;
    // The request's row range and length. When every request has rmax rows (num_rows is
    // B * rmax, which the host knows) the range is [b * rmax, (b + 1) * rmax) without a load,
    // so the loads that depend on it issue at once; the row offsets are then only compared with
    // it, off the critical path, by one thread per request. Otherwise both offsets are loaded
    // before either is waited on.
    const int tid = threadIdx.x, lane = tid & 63;
    const bool checker = tid == 0 && s == 0 && tile == b * HT;
    int r0, r1, ro_check0 = 0, ro_check1 = 0;
    if (prm.uniform_rows) {
        r0 = b * prm.rmax;
        r1 = r0 + prm.rmax;
        if (checker) {
            ro_check0 = prm.row_offsets[b];
            ro_check1 = prm.row_offsets[b + 1];
        }
    } else {
        r0 = prm.row_offsets[b];
        r1 = prm.row_offsets[b + 1];
    }
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave-uniform, so in SGPRs
    const int gq = lane >> 4, li = lane & 15;
    const int R = clip_rows(r0, r1, prm.N, prm.rmax, prm.err, checker);
    if (R >= 0) QSA_STAMP(1);           // (the condition makes the stamp wait for the row range)
    const int Rb = r1 - r0;         // the request's own row count fixes each row's length
    const int G = (int)prm.div_group.d;
    const int TW = prm.tile_cols;   // this tile: columns col0 .. col0 + TW - 1 of the request's R x G
    const int col0 = ct * TW;
    if (col0 >= R * G) {
        QSA_TRACE_END();
        return;
    }
    const int j_lo = (int)fast_div((uint32_t)col0, prm.div_group);
    const int j_hi = min(R - 1, (int)fast_div((uint32_t)(col0 + TW - 1), prm.div_group));
    const int nrow = j_hi - j_lo + 1;                // rows of this tile (<= 4)
    const int MP = prm.MP, P = prm.P, KW = prm.KW;

    // ---- 1. union of the tile's rows' selected pages; the q operand ------------------
    // All threads stage this request's page-table row in LDS (scratch in the V staging
    // area, with a row-mask bitmap of one byte per page) while the selecting waves load their
    // score rows (or every thread its share of the selection rows) and the last wave loads q,
    // so the union costs one dependent global round trip. After the first barrier every
    // thread marks its entries' pages in the bitmap, and after a second one wave 0 lists the
    // marked pages. The last wave converts q into the MFMA B operand in LDS before the first
    // barrier. Union order: ascending page, as for one-row tiles.
    // A one-row tile with the selection fused in takes a shorter way: wave 1 copies the
    // page-table entries of the row's columns into LDS while the selecting wave selects, and
    // after the barrier every thread places its share of the selected pages (ascending) in
    // the union, so neither the bitmap nor the union build and its barrier are needed. One-row
    // unions keep a selected page without a valid physical page in its place, with -1 for its
    // physical page, and the loop skips its sub-chunks.
    const int nwords = ((MP + 3) / 4 + 3) & ~3;
    uint32_t *bm = reinterpret_cast<uint32_t *>(lds_area);
    int32_t *pt_row = reinterpret_cast<int32_t *>(bm + nwords);
    const int nent = nrow * KW;                      // <= kMaxUnion
    // the selection entries a thread holds: one row's k + W <= 256 entries over wave 0's lanes
    // (one-row tiles), or the tile's nrow * (k + W) <= 1024 entries over all 512 threads
    constexpr int kSelPerLane = ONE ? 256 / 64 : kMaxUnion / NT;
    int selp[kSelPerLane];
    int32_t *sel_lds = reinterpret_cast<int32_t *>(u_pm);   // the selections, before the union
    constexpr bool one_row = ONE && SELC > 0;        // fused selection, one row per tile
    // one-row fused selection: per-lane masks and prefix counts (in wave 2's V staging tile)
    // and the page-table entries of the row's columns (in wave 1's), until the union is placed
    uint32_t *one_pub = reinterpret_cast<uint32_t *>(lds_area + 2 * (32 * D * 2));
    int32_t *one_pt = reinterpret_cast<int32_t *>(lds_area + 1 * (32 * D * 2));
    static_assert(SELC <= 16 && 64 * SELC * 4 <= 32 * D * 2, "one-row publish areas");
    constexpr bool lean_one = ONE && SELC == 0;      // selection given, one row per tile

    // The independent global loads go first, so that no wave waits for one of them before
    // issuing the next: each selecting wave's score row (or wave 0's selection rows), the
    // last wave's q columns, then every thread's page-table entries (whose LDS stores wait).
    uint32_t skey[SELC > 0 ? SELC : 8];
    // A launch of 4-wave workgroups (more than two items per CU) starts three workgroups per CU
    // at once, and their prologue loads (score rows, page-table rows, q) queue behind each
    // other. There the request's length comes first, so that the score row and the page-table
    // copy cover only the row's visible columns (the others are never candidates and never
    // selected): one more round trip ahead of the score loads, fewer bytes in the queue. On the
    // wide mixed batch (lengths of 16 to 1024 pages) the fused launch went from 45.3 to 43.8 us;
    // 8-wave launches keep the length behind the score loads.
    constexpr bool vis_first = one_row && NW == 4;
    int nvis = MP;                                  // the row's visible pages (vis_first)
    int64_t Lb_first = 0;
    if constexpr (vis_first) {
        Lb_first = prm.seq_lens[b];
        nvis = row_geom(Lb_first, r1 - r0, j_lo, prm.log2P, MP).pages;
    }
    if constexpr (SELC == 0) {
#pragma unroll
        for (int i = 0; i < kSelPerLane; ++i) {
            const int idx = ONE ? lane + i * 64 : tid + i * NT;
            selp[i] = -1;
            if ((ONE ? wave == 0 : true) && idx < nent) {
                const int jr = (int)fast_div((uint32_t)idx, prm.div_kw);
                selp[i] = prm.selected[(int64_t)(r0 + j_lo + jr) * KW + (idx - jr * KW)];
            }
        }
    } else if constexpr (vis_first) {
        if (wave == 0) {
            if (lane * SELC < nvis) {
                select_row_load<SELC>(prm.scores + (int64_t)(r0 + j_lo) * MP, MP, skey);
            } else {
#pragma unroll
                for (int i = 0; i < SELC; ++i) skey[i] = 0u;   // past the row: no candidate
            }
        }
    } else {
        if (wave < nrow) select_row_load<SELC>(prm.scores + (int64_t)(r0 + j_lo + wave) * MP, MP, skey);
    }
    // One-row tiles with the selection fused in: wave 1 copies the page-table entries of the
    // row's columns into LDS (one_pt, in the selecting wave's column order), so that the
    // selecting wave waits for its score row alone. The entries of the selected columns are
    // read after the barrier.
    if constexpr (one_row) {
        if (wave == 1 && lane * SELC < nvis) {
            const int c0 = lane * SELC;
            const int32_t *ptr = prm.page_table + (int64_t)b * MP;
            if (SELC >= 4 && (MP & 3) == 0 && c0 + SELC <= MP) {
                // 16-byte loads (the table and its rows are 16-byte aligned when MP is a
                // multiple of 4)
                const int4 *v = reinterpret_cast<const int4 *>(ptr + c0);
                int4 *d = reinterpret_cast<int4 *>(one_pt + c0);
#pragma unroll
                for (int j = 0; j < SELC / 4; ++j) d[j] = v[j];
            } else {
                // one clamped load per column; columns past the row are never selected
#pragma unroll
                for (int i = 0; i < SELC; ++i) {
                    const int c = c0 + i;
                    one_pt[c] = ptr[c < MP ? c : 0];
                }
            }
        }
    }
    // this lane's query column
    const int col = col0 + li;
    const int jc = (int)fast_div((uint32_t)col, prm.div_group);   // row of this lane's column
    const bool colv = li < TW && jc < R;              // false: padding column
    uint4 qraw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = make_uint4(0u, 0u, 0u, 0u);
    if (wave == NW - 1 && colv) {
        const int h = g * G + (col - jc * G);
        const uint4 *qp = reinterpret_cast<const uint4 *>(prm.q + ((int64_t)(r0 + jc) * prm.Hq + h) * D + gq * DQ);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qraw[ks] = qp[ks];
    }
    // the request's length: loaded only now, after the loads above have issued, so that
    // waiting for it does not hold them back (nothing above needs it), except in a 4-wave
    // launch, which loaded it first
    const int64_t Lb = vis_first ? Lb_first : (int64_t)prm.seq_lens[b];
    if constexpr (!ONE) {
        for (int w = tid; w < nwords; w += NT) bm[w] = 0u;
        for (int p = tid; p < MP; p += NT) pt_row[p] = prm.page_table[(int64_t)b * MP + p];
    }
    if constexpr (lean_one) {
        if (wave == 0) {
            // The row's listed visible pages, deduplicated and in ascending order (the order the
            // fused selection lists them in). Each one's page-table entry is loaded at once (one
            // dependent round trip for all of them); the pages set their bit in a bitmap over the
            // table and store their physical page beside it; the set bits, read back in ascending
            // order with a prefix count for the positions, are the union. A page without a valid
            // physical page keeps its place with -1 for it, as in the fused selection, so both
            // calls give their waves the same sub-chunks. Wave 0 alone, so no workgroup barrier.
            const RowGeom geo = row_geom(Lb, Rb, j_lo, prm.log2P, MP);
            uint32_t *okmap = reinterpret_cast<uint32_t *>(lds_area);          // kMaxPages bits
            int32_t *phys_of = reinterpret_cast<int32_t *>(okmap + kMaxPages / 32);
            const int nbw = (MP + 31) >> 5;
            int phv[kSelPerLane];
#pragma unroll
            for (int i = 0; i < kSelPerLane; ++i) {
                const int p = selp[i];
                const bool vis = lane + i * 64 < nent && p >= 0 && p < geo.pages;
                phv[i] = vis ? prm.page_table[(int64_t)b * MP + p] : -1;
            }
            for (int w = lane; w < nbw; w += 64) okmap[w] = 0u;
            wave_lds_fence();
            const uint32_t npc = prm.NP < ((int64_t)1 << 31) ? (uint32_t)prm.NP : 0x80000000u;
#pragma unroll
            for (int i = 0; i < kSelPerLane; ++i) {
                if (lane + i * 64 >= nent) continue;
                const int p = selp[i];
                if (p < -1 || p >= MP) {
                    set_error(prm.err, QSA_DEVERR_SELECTED);
                    continue;
                }
                const int ph = phv[i];
                if (p < 0 || p >= geo.pages) continue;
                if (ph != -1 && (uint32_t)ph >= npc) set_error(prm.err, QSA_DEVERR_PAGE_ID);
                phys_of[p] = ph;                          // duplicates store the same value
                atomicOr(&okmap[p >> 5], 1u << (p & 31));
            }
            wave_lds_fence();
            constexpr int kWordsPerLane = kMaxPages / 32 / 64;
            uint32_t wm[kWordsPerLane];
            uint32_t cnt = 0u;
#pragma unroll
            for (int t = 0; t < kWordsPerLane; ++t) {
                const int wi = lane * kWordsPerLane + t;
                wm[t] = wi < nbw ? okmap[wi] : 0u;
                cnt += (uint32_t)__builtin_popcount(wm[t]);
            }
            const uint32_t incl = wave_inclusive_scan(cnt);
            uint32_t pos = incl - cnt;
            const int lenc = (int)min(geo.len, (int64_t)MP << prm.log2P);
#pragma unroll
            for (int t = 0; t < kWordsPerLane; ++t) {
                uint32_t m = wm[t];
                while (m) {
                    const int p = (lane * kWordsPerLane + t) * 32 + __builtin_ctz(m);
                    m &= m - 1u;
                    const int vis = lenc - (p << prm.log2P);
                    const int nc = vis >= P ? P / 32 : (vis + 31) / 32;
                    u_pm[pos] = (uint32_t)p | (1u << 16) | ((uint32_t)nc << 24);
                    const int32_t ph = phys_of[p];
                    u_phys[pos] = (uint32_t)ph < npc ? ph : -1;
                    ++pos;
                }
            }
            if (lane == 63) scan_tmp[0] = incl;
        }
    }
    if constexpr (SELC > 0) {
        if constexpr (one_row) {
            if (wave == 0) {
                // The row's selection is placed by the whole workgroup after the barrier: a
                // single wave placing every column itself would take hundreds of instructions
                // while the other waves wait. This wave publishes, per lane, its columns'
                // selection mask and its prefix count over the lanes.
                const RowGeom geo = row_geom(Lb, Rb, j_lo, prm.log2P, MP);
                const uint32_t take = (uint32_t)select_row_take<SELC>(skey, geo.pages, prm.k, prm.W);
                QSA_STAMP(4);
                const uint32_t cnt = (uint32_t)__builtin_popcount(take);
                const uint32_t incl = wave_inclusive_scan(cnt);
                one_pub[lane] = take;
                one_pub[64 + lane] = incl - cnt;
                if (lane == 63) {
                    scan_tmp[0] = incl;          // union entries: the selected pages
                    scan_tmp[1] = incl;          // selection length
                }
                QSA_STAMP(5);
            }
        } else if (wave < nrow) {
            // wave w selects the tile's row j_lo + w, into LDS
            select_row_keys<SELC>(skey, row_geom(Lb, Rb, j_lo + wave, prm.log2P, MP).pages, prm.k, prm.W,
                                  sel_lds + wave * KW);
        }
    }
    if (wave == NW - 1) {
        // q into the f16 MFMA operand, each query column scaled by an exact power of two 2^-e
        // that puts its largest |element| in [2^14, 2^15): no finite bf16 q overflows f16, and
        // small columns keep all their bits. The column's logit scale takes the 2^e back
        // (q_col_exp), so every logit is the same number as without the scaling. e is clamped
        // so that the column's logit scale stays a normal fp32. A non-finite q element sets
        // QSA_DEVERR_Q_RANGE (and propagates as in any arithmetic).
        float f[KS][8];
        float amax = 0.0f;
        bool qbad = false;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 raw = qraw[ks];
            f[ks][0] = bf16lo(raw.x); f[ks][1] = bf16hi(raw.x); f[ks][2] = bf16lo(raw.y); f[ks][3] = bf16hi(raw.y);
            f[ks][4] = bf16lo(raw.z); f[ks][5] = bf16hi(raw.z); f[ks][6] = bf16lo(raw.w); f[ks][7] = bf16hi(raw.w);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                qbad |= !(fabsf(f[ks][t]) <= 3.4028234663852886e38f);
                amax = fmaxf(amax, fabsf(f[ks][t]));
            }
        }
        amax = max_across_groups(amax);                 // the column's four lanes
        int e = 0;
        if (amax > 0.0f && amax <= 3.4028234663852886e38f) {
            int ea, ec;
            (void)frexpf(amax, &ea);                    // amax in [2^(ea-1), 2^ea)
            (void)frexpf(prm.qk_scale_log2, &ec);
            e = min(max(ea - 1 - 14, -125 - ec), 126 - ec);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            f16x8 v;
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = (half_t)ldexpf(f[ks][t], -e);
            q_lds[ks][lane] = v;
        }
        if (gq == 0) q_col_exp[li] = e;
        if (qbad) set_error(prm.err, QSA_DEVERR_Q_RANGE);
    }
    QSA_STAMP(6);
    __syncthreads();
    QSA_STAMP(7);
    if constexpr (one_row) {
        // every thread places up to four of the row's columns (64 * SELC <= 1024) in the
        // selection row (ascending, in wave 0's V staging tile) and in the union. The union
        // lists every selected page at the same position; a page without a valid physical page
        // has -1 for it (the loop skips its sub-chunks), and one outside the pool also sets the
        // error.
        const int lenc = (int)min(row_geom(Lb, Rb, j_lo, prm.log2P, MP).len, (int64_t)MP << prm.log2P);
        const uint32_t npc = prm.NP < ((int64_t)1 << 31) ? (uint32_t)prm.NP : 0x80000000u;
        int32_t *sel_row = reinterpret_cast<int32_t *>(lds_area);
        // a fixed number of columns per thread, so that all their mask reads issue before the
        // first is used (one LDS round trip for them, one more for the few selected ones)
        constexpr int kPlace = (64 * SELC + NT - 1) / NT;
        uint32_t tks[kPlace];
#pragma unroll
        for (int k = 0; k < kPlace; ++k) {
            const int c = tid + k * NT;
            tks[k] = c < 64 * SELC ? one_pub[c / SELC] : 0u;
        }
#pragma unroll
        for (int k = 0; k < kPlace; ++k) {
            const int c = tid + k * NT, ol = c / SELC, i = c % SELC;
            const uint32_t tk = tks[k];
            if ((tk >> i) & 1u) {
                const int pos = (int)(one_pub[64 + ol] + (uint32_t)__builtin_popcount(tk & ((1u << i) - 1u)));
                sel_row[pos] = c;
                const int vis = lenc - (c << prm.log2P);
                const int nc = vis >= P ? P / 32 : (vis + 31) / 32;
                u_pm[pos] = (uint32_t)c | (1u << 16) | ((uint32_t)nc << 24);
                const int32_t ph = one_pt[c];
                const bool valid = (uint32_t)ph < npc;
                if (!valid && ph != -1) set_error(prm.err, QSA_DEVERR_PAGE_ID);
                u_phys[pos] = valid ? ph : -1;
            }
        }
        __syncthreads();
        QSA_STAMP(12);
    }
    if (one_row && wave == 0 && g == 0 && s == 0 && col0 <= j_lo * G) {
        // the row's selection, ascending, then -1 padding (before this wave's V staging
        // reuses the LDS copy)
        const int32_t *sel_row = reinterpret_cast<const int32_t *>(lds_area);
        const int nsel = (int)scan_tmp[1];
        int32_t *dst = prm.selected + (int64_t)(r0 + j_lo) * KW;
        for (int i = lane; i < KW; i += 64) dst[i] = i < nsel ? sel_row[i] : -1;
        wave_lds_fence();
    }
    if constexpr (!ONE) {
        // The union of the tile's rows, in two steps. Every thread marks up to two of the tile's
        // nrow * (k + W) selection entries: a listed page that its row can see and whose
        // page-table entry is a valid physical page sets the row's bit in the page's byte of the
        // bitmap (a page listed twice sets it twice). Then wave 0 lists the marked pages in
        // ascending order, each with its row mask and the sub-chunks its longest requesting row
        // can see, with a wave prefix count per 64 words of the bitmap for the positions.
        // The rows' page counts and lengths are the same for every entry, so they are taken once.
        int rpages[kTileRows], rlen[kTileRows];
        const int64_t lfull_p = (int64_t)MP << prm.log2P;
#pragma unroll
        for (int r = 0; r < kTileRows; ++r) {
            const RowGeom geo = row_geom(Lb, Rb, j_lo + min(r, nrow - 1), prm.log2P, MP);
            rpages[r] = geo.pages;
            rlen[r] = (int)min(geo.len, lfull_p);
        }
        auto of_row = [&](const int (&v)[kTileRows], int r) {
            return r == 0 ? v[0] : r == 1 ? v[1] : r == 2 ? v[2] : v[3];
        };
        const uint32_t npc = prm.NP < ((int64_t)1 << 31) ? (uint32_t)prm.NP : 0x80000000u;
#pragma unroll
        for (int i = 0; i < kSelPerLane; ++i) {
            const int idx = tid + i * NT;
            if (idx >= nent) break;
            const int jr = (int)fast_div((uint32_t)idx, prm.div_kw);
            int p;
            if constexpr (SELC > 0) {
                p = sel_lds[idx];
                // this workgroup publishes the rows that start in its tile (KV head 0, split 0)
                if (g == 0 && s == 0 && col0 <= (j_lo + jr) * G)
                    prm.selected[(int64_t)(r0 + j_lo + jr) * KW + (idx - jr * KW)] = p;
            } else {
                p = selp[i];
            }
            if (p < -1 || p >= MP) {
                set_error(prm.err, QSA_DEVERR_SELECTED);
                continue;
            }
            if (p < 0 || p >= of_row(rpages, jr)) continue;      // no visible token
            const int phys = pt_row[p];
            if (phys == -1) continue;
            if ((uint32_t)phys >= npc) {                          // below -1 or past the pool
                set_error(prm.err, QSA_DEVERR_PAGE_ID);
                continue;
            }
            atomicOr(&bm[p >> 2], 1u << ((p & 3) * 8 + jr));
        }
        __syncthreads();             // every mark is in; the selections' LDS copy is read
        if (wave == 0) {
            const int nw = (MP + 3) / 4;                          // bitmap words, 4 pages each
            uint32_t base = 0u;
            for (int t = 0; t * 64 < nw; ++t) {
                const int wi = t * 64 + lane;
                const uint32_t x = wi < nw ? bm[wi] : 0u;
                uint32_t y = x | (x >> 4);
                y |= y >> 2;
                y |= y >> 1;
                y &= 0x01010101u;                                 // bit 8k: page 4 wi + k is marked
                const uint32_t cnt = (uint32_t)__builtin_popcount(y);
                const uint32_t incl = wave_inclusive_scan(cnt);
                uint32_t pos = base + incl - cnt;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t m = (x >> (8 * k)) & 0xffu;
                    if (m == 0u) continue;
                    const int p = wi * 4 + k;
                    const int jmax = 31 - __builtin_clz(m);            // later rows see more tokens
                    const int vis = of_row(rlen, jmax) - (p << prm.log2P);
                    const int nc = vis >= P ? P / 32 : (vis + 31) / 32;
                    u_pm[pos] = (uint32_t)p | (m << 16) | ((uint32_t)nc << 24);
                    u_phys[pos] = pt_row[p];
                    ++pos;
                }
                base += __builtin_amdgcn_readlane(incl, 63);
            }
            if (lane == 0) scan_tmp[0] = base;
        }
        __syncthreads();             // union list ready; the scratch area becomes V staging
    }
    const uint32_t U = scan_tmp[0];
    // The lane's bit in a page's row mask (bit 8, always set below, for a padding column) and
    // its row's visible length, at most MP pages. A padding column has a zero q, so it sees
    // every token: its logits are exactly 0 and its results are never written.
    const uint32_t selbit = colv ? 1u << (jc - j_lo) : 0x100u;
    const int64_t lfull = (int64_t)MP << prm.log2P;
    const int lcol = colv ? (int)min(row_geom(Lb, Rb, jc, prm.log2P, MP).len, lfull) : (int)lfull;

    // ---- 3. online softmax over this wave's sub-chunks, the next one in flight -----
    const int lc = prm.log2P - 5;                   // log2(sub-chunks per page)
    const int NU = (int)U << lc;
    // (s + 1) * NU <= 64 * 4096 sub-chunks: 32-bit products and the host's divisor for S
    const int u_lo = S == 1 ? 0 : (int)fast_div((uint32_t)(s * NU), prm.div_splits);
    const int u_hi = S == 1 ? NU : (int)fast_div((uint32_t)((s + 1) * NU), prm.div_splits);
    // this lane's column's logit scale: sm_scale * k_global * log2(e), times the 2^e its q
    // operand was scaled down by (exact)
    const float c1 = ldexpf(prm.qk_scale_log2, q_col_exp[li]);
    const float NEG_INF = -__builtin_inff();

    // O^T accumulators; tile NDT is a ones-row of V, so it accumulates sum_t P[t][col],
    // the softmax denominator of the very f16 P values that feed the other tiles.
    f32x4 oacc[NDT + 1];
#pragma unroll
    for (int dt = 0; dt <= NDT; ++dt) oacc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_col = NEG_INF;
    float thr = NEG_INF;                            // (m_col + kLazy) / c1
    half_t *vs = &vsm[wave][0];
    const f16x8 ones = {(half_t)1.0f, (half_t)1.0f, (half_t)1.0f, (half_t)1.0f,
                        (half_t)1.0f, (half_t)1.0f, (half_t)1.0f, (half_t)1.0f};
    const int trow = 4 * gq + (li >> 2);            // transposed-read rows trow, trow + 16
    // this lane's byte offsets inside a sub-chunk's codes and scales (token li, chunk gq)
    const uint32_t lco = (uint32_t)(li * code_bytes<D, F>() + gq * (code_bytes<D, F>() / 4));
    const uint32_t lso = (uint32_t)(li * scale_bytes<D, F>() + gq * (scale_bytes<D, F>() / 4));

    // The q operand of S^T = K Q^T: held in registers by one-row tiles (which have them to
    // spare), read from LDS per sub-chunk otherwise.
    f16x8 qreg[ONE ? KS : 1];
    if constexpr (ONE) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = q_lds[ks][lane];
    }
    auto qop = [&](int ks) -> f16x8 {
        if constexpr (ONE) return qreg[ks];
        else return q_lds[ks][lane];
    };

    // One register set: a sub-chunk's raw codes are consumed (K into the MFMA operands, V into
    // LDS) before the next sub-chunk's loads are issued into the same registers; those loads
    // are then in flight during the softmax and the P.V products.
    RawTile<D, F> kr[2], vr[2];
    auto process = [&](const UnitCursor &u, const UnitCursor &un, RawTile<D, F>(&kr)[2], RawTile<D, F>(&vr)[2]) {
        const int p = (int)(u.pm & 0xffffu);
        const uint32_t rmask = (u.pm >> 16) & 0xffu;

        // S^T = K Q^T (unscaled logits)
        f32x4 sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const f16x2 ksc = tile_scales<D, F>(kr[mt]);
            sacc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant_group<D, F>(kr[mt], ksc, ks), qop(ks),
                                                                  sacc[mt], 0, 0, 0);
        }

        // V -> LDS, token-major rows of this 32-token sub-chunk (16-byte chunks swizzled)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const f16x2 vsc = tile_scales<D, F>(vr[mt]);
            const int row = mt * 16 + li;
#pragma unroll
            for (int i = 0; i < DQ / 8; ++i) {
                const int ch = gq * (DQ / 8) + i;
                *reinterpret_cast<f16x8 *>(vs + row * D + ((ch ^ vswz(row)) & (D / 8 - 1)) * 8) =
                    dequant_group<D, F>(vr[mt], vsc, i);
            }
        }
        if (un.have) load_unit<D, F>(prm, un.phys, g, un.c, lco, lso, kr, vr);

        // online softmax with a lazily raised column max; P stays in registers
        const int tok0 = (p << prm.log2P) + u.c * 32;                  // wave-uniform
        int lim = min(max(lcol - tok0, 0), 32);                        // visible tokens of the column
        if (((rmask | 0x100u) & selbit) == 0u) lim = 0;                // its row did not select the page
        float x[8];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) x[mt * 4 + r] = sacc[mt][r];
        if (__any(lim < 32)) {
            // a row ends inside this sub-chunk, or whole columns are masked
            const int limq = lim - gq * 4;          // token (i / 4) * 16 + gq * 4 + (i & 3) is visible
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((i / 4) * 16 + (i & 3) >= limq) x[i] = NEG_INF;
        }
        // raise the column max only when a logit passes it by more than kLazy (log2 units):
        // x * c1 > m_col + kLazy, i.e. x > thr with c1 > 0
        bool over = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) over |= x[i] > thr;
        if (__any(over)) {
            const float lmx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                    fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            const float m_new = fmaxf(m_col, max_across_groups(lmx) * c1);
            const float alpha = (m_new == NEG_INF) ? 1.0f : __builtin_amdgcn_exp2f(m_col - m_new);
#pragma unroll
            for (int dt = 0; dt <= NDT; ++dt) oacc[dt] *= alpha;
            m_col = m_new;
            thr = (m_col + kLazy) / c1;
        }
        const float negm = (m_col == NEG_INF) ? NEG_INF : -m_col;
        float pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c1, negm));
        const f16x2 p0 = {(half_t)pr[0], (half_t)pr[1]}, p1 = {(half_t)pr[2], (half_t)pr[3]};
        const f16x2 p2 = {(half_t)pr[4], (half_t)pr[5]}, p3 = {(half_t)pr[6], (half_t)pr[7]};
        const f16x8 pop = __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                                  __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);

        // O^T += V^T P^T, and the ones-row tile for the denominator
        wave_lds_fence();            // this wave's V staging writes are complete
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int ch = 2 * dt + ((li >> 1) & 1), sub = (li & 1) * 4;
            const half_t *a0 = vs + trow * D + ((ch ^ vswz(trow)) & (D / 8 - 1)) * 8 + sub;
            const half_t *a1 = vs + (trow + 16) * D + ((ch ^ vswz(trow + 16)) & (D / 8 - 1)) * 8 + sub;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(a0));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(a1));
            const f16x8 a = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pop, oacc[dt], 0, 0, 0);
        }
        oacc[NDT] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pop, oacc[NDT], 0, 0, 0);
    };

    UnitCursor u = seek_unit<NW>(u_lo + wave, u_hi, lc, u_pm, u_phys);
    if (u.have) load_unit<D, F>(prm, u.phys, g, u.c, lco, lso, kr, vr);
    QSA_STAMP(8);
    while (u.have) {
        const UnitCursor un = seek_unit<NW>(u.u + NW, u_hi, lc, u_pm, u_phys);
        process(u, un, kr, vr);
        u = un;
    }
    QSA_STAMP(9);
    // (the offsets loaded at the start have long arrived; before any early return of a split)
    if (prm.uniform_rows && checker && (ro_check0 != r0 || ro_check1 != r1)) set_error(prm.err, QSA_DEVERR_ROWS);

    // ---- 4. merge the waves (fixed order); wave w finishes output tiles w, w + NW, ... ----
    // Every wave publishes its column maxima and denominators, and all its O^T tiles in its
    // own V staging tile (which no other wave touches; d/16 tiles of 64 lanes x 16 bytes fill
    // it exactly). After one barrier, each wave reads the maxima, the denominators and the
    // tiles it owns from every wave, all loads issued before the first use, takes the common
    // column max M and the weights 2^(m_w - M), and sums in ascending wave order, as every wave
    // sums the denominators, so the result does not depend on which wave does the sum. No
    // branch on the wave index: a wave that owns fewer tiles sums tile 0 in their place and
    // drops it.
    constexpr int TPW = (NDT + NW - 1) / NW;        // output tiles per wave
    {
        float *pub = reinterpret_cast<float *>(vs);
        if (gq == 0) {
            ml_m[wave][li] = m_col;
            ml_l[wave][li] = oacc[NDT][0];
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4 *>(pub + (dt * 64 + lane) * 4) = oacc[dt];
    }
    __syncthreads();
    int own[TPW];                                    // the tiles this wave finishes (< NDT: owned)
#pragma unroll
    for (int ot = 0; ot < TPW; ++ot) own[ot] = wave + ot * NW;
    float mws[NW], lws[NW];
    f32x4 ows[TPW][NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        mws[w] = ml_m[w][li];
        lws[w] = ml_l[w][li];
#pragma unroll
        for (int ot = 0; ot < TPW; ++ot) {
            const int tsel = own[ot] < NDT ? own[ot] : 0;
            ows[ot][w] = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(&vsm[w][0]) +
                                                          (tsel * 64 + lane) * 4);
        }
    }
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mws[w]);
    float Lsum = 0.0f;
    f32x4 o_own[TPW];                                // the merged tiles own[ot] (owned ones only)
#pragma unroll
    for (int ot = 0; ot < TPW; ++ot) o_own[ot] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float wgt = (mws[w] == NEG_INF) ? 0.0f : __builtin_amdgcn_exp2f(mws[w] - M);
        Lsum = __builtin_fmaf(wgt, lws[w], Lsum);
#pragma unroll
        for (int ot = 0; ot < TPW; ++ot)
#pragma unroll
            for (int i = 0; i < 4; ++i) o_own[ot][i] = __builtin_fmaf(wgt, ows[ot][w][i], o_own[ot][i]);
    }
    m_col = M;
    QSA_STAMP(11);
    if (S > 1) {
        // Publish this split's partial (each owner its tiles, wave 0 the denominators and the
        // column maxima), count it, and let the tile's last split merge. The partial moves
        // through agent-scope (coherent) stores and loads: each such access is coherent
        // across the XCDs' L2s on its own, so the handoff needs only the stores' completion
        // (vmcnt 0, then a barrier) before the count -- not an agent-scope fence, whose L2
        // writeback and invalidate cost several microseconds per workgroup here.
        constexpr int PF = decode_part_floats(D);
        constexpr int kOff = (NDT + 1) * 64 * 4;
        float *tile_part = prm.part + (int64_t)tile * S * PF;
        float *mine = tile_part + (int64_t)s * PF;
#pragma unroll
        for (int ot = 0; ot < TPW; ++ot) {
            if (own[ot] < NDT) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __hip_atomic_store(mine + (own[ot] * 4 + i) * 64 + lane, o_own[ot][i], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (wave == 0) {
            __hip_atomic_store(mine + (NDT * 4) * 64 + lane, Lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(mine + kOff + lane, m_col, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0): this wave's partial stores are complete
        __syncthreads();
        if (wave == 0) {
            uint32_t done = 0u;
            if (lane == 0) done = __hip_atomic_fetch_add(prm.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            done = __builtin_amdgcn_readfirstlane(done);
            if (lane == 0) scan_tmp[1] = done;
        }
        __syncthreads();
        if (scan_tmp[1] != (uint32_t)(S - 1)) {
            QSA_TRACE_END();
            return;
        }
        // the last split: every partial's stores completed before its count. Each wave merges
        // the partials (its owned tiles, the denominators, the maxima) in ascending split order
        // with a running max, eight splits at a time: a group's loads, its own partial's
        // included, all issue before the first is used (clamped, unconditional), so a group
        // costs one round trip. With at most eight splits this is one group and the plain
        // weighted sum with the common max. A wave with two tiles merges them one after the
        // other, each the same way, so the denominators and maxima come out the same.
        constexpr int kGroup = 8;
#pragma unroll
        for (int ot = 0; ot < TPW; ++ot) {
            const int tsel = own[ot] < NDT ? own[ot] : 0;
            float Ms = NEG_INF, Ls = 0.0f;
            f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
            for (int sp0 = 0; sp0 < S; sp0 += kGroup) {
                float mv[kGroup], lv[kGroup];
                f32x4 ov[kGroup];
#pragma unroll
                for (int i = 0; i < kGroup; ++i) {
                    const float *part = tile_part + (int64_t)min(sp0 + i, S - 1) * PF;
                    mv[i] = __hip_atomic_load(part + kOff + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    lv[i] = __hip_atomic_load(part + (NDT * 4) * 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ov[i][e] = __hip_atomic_load(part + (tsel * 4 + e) * 64 + lane, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                }
                float cm = Ms;
#pragma unroll
                for (int i = 0; i < kGroup; ++i)
                    if (sp0 + i < S) cm = fmaxf(cm, mv[i]);
                const float resc = (Ms == NEG_INF) ? 0.0f : __builtin_amdgcn_exp2f(Ms - cm);
                Ls *= resc;
                acc *= resc;
#pragma unroll
                for (int i = 0; i < kGroup; ++i) {
                    const float wgt = (sp0 + i >= S || mv[i] == NEG_INF) ? 0.0f : __builtin_amdgcn_exp2f(mv[i] - cm);
                    Ls = __builtin_fmaf(wgt, lv[i], Ls);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(wgt, ov[i][e], acc[e]);
                }
                Ms = cm;
            }
            o_own[ot] = acc;
            Lsum = Ls;
            m_col = Ms;
        }
        if (wave == 0 && lane == 0) __hip_atomic_store(prm.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    QSA_TRACE_END();
    if (!colv) return;
    const int row = r0 + jc, head = g * G + (col - jc * G);
    const float sc = (Lsum > 0.0f) ? prm.v_global / Lsum : 0.0f;
#pragma unroll
    for (int ot = 0; ot < TPW; ++ot) {
        if (own[ot] >= NDT) continue;
        const int dt = own[ot];
        f32x4 o = o_own[ot] * sc;
        if (prm.gate) {
            // the gated epilogue: out * sigmoid(gate), one rounding to bf16 after the product
            const uint2 gr = *reinterpret_cast<const uint2 *>(prm.gate + ((int64_t)row * prm.Hq + head) * D +
                                                                dt * 16 + gq * 4);
            const float gv[4] = {bf16lo(gr.x), bf16hi(gr.x), bf16lo(gr.y), bf16hi(gr.y)};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] *= __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gv[i]));
        }
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
        packed.y = (uint32_t)f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
        *reinterpret_cast<uint2 *>(prm.out + ((int64_t)row * prm.Hq + head) * D + dt * 16 + gq * 4) = packed;
    }
    if (wave == 0 && gq == 0 && prm.lse)
        prm.lse[(int64_t)row * prm.Hq + head] = (Lsum > 0.0f) ? (m_col + __log2f(Lsum)) * 0.69314718055994531f : NEG_INF;
    QSA_STAMP(10);
    QSA_TRACE_END();
}

template <int D, int SELC>
static hipError_t launch_decode_d(const DecodeParams &prm, hipStream_t stream)
{
    const int64_t per = ((int64_t)prm.tiles * prm.splits + kXcds - 1) / kXcds;   // work items per XCD
    const unsigned grid = (unsigned)(per * kXcds);
    const bool fp8 = prm.kv_format == kFp8;
    if (prm.one_row_tiles && decode_waves(prm.one_row_tiles, prm.tiles, prm.splits) == 4) {
        if (fp8)
            sparse_decode_kernel<D, SELC, kFp8, true, 4><<<grid, 4 * 64, 0, stream>>>(prm);
        else
            sparse_decode_kernel<D, SELC, kNvfp4, true, 4><<<grid, 4 * 64, 0, stream>>>(prm);
    } else if (prm.one_row_tiles) {
        if (fp8)
            sparse_decode_kernel<D, SELC, kFp8, true, kDecodeWaves><<<grid, kDecodeWaves * 64, 0, stream>>>(prm);
        else
            sparse_decode_kernel<D, SELC, kNvfp4, true, kDecodeWaves><<<grid, kDecodeWaves * 64, 0, stream>>>(prm);
    } else {
        if (fp8)
            sparse_decode_kernel<D, SELC, kFp8, false, kDecodeWaves><<<grid, kDecodeWaves * 64, 0, stream>>>(prm);
        else
            sparse_decode_kernel<D, SELC, kNvfp4, false, kDecodeWaves><<<grid, kDecodeWaves * 64, 0, stream>>>(prm);
    }
    return hipGetLastError();
}

hipError_t launch_sparse_decode(const DecodeParams &prm, int D, hipStream_t stream)
{
    return D == 64 ? launch_decode_d<64, 0>(prm, stream) : launch_decode_d<128, 0>(prm, stream);
}

hipError_t launch_select_sparse_decode(const DecodeParams &prm, int D, hipStream_t stream)
{
    switch (fused_select_cols(prm.MP)) {
    case 2: return D == 64 ? launch_decode_d<64, 2>(prm, stream) : launch_decode_d<128, 2>(prm, stream);
    case 4: return D == 64 ? launch_decode_d<64, 4>(prm, stream) : launch_decode_d<128, 4>(prm, stream);
    case 8: return D == 64 ? launch_decode_d<64, 8>(prm, stream) : launch_decode_d<128, 8>(prm, stream);
    case 16: return D == 64 ? launch_decode_d<64, 16>(prm, stream) : launch_decode_d<128, 16>(prm, stream);
    default: return hipErrorInvalidValue;
    }
}

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *p, int n)
{
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_clear_words(uint32_t *p, int n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int blocks = (n + 255) / 256 < 32 ? (n + 255) / 256 : 32;
    clear_words_kernel<<<blocks, 256, 0, stream>>>(p, n);
    return hipGetLastError();
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
    const f16x8 v = nvfp4_dequant8(codes, e4m3x2_to_f16x2(sb).x);
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

#if defined(QSA_TRACE)
// Copies the first `count` stamps ([workgroup][wave][point], 100 MHz ticks) of the last traced
// launch to host memory. Traced builds only.
extern "C" int qsa_trace_read(unsigned long long *host, size_t count)
{
    const size_t cap = sizeof(qsa::qsa_trace_stamps) / sizeof(unsigned long long);
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(qsa::qsa_trace_stamps),
                                    (count < cap ? count : cap) * sizeof(unsigned long long), 0,
                                    hipMemcpyDeviceToHost);
}
#endif
