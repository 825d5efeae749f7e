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
// one query row; each lane owns one page and holds that page's key for the current KV head
// in VGPRs: as raw bf16 pairs, loaded a few 16-element chunks ahead and converted to fp32 one
// chunk at a time when one pass covers all of the KV head's q heads (at most 8), else kept
// whole as fp32 for the later passes. Each wave takes KV heads in turn, eight of the KV head's q heads per pass. q is wave-uniform, so it reaches the lanes through the cross-lane operand network
// rather than through per-element LDS reads: a VGPR holds 16 consecutive elements of one
// head, element m in lane m of every 16-lane row, and each v_fmac_f32 reads its q operand
// through DPP row_newbcast, which hands one lane's value to its whole row. Each head's sum
// stays one fp32 fma after another in ascending element order. A product of two bf16 values
// is exact in fp32, so the fma equals the separate multiply and add. The loads that do not
// depend on each other (row offsets, the request's length, the page-table entries, q) are
// issued together at the start. An LDS max over the waves combines the KV heads (max is
// exact in any order).
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

constexpr int kIndexWaves = 4;
constexpr int kIndexCUs = 256;
constexpr int kHeadGroup = 8;        // q heads per pass
// One-pass form: key chunks in registers at once, and the waves per SIMD the compiler is asked
// to allow (its registers: 67 per lane at d = 128, so seven waves fit a SIMD). Measured against
// the whole key in registers (115 per lane, four waves): 32K verify 8.9 -> 8.4 us, context step
// 22.2 -> 21.0 us, 131K 8.9 -> 8.5 us, the others unchanged; a ring of one chunk (eight waves)
// lost 0.7 us on the wide mixed batch.
constexpr int kRing = 2;
constexpr int kOnePassWaves = 6;

// acc[t] = fma(q_t[16c + n], k[16c + n], acc[t]) for n = 0 .. 15 in order and t = 0 .. 7:
// operand 8 + t holds q_t[16c + m] in lane m of each 16-lane row, and row_newbcast:n gives
// every lane of the row lane n's value. Operands 16 .. 31 are k[16c .. 16c + 15]. The
// leading s_nop covers the wait states that a DPP read needs after a VALU write of its
// source or an SALU write of EXEC, which the compiler does not track inside inline asm.
#define QSA_FMAC(A, Q, K, N) "v_fmac_f32_dpp %" #A ", %" #Q ", %" #K " row_newbcast:" #N " row_mask:0xf bank_mask:0xf\n"
#define QSA_FMAC8(K, N)                                                                                           \
    QSA_FMAC(0, 8, K, N) QSA_FMAC(1, 9, K, N) QSA_FMAC(2, 10, K, N) QSA_FMAC(3, 11, K, N) QSA_FMAC(4, 12, K, N) \
        QSA_FMAC(5, 13, K, N) QSA_FMAC(6, 14, K, N) QSA_FMAC(7, 15, K, N)

__device__ __forceinline__ void fmac16x8(float (&a)[kHeadGroup], const float (&qc)[kHeadGroup], const float *k)
{
    asm("s_nop 4\n" QSA_FMAC8(16, 0) QSA_FMAC8(17, 1) QSA_FMAC8(18, 2) QSA_FMAC8(19, 3) QSA_FMAC8(20, 4)
            QSA_FMAC8(21, 5) QSA_FMAC8(22, 6) QSA_FMAC8(23, 7) QSA_FMAC8(24, 8) QSA_FMAC8(25, 9) QSA_FMAC8(26, 10)
                QSA_FMAC8(27, 11) QSA_FMAC8(28, 12) QSA_FMAC8(29, 13) QSA_FMAC8(30, 14) QSA_FMAC8(31, 15)
        : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
        : "v"(qc[0]), "v"(qc[1]), "v"(qc[2]), "v"(qc[3]), "v"(qc[4]), "v"(qc[5]), "v"(qc[6]), "v"(qc[7]), "v"(k[0]),
          "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(k[4]), "v"(k[5]), "v"(k[6]), "v"(k[7]), "v"(k[8]), "v"(k[9]),
          "v"(k[10]), "v"(k[11]), "v"(k[12]), "v"(k[13]), "v"(k[14]), "v"(k[15]));
}
#undef QSA_FMAC8
#undef QSA_FMAC

// NW waves per workgroup, each taking KV heads wave, wave + NW, ...: 4 by default; 8 when the
// grid is small and there are at least 8 KV heads, so that the KV heads of a (row, page tile)
// spread over more SIMDs. ONEG: at most 8 q heads per KV head, so one pass covers them all and
// the key is converted to fp32 one 16-element chunk at a time instead of being kept whole,
// and it is loaded as it is used, kRing chunks ahead; that cuts the VGPRs to a third, and a
// grid then holds up to seven waves per SIMD, so one wave's loads overlap others' fmas.
// ORD: the dispatch order of a grid whose rows have more than one aligned group of 8 tiles
// (below).
template <int D, int NW, bool ONEG, bool ORD>
__global__ __launch_bounds__(NW * 64, ONEG ? kOnePassWaves : 2) void index_scores_kernel(IndexParams prm)
{
    constexpr int HG = kHeadGroup;
    __shared__ float red[NW][kWave];
    constexpr int NC = D / 16;                        // 16-element chunks of a row
    // per wave: q of one head group, [head][element mod 16][element / 16]; with ONEG
    // [element / 16][element mod 16][head], so that a chunk's eight heads are adjacent
    __shared__ __align__(16) float qs[NW][HG][16][NC];

    // every kernel argument the prologue needs, in scalar registers before anything waits on
    // one (each first read of an argument's cache line misses the scalar cache at launch)
    asm volatile("" ::"s"(prm.row_offsets), "s"(prm.seq_lens), "s"(prm.page_table), "s"(prm.keys), "s"(prm.q32),
                 "s"(prm.MP), "s"(prm.N), "s"(prm.rmax), "s"(prm.uniform_rows), "s"(prm.Hq), "s"(prm.Hkv),
                 "s"(prm.W), "s"(prm.log2P), "s"(prm.NP));
    // Page tile of this workgroup. The dispatcher deals workgroups to the 8 XCDs by linear id,
    // so with the tile index fastest, tile x of every row lands on XCD x mod 8 whenever the
    // tiles per row are a multiple of 8. Tiles past a short request's pages leave at once, so
    // the low tiles carry most of the work, and on a batch of mixed lengths the low XCDs
    // would get most of it. Request b therefore rotates its tiles by b within each aligned
    // group of 8 (a partial last group is left as it is): a bijection of the row's tiles that
    // spreads the live ones over the XCDs and keeps the rows of one (request, tile) on one
    // XCD, where they share the tile's keys.
    // The dispatcher also starts workgroups in linear-id order, and with the tile fastest
    // the tiles past short requests' pages are spread over the whole dispatch, each holding
    // a slot for the round trip of its request's length while live tiles wait. With ORD (a
    // multiple of 8 tiles per row, more than 8) the linear id is taken apart anew: its value
    // mod 8 (the XCD) stays the tile's position in its group, and the tile group becomes the
    // slowest index, so that every request's first group of tiles starts before any second
    // group, and the groups past short requests come last. Each (tile, row, request) still
    // runs on the same XCD; the map is a bijection of the grid.
    // (the tile count from MP, an argument already in registers: gridDim would be read from
    // the dispatch packet, one more scalar-cache miss ahead of the page-table load)
    const int tiles_per_row = (prm.MP + kWave - 1) / kWave;
    int j = blockIdx.y, b = blockIdx.z, x = blockIdx.x;
    if constexpr (ORD) {
        // grid (tiles_per_row, rmax, B), tiles_per_row = 8m: id = x + tiles * (j + rmax * b);
        // id mod 8 = x mod 8, and id / 8 = group * (rmax * B) + (j + rmax * b) afterwards. The
        // id is unsigned: up to 64 tiles x 1024 rows x 65535 requests, just under 2^32.
        const int RB = prm.rmax * (int)gridDim.z;
        const uint32_t lin = (uint32_t)x + (uint32_t)tiles_per_row * ((uint32_t)j + (uint32_t)prm.rmax * (uint32_t)b);
        const int slot = (int)(lin >> 3), grp = slot / RB, rem = slot - grp * RB;
        b = rem / prm.rmax;
        j = rem - b * prm.rmax;
        x = grp * 8 + (int)(lin & 7u);
    }
    const int tile = ((x | 7) < tiles_per_row) ? ((x & ~7) | ((x + b) & 7)) : x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wv = __builtin_amdgcn_readfirstlane(wave);     // wave-uniform
    // independent loads first: the row range, the request's length and this lane's page. When
    // every request has rmax rows (num_rows is B * rmax) the range is [b * rmax, (b + 1) * rmax)
    // with no load, and the offsets are only compared with it at the end.
    int r0, r1;
    if (prm.uniform_rows) {
        r0 = b * prm.rmax;
        r1 = r0 + prm.rmax;
    } else {
        r0 = prm.row_offsets[b];
        r1 = prm.row_offsets[b + 1];
    }
    const int p = tile * kWave + lane;
    const int32_t phys = p < prm.MP ? prm.page_table[(int64_t)b * prm.MP + p] : -1;
    const int64_t L_b = prm.seq_lens[b];
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
    float(*qw)[16][NC] = qs[wv];
    float best = __builtin_nanf("");
    // q heads h0 .. h0 + nh - 1 of KV head g, as bf16 pairs: lane l holds elements 2l, 2l + 1
    // of every head (zeros past nh, and for lanes past d / 2)
    auto load_q = [&](int g, int h0, uint32_t (&qu)[HG]) {
        const int nh = min(HG, G - h0);
        const uint32_t *qb = prm.q32 + ((int64_t)row * prm.Hq + g * G + h0) * (D / 2) + lane;
#pragma unroll
        for (int t = 0; t < HG; ++t) qu[t] = (lane < D / 2 && t < nh) ? qb[t * (D / 2)] : 0u;
    };
    // q of the head group into LDS as fp32, then into qc[c][t] (head t, elements 16c .. 16c + 15,
    // element 16c + m in lane m of each 16-lane row)
    auto stage_q = [&](const uint32_t (&qu)[HG], float (&qc)[NC][HG]) {
        if (lane < D / 2) {
            const int m = (2 * lane) & 15, c = (2 * lane) >> 4;
#pragma unroll
            for (int t = 0; t < HG; ++t) {
                qw[t][m][c] = bf16lo(qu[t]);
                qw[t][m + 1][c] = bf16hi(qu[t]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): this wave's q rows are in LDS
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int t = 0; t < HG; ++t)
#pragma unroll
            for (int c4 = 0; c4 < NC; c4 += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(&qw[t][lane & 15][c4]);
                qc[c4][t] = v.x;
                qc[c4 + 1][t] = v.y;
                qc[c4 + 2][t] = v.z;
                qc[c4 + 3][t] = v.w;
            }
    };
    auto fold = [&](const float (&a)[HG], int nh) {
#pragma unroll
        for (int t = 0; t < HG; ++t)
            if (t < nh && !(a[t] != a[t]) && ((best != best) || a[t] > best)) best = a[t];
    };

    if constexpr (ONEG) {
        float *qf = &qs[wv][0][0][0];
        for (int g = wv; g < prm.Hkv && any_cand; g += NW) {
            uint32_t qu[HG];
            load_q(g, 0, qu);
            const uint4 *kp = reinterpret_cast<const uint4 *>(prm.keys + ((int64_t)(cand ? phys : 0) * prm.Hkv + g) * D);
            // the key in a ring of kRing 16-element chunks (two 16-byte loads each): the first
            // kRing chunks load now, and chunk c + kRing loads into chunk c's registers once
            // chunk c is converted, so a wave holds a fraction of the key and a SIMD more waves
            uint4 kraw[2 * kRing];
#pragma unroll
            for (int c = 0; c < 2 * kRing; ++c) kraw[c] = kp[c];
            __builtin_amdgcn_sched_barrier(0);    // keep these key loads ahead of the wait for q
            // q as fp32: element e of head t at [(e / 16) * 16 + e % 16][t]
            if (lane < D / 2) {
                float4 *dst = reinterpret_cast<float4 *>(qf + 2 * lane * HG);
                dst[0] = make_float4(bf16lo(qu[0]), bf16lo(qu[1]), bf16lo(qu[2]), bf16lo(qu[3]));
                dst[1] = make_float4(bf16lo(qu[4]), bf16lo(qu[5]), bf16lo(qu[6]), bf16lo(qu[7]));
                dst[2] = make_float4(bf16hi(qu[0]), bf16hi(qu[1]), bf16hi(qu[2]), bf16hi(qu[3]));
                dst[3] = make_float4(bf16hi(qu[4]), bf16hi(qu[5]), bf16hi(qu[6]), bf16hi(qu[7]));
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): this wave's q is in LDS
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float a[HG];
#pragma unroll
            for (int t = 0; t < HG; ++t) a[t] = 0.0f;
            // chunk c of q: head t's element 16c + m in lane m of each 16-lane row; the next
            // chunk's reads are issued before this chunk's fmas, so their latency is hidden
            const float4 *qsrc = reinterpret_cast<const float4 *>(qf + (lane & 15) * HG);
            float4 q0n = qsrc[0], q1n = qsrc[1];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float4 q0 = q0n, q1 = q1n;
                if (c + 1 < NC) {
                    q0n = qsrc[(c + 1) * 16 * HG / 4];
                    q1n = qsrc[(c + 1) * 16 * HG / 4 + 1];
                }
                __builtin_amdgcn_sched_barrier(0);    // the next chunk's reads stay ahead of these fmas
                const float qc[HG] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
                float kk[16];
                const int slot = c % kRing;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint4 v = kraw[2 * slot + h];
                    float *k8 = &kk[8 * h];
                    k8[0] = bf16lo(v.x); k8[1] = bf16hi(v.x); k8[2] = bf16lo(v.y); k8[3] = bf16hi(v.y);
                    k8[4] = bf16lo(v.z); k8[5] = bf16hi(v.z); k8[6] = bf16lo(v.w); k8[7] = bf16hi(v.w);
                }
                if (c + kRing < NC) {
                    kraw[2 * slot] = kp[2 * (c + kRing)];
                    kraw[2 * slot + 1] = kp[2 * (c + kRing) + 1];
                }
                fmac16x8(a, qc, kk);
            }
            fold(a, G);
            __builtin_amdgcn_s_waitcnt(0xc07f);   // reads done before the next KV head's staging
        }
    } else
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
        float qc[NC][HG];
        stage_q(qu, qc);
        // first head group: each 16-element chunk of the key is converted to fp32 and used as
        // soon as it has arrived, while the later chunks are still in flight
        float k[D];
        float a[HG];
#pragma unroll
        for (int t = 0; t < HG; ++t) a[t] = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint4 v = kraw[2 * c + h];
                float *kk = &k[16 * c + 8 * h];
                kk[0] = bf16lo(v.x); kk[1] = bf16hi(v.x); kk[2] = bf16lo(v.y); kk[3] = bf16hi(v.y);
                kk[4] = bf16lo(v.z); kk[5] = bf16hi(v.z); kk[6] = bf16lo(v.w); kk[7] = bf16hi(v.w);
            }
            fmac16x8(a, qc[c], &k[16 * c]);
        }
        fold(a, min(HG, G));
        // further head groups reuse the converted key
        for (int h0 = HG; h0 < G; h0 += HG) {
            load_q(g, h0, qu);
            stage_q(qu, qc);
#pragma unroll
            for (int t = 0; t < HG; ++t) a[t] = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) fmac16x8(a, qc[c], &k[16 * c]);
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
        if (prm.uniform_rows && (prm.row_offsets[b] != r0 || prm.row_offsets[b + 1] != r1))
            set_error(prm.err, QSA_DEVERR_ROWS);
    }
}

hipError_t launch_index_scores(const IndexParams &prm, int D, int B, hipStream_t stream)
{
    dim3 grid((prm.MP + kWave - 1) / kWave, prm.rmax, B);
    // a grid of fewer waves than two per SIMD (4 x 256) takes eight waves per workgroup when
    // the KV heads are enough to occupy them
    const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
    const bool wide = prm.Hkv >= 8 && wgs * kIndexWaves < 2 * 4 * kIndexCUs;
    // at most 8 q heads per KV head: one pass per KV head, the key converted chunk by chunk
    const bool oneg = prm.Hq <= kHeadGroup * prm.Hkv;
    // large grids whose rows have several aligned groups of 8 tiles start them group by group
    const bool ord = !wide && grid.x > 8 && grid.x % 8 == 0;
    auto go = [&](auto kern, int nw) { kern<<<grid, nw * 64, 0, stream>>>(prm); };
    if (D == 64) {
        if (oneg) {
            if (wide) go(index_scores_kernel<64, 8, true, false>, 8);
            else if (ord) go(index_scores_kernel<64, kIndexWaves, true, true>, kIndexWaves);
            else go(index_scores_kernel<64, kIndexWaves, true, false>, kIndexWaves);
        } else {
            if (wide) go(index_scores_kernel<64, 8, false, false>, 8);
            else if (ord) go(index_scores_kernel<64, kIndexWaves, false, true>, kIndexWaves);
            else go(index_scores_kernel<64, kIndexWaves, false, false>, kIndexWaves);
        }
    } else {
        if (oneg) {
            if (wide) go(index_scores_kernel<128, 8, true, false>, 8);
            else if (ord) go(index_scores_kernel<128, kIndexWaves, true, true>, kIndexWaves);
            else go(index_scores_kernel<128, kIndexWaves, true, false>, kIndexWaves);
        } else {
            if (wide) go(index_scores_kernel<128, 8, false, false>, 8);
            else if (ord) go(index_scores_kernel<128, kIndexWaves, false, true>, kIndexWaves);
            else go(index_scores_kernel<128, kIndexWaves, false, false>, kIndexWaves);
        }
    }
    return hipGetLastError();
}

}  // namespace qsa
