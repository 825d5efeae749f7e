/*
 * qsa_oracle.c -- plain CPU oracle for query-sparse NVFP4 decode / verify attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the benchmark's CPU
 * baseline may load this file's library. The product path never links, calls
 * or falls back to it.
 *
 * Each function writes out the definition of one step, as slowly and plainly
 * as it can be written: scalar loops, fp64 wherever the pages fix no precision,
 * no SIMD and no blocking. It shares no code, header or table with the GPU
 * library. Compile with -ffp-contract=off so that every fp32 operation written
 * here is the operation executed.
 *
 * Sources (three pull-request pages of the TensorRT-LLM project):
 *   [PR20276] "Qwen3.8-Flash-Next target completion", sections Features,
 *             Performance ("What runs on the fast paths"), Decisions worth knowing
 *   [PR20937] "GB300 performance work", Description > What changes
 *             (NVFP4 sparse GQA decode; MTP > Verify), and the verify-test review
 *             comment that fixes E4M3_NAN = 0x7F
 *   [OCP-MX]  OCP Microscaling Formats (MX) v1.0, the E2M1 element format
 *   [OCP-FP8] OCP 8-bit Floating Point Specification (OFP8), E4M3 with NaN at S.1111.111
 *
 * Layouts (row-major):
 *   q           bf16 bits [N][Hq][d]
 *   k/v codes   uint8     [NP][Hkv][P][d/2]  e2m1, low nibble = even element
 *   k/v scales  uint8     [NP][Hkv][P][d/16] e4m3, one per 16 consecutive elements
 *   index_keys  bf16 bits [NP][Hkv][d]
 *   page_table  int32     [B][MP], -1 = invalid
 *   seq_lens    int32     [B]
 *   row_offsets int32     [B+1]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats -- */

/* E2M1 (4 bits: sign, 2-bit exponent with bias 1, 1-bit mantissa) [OCP-MX].
   Exponent 0 is subnormal: m * 0.5. Otherwise 2^(e-1) * (1 + m/2). */
double oracle_e2m1(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* E4M3FN (sign, 4-bit exponent with bias 7, 3-bit mantissa; no infinities;
   S.1111.111 is NaN) [OCP-FP8]. The NaN code 0x7F is the one the verify test of
   [PR20937] names. Exponent 0 is subnormal: m * 2^-9. */
double oracle_e4m3(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* bf16 is the top half of an IEEE binary32. */
double oracle_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static float bf16_to_f32(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ---------------------------------------------------------------- dequant -- */

/* One element of an NVFP4 page [PR20276, Features: "uint8 e2m1 pages + e4m3 block
   scales"]: x = e2m1(code) * e4m3(scale of its 16-element block) * global. */
double oracle_dequant_elem(const uint8_t *codes, const uint8_t *scales, double global,
                           int Hkv, int P, int d, int64_t page, int h, int t, int i)
{
    int64_t tok = ((page * Hkv + h) * P + t);
    uint8_t byte = codes[tok * (d / 2) + i / 2];
    int c = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    uint8_t sb = scales[tok * (d / 16) + i / 16];
    return oracle_e2m1(c) * oracle_e4m3(sb) * global;
}

/* One element of an FP8 page [PR20937, the FP8 KV cache of the tested configurations: unit
   scales]: codes [NP][Hkv][P][d] hold one OCP E4M3FN byte per element, x = e4m3(byte) * global. */
double oracle_fp8_elem(const uint8_t *codes, double global, int Hkv, int P, int d, int64_t page, int h, int t, int i)
{
    int64_t tok = ((page * Hkv + h) * P + t);
    return oracle_e4m3(codes[tok * d + i]) * global;
}

/* The element of either cache format: kv_format 0 = NVFP4, 1 = FP8 (scales unused). */
static double kv_elem(int kv_format, const uint8_t *codes, const uint8_t *scales, double global,
                      int Hkv, int P, int d, int64_t page, int h, int t, int i)
{
    return kv_format == 1 ? oracle_fp8_elem(codes, global, Hkv, P, d, page, h, t, i)
                          : oracle_dequant_elem(codes, scales, global, Hkv, P, d, page, h, t, i);
}

/* Dequantise the listed physical pages: out[j][h][t][i] for j < n (fp64). */
void oracle_dequant_pages(const uint8_t *codes, const uint8_t *scales, double global,
                          int Hkv, int P, int d, const int32_t *pages, int n, double *out)
{
    for (int j = 0; j < n; ++j)
        for (int h = 0; h < Hkv; ++h)
            for (int t = 0; t < P; ++t)
                for (int i = 0; i < d; ++i)
                    out[(((int64_t)j * Hkv + h) * P + t) * d + i] =
                        oracle_dequant_elem(codes, scales, global, Hkv, P, d, pages[j], h, t, i);
}

/* ------------------------------------------------------------------- rows -- */

/* Row bookkeeping for MTP verify [PR20937, What changes > MTP > Verify; PR20276,
   Known limitations: verify rows P <= 4]. Request b owns rows
   [row_offsets[b], row_offsets[b+1]). All R_b rows sit at the end of its L_b
   tokens and are causal among themselves, so row j (0-based) sees
   L = L_b - (R_b - 1 - j) tokens and n = ceil(L / P) pages (at most MP). */
void oracle_rows(int B, const int32_t *seq_lens, const int32_t *row_offsets, int P, int MP,
                 int32_t *row_req, int32_t *row_len, int32_t *row_pages)
{
    for (int b = 0; b < B; ++b) {
        int r0 = row_offsets[b], r1 = row_offsets[b + 1];
        int R = r1 - r0;
        for (int j = 0; j < R; ++j) {
            int64_t L = (int64_t)seq_lens[b] - (R - 1 - j);
            if (L < 0) L = 0;
            int64_t n = (L + P - 1) / P;
            if (n > MP) n = MP;
            row_req[r0 + j] = b;
            row_len[r0 + j] = (int32_t)L;
            row_pages[r0 + j] = (int32_t)n;
        }
    }
}

static int valid_page(int32_t phys, int64_t NP) { return phys >= 0 && (int64_t)phys < NP; }

/* ----------------------------------------------------------- index scores -- */

/* Block index scores [PR20276, "What runs on the fast paths": index store and
   compression, then index scores; PR20937, MTP > Verify: request-tiled index
   scores]. Each page's index key is one bf16 vector per KV head. A row's score
   for page p is
       sm_scale * max over q heads h of  sum_i q[row][h][i] * key[phys(p)][h / G][i]
   where the sum runs in fp32, with i ascending, rounded after every step.
   A product of two bf16 values is exact in fp32, so only the order of the sum
   matters, and this order is the canonical one. The final fp32 multiply is one
   rounding. A zero score is written as +0. Only candidate pages are scored:
   p < n_row - W with a valid page-table entry. Every other column < MP is -inf. */
void oracle_index_scores(int B, const int32_t *seq_lens, const int32_t *row_offsets,
                         const int32_t *page_table, int MP, int64_t NP, int P, int W,
                         int Hq, int Hkv, int d, float sm_scale,
                         const uint16_t *q, const uint16_t *keys, float *scores)
{
    int N = row_offsets[B];
    int32_t *rq = malloc(sizeof(int32_t) * (N > 0 ? N : 1));
    int32_t *rl = malloc(sizeof(int32_t) * (N > 0 ? N : 1));
    int32_t *rn = malloc(sizeof(int32_t) * (N > 0 ? N : 1));
    oracle_rows(B, seq_lens, row_offsets, P, MP, rq, rl, rn);
    int G = Hq / Hkv;
    for (int r = 0; r < N; ++r) {
        int b = rq[r];
        for (int p = 0; p < MP; ++p) {
            int32_t phys = page_table[(int64_t)b * MP + p];
            if (!(p < rn[r] - W && valid_page(phys, NP))) {
                scores[(int64_t)r * MP + p] = -INFINITY;
                continue;
            }
            float best = NAN;
            for (int h = 0; h < Hq; ++h) {
                const uint16_t *qv = q + ((int64_t)r * Hq + h) * d;
                const uint16_t *kv = keys + ((int64_t)phys * Hkv + h / G) * d;
                float acc = 0.0f;
                for (int i = 0; i < d; ++i) {
                    float prod = bf16_to_f32(qv[i]) * bf16_to_f32(kv[i]);
                    acc = acc + prod;
                }
                if (!isnan(acc) && (isnan(best) || acc > best)) best = acc;
            }
            float s = sm_scale * best;
            if (s == 0.0f) s = 0.0f;
            scores[(int64_t)r * MP + p] = s;
        }
    }
    free(rq);
    free(rl);
    free(rn);
}

/* -------------------------------------------------------------- selection -- */

typedef struct { float s; int p; } cand_t;

/* Canonical order: score descending, then page index descending ("ties to the
   highest index"). -0 == +0 numerically. */
static int cand_cmp(const void *a, const void *b)
{
    const cand_t *x = a, *y = b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->p > y->p) ? -1 : (x->p < y->p) ? 1 : 0;
}

static int int_cmp(const void *a, const void *b)
{
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

/* Canonical QSA selection [PR20276, Features, "Canonical QSA selection" row;
   Decisions worth knowing]. The result depends on the scores, W and k alone:
   candidates scoring above the k-th largest value are kept, and among equal
   scores the larger page index ranks first, whatever the launch order.
   For each row: window = pages [max(0, n - W), n). Candidates = columns
   p < n - W whose score is neither NaN nor -inf. Take the first min(k, |C|)
   candidates in canonical order, add the window, sort ascending, and pad with -1
   to k + W entries. The page table is not read: a page that index scoring
   skipped carries -inf. */
void oracle_select(int B, const int32_t *seq_lens, const int32_t *row_offsets, int P, int MP,
                   int k, int W, const float *scores, int32_t *selected)
{
    int N = row_offsets[B];
    int32_t *rq = malloc(sizeof(int32_t) * (N > 0 ? N : 1));
    int32_t *rl = malloc(sizeof(int32_t) * (N > 0 ? N : 1));
    int32_t *rn = malloc(sizeof(int32_t) * (N > 0 ? N : 1));
    cand_t *c = malloc(sizeof(cand_t) * (MP > 0 ? MP : 1));
    int *out = malloc(sizeof(int) * (k + W > 0 ? k + W : 1));
    oracle_rows(B, seq_lens, row_offsets, P, MP, rq, rl, rn);
    for (int r = 0; r < N; ++r) {
        int n = rn[r];
        int wlo = n - W > 0 ? n - W : 0;
        int nc = 0;
        for (int p = 0; p < wlo; ++p) {
            float s = scores[(int64_t)r * MP + p];
            if (isnan(s) || s == -INFINITY) continue;
            c[nc].s = s;
            c[nc].p = p;
            ++nc;
        }
        qsort(c, nc, sizeof(cand_t), cand_cmp);
        int take = nc < k ? nc : k;
        int m = 0;
        for (int j = 0; j < take; ++j) out[m++] = c[j].p;
        for (int p = wlo; p < n; ++p) out[m++] = p;
        qsort(out, m, sizeof(int), int_cmp);
        for (int j = 0; j < k + W; ++j)
            selected[(int64_t)r * (k + W) + j] = (j < m) ? out[j] : -1;
    }
    free(rq);
    free(rl);
    free(rn);
    free(c);
    free(out);
}

/* -------------------------------------------------------------- attention -- */

/* Sparse GQA attention over the selected pages [PR20937, What changes > Decode at
   small batch: NVFP4 sparse GQA decode, split-K + merge; MTP > Verify: request-grouped
   sparse GQA with a per-row merge]. The splits and the merge are an implementation
   device: the result they compute is plain softmax attention over the token set
       T = { (p, j) : p listed in the row's selection (once), 0 <= p < MP,
                      page_table[b][p] valid, j < P, p * P + j < L_row }.
   For q head h (KV head h / G):
       logit_t = sm_scale * sum_i q[h][i] * K_t[i]        (K, V dequantised, fp64)
       out[h]  = sum_t exp(logit_t - m) V_t / sum_t exp(logit_t - m),  m = max logit
       lse[h]  = m + ln(sum_t exp(logit_t - m))
   An empty T gives out = 0 and lse = -inf. With a gate [PR20937, What changes > MTP >
   Verify: the gated epilogue], out[h][i] is multiplied by sigmoid(gate[row][h][i]) =
   1 / (1 + exp(-g)), g the bf16 gate value; lse is not gated. kv_format selects the cache
   format of K and V (0 NVFP4, 1 FP8). */
void oracle_attention(int B, const int32_t *seq_lens, const int32_t *row_offsets,
                      const int32_t *page_table, int MP, int64_t NP, int P,
                      int Hq, int Hkv, int d, float sm_scale, double k_global, double v_global,
                      const uint16_t *q, const uint8_t *k_codes, const uint8_t *k_scales,
                      const uint8_t *v_codes, const uint8_t *v_scales, int kv_format,
                      const int32_t *selected, int sel_width, const uint16_t *gate, double *out, double *lse)
{
    int N = row_offsets[B];
    int32_t *rq = malloc(sizeof(int32_t) * (N > 0 ? N : 1));
    int32_t *rl = malloc(sizeof(int32_t) * (N > 0 ? N : 1));
    int32_t *rn = malloc(sizeof(int32_t) * (N > 0 ? N : 1));
    char *listed = malloc(MP > 0 ? MP : 1);
    int64_t max_tok = (int64_t)sel_width * P;
    int32_t *tp = malloc(sizeof(int32_t) * (max_tok > 0 ? max_tok : 1));   /* physical page */
    int32_t *tt = malloc(sizeof(int32_t) * (max_tok > 0 ? max_tok : 1));   /* token in page */
    double *logit = malloc(sizeof(double) * (max_tok > 0 ? max_tok : 1));
    oracle_rows(B, seq_lens, row_offsets, P, MP, rq, rl, rn);
    int G = Hq / Hkv;
    for (int r = 0; r < N; ++r) {
        int b = rq[r];
        memset(listed, 0, MP > 0 ? MP : 1);
        for (int j = 0; j < sel_width; ++j) {
            int p = selected[(int64_t)r * sel_width + j];
            if (p >= 0 && p < MP) listed[p] = 1;
        }
        int64_t nt = 0;
        for (int p = 0; p < MP; ++p) {
            if (!listed[p]) continue;
            int32_t phys = page_table[(int64_t)b * MP + p];
            if (!valid_page(phys, NP)) continue;
            for (int j = 0; j < P; ++j) {
                if ((int64_t)p * P + j >= rl[r]) break;
                tp[nt] = phys;
                tt[nt] = j;
                ++nt;
            }
        }
        for (int h = 0; h < Hq; ++h) {
            const uint16_t *qv = q + ((int64_t)r * Hq + h) * d;
            double *o = out + ((int64_t)r * Hq + h) * d;
            int g = h / G;
            for (int i = 0; i < d; ++i) o[i] = 0.0;
            if (nt == 0) {
                lse[(int64_t)r * Hq + h] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int64_t t = 0; t < nt; ++t) {
                double dot = 0.0;
                for (int i = 0; i < d; ++i)
                    dot += oracle_bf16(qv[i]) *
                           kv_elem(kv_format, k_codes, k_scales, k_global, Hkv, P, d, tp[t], g, tt[t], i);
                logit[t] = (double)sm_scale * dot;
                if (logit[t] > m) m = logit[t];
            }
            double l = 0.0;
            for (int64_t t = 0; t < nt; ++t) {
                double w = exp(logit[t] - m);
                l += w;
                for (int i = 0; i < d; ++i)
                    o[i] += w * kv_elem(kv_format, v_codes, v_scales, v_global, Hkv, P, d, tp[t], g, tt[t], i);
            }
            for (int i = 0; i < d; ++i) o[i] /= l;
            if (gate) {
                const uint16_t *gv = gate + ((int64_t)r * Hq + h) * d;
                for (int i = 0; i < d; ++i) o[i] *= 1.0 / (1.0 + exp(-oracle_bf16(gv[i])));
            }
            lse[(int64_t)r * Hq + h] = m + log(l);
        }
    }
    free(rq);
    free(rl);
    free(rn);
    free(listed);
    free(tp);
    free(tt);
    free(logit);
}

/* Attention for one (row, q head) only: the same definition as oracle_attention,
   for sampled checks at sizes where the full oracle would take too long. */
void oracle_attention_one(int B, const int32_t *seq_lens, const int32_t *row_offsets,
                          const int32_t *page_table, int MP, int64_t NP, int P,
                          int Hq, int Hkv, int d, float sm_scale, double k_global, double v_global,
                          const uint16_t *q, const uint8_t *k_codes, const uint8_t *k_scales,
                          const uint8_t *v_codes, const uint8_t *v_scales, int kv_format,
                          const int32_t *selected, int sel_width, const uint16_t *gate, int row, int head,
                          double *out_d, double *lse_1)
{
    /* Run the full definition on a one-row, one-head view of the batch. */
    int b = 0;
    while (b < B && row_offsets[b + 1] <= row) ++b;
    int32_t ro[2] = {0, row_offsets[b + 1] - row_offsets[b]};
    int jrow = row - row_offsets[b];
    int R = ro[1];
    /* rows of this request, but only `jrow` gets a real selection; the others select nothing */
    int32_t *sel = malloc(sizeof(int32_t) * (size_t)R * (sel_width > 0 ? sel_width : 1));
    for (int x = 0; x < R * sel_width; ++x) sel[x] = -1;
    for (int x = 0; x < sel_width; ++x) sel[jrow * sel_width + x] = selected[(int64_t)row * sel_width + x];
    int G = Hq / Hkv;
    int g = head / G;
    /* one q head per KV head is enough: evaluate with Hq' = Hkv, head index g */
    uint16_t *qv = malloc(sizeof(uint16_t) * (size_t)R * Hkv * d);
    memset(qv, 0, sizeof(uint16_t) * (size_t)R * Hkv * d);
    memcpy(qv + ((size_t)jrow * Hkv + g) * d, q + ((int64_t)row * Hq + head) * d, sizeof(uint16_t) * d);
    double *o = malloc(sizeof(double) * (size_t)R * Hkv * d);
    double *ls = malloc(sizeof(double) * (size_t)R * Hkv);
    oracle_attention(1, seq_lens + b, ro, page_table + (int64_t)b * MP, MP, NP, P, Hkv, Hkv, d,
                     sm_scale, k_global, v_global, qv, k_codes, k_scales, v_codes, v_scales, kv_format,
                     sel, sel_width, NULL, o, ls);
    memcpy(out_d, o + ((size_t)jrow * Hkv + g) * d, sizeof(double) * d);
    *lse_1 = ls[(size_t)jrow * Hkv + g];
    if (gate) {
        const uint16_t *gv = gate + ((int64_t)row * Hq + head) * d;
        for (int i = 0; i < d; ++i) out_d[i] *= 1.0 / (1.0 + exp(-oracle_bf16(gv[i])));
    }
    free(sel);
    free(qv);
    free(o);
    free(ls);
}

/* ------------------------------------------------------------- KV store -- */
/*
 * The KV-store prologue of a decode / verify step [PR20276, Performance > What runs on
 * the fast paths: the decode prologue covers index store and compression; PR20937, What
 * changes: the prologue that writes a decode step's NVFP4 KV, fused]: this step's new K and V tokens are
 * quantised into their page slots, and the index key of every page that received a token
 * is recomputed. The pages fix neither the encoder's rounding nor the index compression;
 * this file takes these readings:
 *
 *   placement  row j of request b (R rows, L = seq_lens[b] tokens including the new ones)
 *              is the token at position pos = L - R + j, page pos / P, slot pos % P, in
 *              physical page page_table[b][pos / P] (skipped if that entry is not valid);
 *   scale      per block of 16 consecutive elements x (bf16 inputs, exact in fp32):
 *              amax = max |x|; t = fl32(fl32(amax / 6) / global); scale = the E4M3 code
 *              nearest to t (ties to the even code), at most 448 (code 0x7E);
 *   codes      with s = e4m3(scale) * global (fp32): c = the E2M1 code nearest to
 *              fl32(x / s) (ties to the even code), magnitude at most 6; all codes 0 when
 *              s == 0;
 *   index key  for each KV head and element i: bf16_RNE(fl32(S_i / n)), S_i the fp32 sum,
 *              in ascending token order, of the page's stored K (dequantised, exact in
 *              fp32) over its n = min(P, L - page * P) valid tokens.
 */

/* nearest code of a non-negative value among `n` increasing grid values (ties to the even code) */
static int nearest_even(double y, const double *grid, int n)
{
    int best = 0;
    for (int c = 1; c < n; ++c) {
        const double dc = fabs(y - grid[c]), db = fabs(y - grid[best]);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return best;
}

uint8_t oracle_e4m3_encode(float t)
{
    /* t >= 0; the 127 finite non-negative codes 0x00..0x7E in increasing order */
    double grid[127];
    for (int c = 0; c < 127; ++c) grid[c] = oracle_e4m3(c);
    if (t >= 448.0f) return 0x7E;
    return (uint8_t)nearest_even((double)t, grid, 127);
}

uint8_t oracle_e2m1_encode(float y)
{
    double grid[8];
    for (int c = 0; c < 8; ++c) grid[c] = oracle_e2m1(c);
    const int sign = y < 0.0f;
    const double a = fabs((double)y);
    const int mag = a >= 6.0 ? 7 : nearest_even(a, grid, 8);
    return (uint8_t)(mag | (sign && mag ? 8 : 0));
}

/* one block of 16 elements: codes[8] (low nibble = even element) and the scale byte */
void oracle_nvfp4_encode_block(const float *x, float global, uint8_t *codes, uint8_t *scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 16; ++i)
        if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
    const float t = (amax / 6.0f) / global;
    const uint8_t sc = oracle_e4m3_encode(t);
    const float s = (float)oracle_e4m3(sc) * global;
    for (int i = 0; i < 8; ++i) {
        uint8_t lo = 0, hi = 0;
        if (s != 0.0f) {
            lo = oracle_e2m1_encode(x[2 * i] / s);
            hi = oracle_e2m1_encode(x[2 * i + 1] / s);
        }
        codes[i] = (uint8_t)(lo | (hi << 4));
    }
    *scale = sc;
}

/* The whole store: writes the new tokens' codes and scales into the planes and rewrites
   the index keys of the pages that received a token. new_k / new_v: bf16 [N][Hkv][d]. */
void oracle_kv_store(int B, const int32_t *seq_lens, const int32_t *row_offsets, const int32_t *page_table,
                     int MP, int64_t NP, int Hkv, int P, int d, float k_global, float v_global,
                     const uint16_t *new_k, const uint16_t *new_v, uint8_t *k_codes, uint8_t *k_scales,
                     uint8_t *v_codes, uint8_t *v_scales, uint16_t *index_keys)
{
    for (int b = 0; b < B; ++b) {
        const int r0 = row_offsets[b], R = row_offsets[b + 1] - r0;
        const int64_t L = seq_lens[b];
        for (int j = 0; j < R; ++j) {
            const int64_t pos = L - R + j;
            if (pos < 0 || pos / P >= MP) continue;
            const int32_t phys = page_table[(int64_t)b * MP + pos / P];
            if (!valid_page(phys, NP)) continue;
            for (int h = 0; h < Hkv; ++h) {
                const int64_t tok = ((int64_t)phys * Hkv + h) * P + pos % P;
                for (int blk = 0; blk < d / 16; ++blk) {
                    float xk[16], xv[16];
                    for (int i = 0; i < 16; ++i) {
                        xk[i] = bf16_to_f32(new_k[((int64_t)(r0 + j) * Hkv + h) * d + blk * 16 + i]);
                        xv[i] = bf16_to_f32(new_v[((int64_t)(r0 + j) * Hkv + h) * d + blk * 16 + i]);
                    }
                    oracle_nvfp4_encode_block(xk, k_global, k_codes + tok * (d / 2) + blk * 8, k_scales + tok * (d / 16) + blk);
                    oracle_nvfp4_encode_block(xv, v_global, v_codes + tok * (d / 2) + blk * 8, v_scales + tok * (d / 16) + blk);
                }
            }
        }
        /* index keys of the pages that received a token */
        for (int j = 0; j < R; ++j) {
            const int64_t pos = L - R + j;
            if (pos < 0 || pos / P >= MP) continue;
            const int64_t page = pos / P;
            if (j > 0 && (L - R + j - 1) >= 0 && (L - R + j - 1) / P == page) continue;   /* page done already */
            const int32_t phys = page_table[(int64_t)b * MP + page];
            if (!valid_page(phys, NP)) continue;
            const int64_t n = L - page * P < P ? L - page * P : P;
            for (int h = 0; h < Hkv; ++h) {
                for (int i = 0; i < d; ++i) {
                    float S = 0.0f;
                    for (int64_t t = 0; t < n; ++t) {
                        S = S + (float)oracle_dequant_elem(k_codes, k_scales, k_global, Hkv, P, d, phys, h, (int)t, i);
                    }
                    const float mean = S / (float)n;
                    uint32_t u;
                    memcpy(&u, &mean, 4);
                    index_keys[((int64_t)phys * Hkv + h) * d + i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                }
            }
        }
    }
}
