/*
 * kvq_oracle.c -- plain, slow, obviously-correct CPU oracle for the decode step
 * of paged, quantized, query-aware sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header or constant with the HIP library; the two only agree on the storage
 * layout written out below, which each side states on its own.
 *
 * Sources (web pages, cited by title and section):
 *   [TS]  "TinyServe" query-aware page selection page (lpnh.cn): section 2.1
 *         (page metadata phi = per-channel min/max, score r, no-underestimate
 *         property), section 3.1 (four-phase decode: score, top-K, sparse load,
 *         reduce), section 5.1 (page_size 16, selection_ratio 0.3), section 5.2
 *         (fp32 metadata).
 *   [LY]  "KV-cache layout from the HBM-bandwidth viewpoint" (pzsr.cn):
 *         section 2 (paged layout C with 16-token pages; per-token dynamic
 *         INT8 from each token's own min/max, dequantized before attention),
 *         section 3 (block table, offset of (block, token, head, dim)).
 *   [GM]  "Gemini KV cache: FlashAttention-3 adaptation" (uyd888.cn): chapter 1
 *         (FP16 -> INT8 per-group quantization, 64 tokens share one
 *         scale/zero-point).
 *   [KV]  "KV-cache optimization and memory management" (intelliparadigm.com):
 *         section 2.1, Attention(Q,K,V) = softmax(Q K^T / sqrt(d)) V.
 *   [TS] section 6 also lists a mixed-precision cache: pages of high
 *         importance kept in FP16, the rest in INT8 (format MIXED below).
 *
 * Readings where the pages are silent:
 *   - quantization: unsigned codes 0..255 (INT8) or 0..15 (INT4, two per
 *     byte, channel 2i in the low nibble), zero = row minimum (fp32, a
 *     minimum of -0 stored as +0),
 *     scale = (max - min) / 255 in fp32, codes = clamp(rint((x - zero) * (1/scale)))
 *     with round-half-to-even and every operation rounded to fp32; a constant
 *     row gets scale 1 and all-zero codes; dequant = fmaf(code, scale, zero).
 *   - per-group: groups are 64-token runs aligned to logical position 64g,
 *     one (scale, zero) per (group, KV head) and per K / V, over the group's
 *     valid tokens and all channels; copied into each page of the group.
 *   - metadata: min/max of the keys as decoded (what attention reads).
 *   - GQA: query head h reads KV head h / G; the group's page score is the
 *     max over its G query heads.
 *   - K from the ratio: ceil(num * P / den) clamped to [1, P], in integers;
 *     ties go to the lower logical page index; output ascending.
 *   - attention: softmax over every valid token of the selected pages, with
 *     the 1/sqrt(d) scale of [KV] section 2.1, in fp64.
 *   - mixed precision: a page's precision is where it lives.  Physical pages
 *     0 .. n16-1 form an FP16 pool, n16 .. P_phys-1 an INT8 pool quantized
 *     per token; which pages are important is the caller's choice (it
 *     allocates them from the FP16 pool and demotes them later).
 *
 * Storage layout (caller-owned arrays, the paged layout C of [LY] section 2,
 * head-major inside each page so a (page, KV head) tile is contiguous):
 *   k_pages, v_pages : [P_phys][H_kv][16][d]   fp16 bits (FP16) or uint8 codes,
 *                      [P_phys][H_kv][16][d/2] packed 4-bit codes (INT4)
 *   params  INT8/INT4_TOKEN  : [P_phys][H_kv][16][4] fp32 (k_scale, k_zero, v_scale, v_zero)
 *           INT8/INT4_GROUP64: [P_phys][H_kv][4]     fp32, the group's values in each of its pages
 *   MIXED   : k_pages, v_pages = the FP16 pool [n16][H_kv][16][d] fp16 bits,
 *             then (at byte n16*H_kv*16*d*2) the INT8 pool [P_phys-n16][H_kv][16][d];
 *             params [P_phys-n16][H_kv][16][4] for the INT8 pool only
 *   meta    : [P_phys][H_kv][2][d] fp32, row 0 = per-channel min, row 1 = max
 *   block_table : [B][max_pages] int32, logical page j of sequence b -> physical page
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (x86-64 SSE arithmetic, FLT_EVAL_METHOD == 0: every float operation rounds to fp32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PAGE 16

enum { FMT_FP16 = 0, FMT_INT8_TOKEN = 1, FMT_INT8_GROUP64 = 2, FMT_INT4_TOKEN = 3, FMT_INT4_GROUP64 = 4,
       FMT_MIXED = 5 };

/* Storage formats that keep one (scale, zero) per token, and per 64-token   */
/* group; the largest code of each quantized format (INT8: 255, INT4: 15, the */
/* 4-bit row of the quantization table on the KV-cache optimization page,     */
/* section 3.2).                                                              */
static int per_token(int fmt) { return fmt == FMT_INT8_TOKEN || fmt == FMT_INT4_TOKEN; }
static int per_group(int fmt) { return fmt == FMT_INT8_GROUP64 || fmt == FMT_INT4_GROUP64; }
static int code_max(int fmt) { return fmt == FMT_INT4_TOKEN || fmt == FMT_INT4_GROUP64 ? 15 : 255; }

/* ------------------------------------------------------------------------- */
/* fp16 bits -> fp32, exactly, by decoding sign / exponent / mantissa.        */
/* ------------------------------------------------------------------------- */
static float half_bits_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    float v;
    if (expo == 0)
        v = ldexpf((float)mant, -24);                 /* zero and subnormals */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexpf((float)(mant | 0x400), expo - 25); /* (1024 + m) * 2^(e-25) */
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------- */
/* Asymmetric min/max INT8 quantization of one row ([LY] section 2 per token, */
/* [GM] chapter 1 per group).                                                 */
/* ------------------------------------------------------------------------- */
static void quant_scale_levels(float lo, float hi, int levels, float *scale, float *inv)
{
    if (hi > lo) {
        float range = hi - lo;          /* rounded to fp32 */
        *scale = range / (float)levels; /* IEEE divide, rounded to fp32 */
        *inv = 1.0f / *scale;           /* IEEE divide, rounded to fp32 */
    } else {
        *scale = 1.0f;
        *inv = 1.0f;
    }
}

static void quant_scale(float lo, float hi, float *scale, float *inv)
{
    quant_scale_levels(lo, hi, 255, scale, inv);
}

/* The zero-point is the row minimum; a minimum of -0 is stored as +0 (both  */
/* are the number zero, and -0 + 0 = +0 while x + 0 = x otherwise), so the   */
/* stored bits do not depend on which of two equal zeros came first.          */
static float zero_point(float lo)
{
    return lo + 0.0f;
}

static uint8_t quant_code_levels(float x, float zero, float inv, int levels)
{
    float shifted = x - zero;           /* rounded to fp32 */
    float t = shifted * inv;            /* rounded to fp32, not contracted */
    float r = rintf(t);                 /* round half to even */
    if (r < 0.0f) r = 0.0f;
    if (r > (float)levels) r = (float)levels;
    return (uint8_t)r;
}

static uint8_t quant_code(float x, float zero, float inv)
{
    return quant_code_levels(x, zero, inv, 255);
}

static float dequant(uint8_t c, float scale, float zero)
{
    return fmaf((float)c, scale, zero);
}

/* ------------------------------------------------------------------------- */
/* Addressing helpers for the layout above.                                   */
/* ------------------------------------------------------------------------- */
static size_t tile_elem(int phys, int h, int slot, int ch, int H, int d)
{
    return (((size_t)phys * H + h) * PAGE + slot) * (size_t)d + ch;
}

/* The code of channel ch of a token row: one byte (INT8), or one nibble of   */
/* the row's d/2 bytes (INT4: channel 2i in the low nibble of byte i, 2i+1 in */
/* its high nibble).                                                          */
static unsigned get_code(int fmt, const void *pages, int phys, int h, int slot, int ch, int H, int d)
{
    if (code_max(fmt) == 255)
        return ((const uint8_t *)pages)[tile_elem(phys, h, slot, ch, H, d)];
    uint8_t byte = ((const uint8_t *)pages)[tile_elem(phys, h, slot, ch / 2, H, d / 2)];
    return ch % 2 ? byte >> 4 : byte & 0xF;
}

static void put_code(int fmt, void *pages, int phys, int h, int slot, int ch, int H, int d, unsigned code)
{
    if (code_max(fmt) == 255) {
        ((uint8_t *)pages)[tile_elem(phys, h, slot, ch, H, d)] = (uint8_t)code;
        return;
    }
    uint8_t *byte = (uint8_t *)pages + tile_elem(phys, h, slot, ch / 2, H, d / 2);
    *byte = ch % 2 ? (uint8_t)((*byte & 0x0F) | (code << 4)) : (uint8_t)((*byte & 0xF0) | code);
}

/* Where physical page phys is stored: its own format, the array that holds */
/* it and its index there (a MIXED cache keeps two pools in one array, the  */
/* INT8 pool and its params indexed from 0).  Other formats: unchanged.     */
typedef struct {
    int fmt;
    const void *pages;
    const float *params;
    int idx;
} PageLoc;

static PageLoc locate(int fmt, int n16, const void *pages, const float *params, int phys, int H, int d)
{
    PageLoc l = {fmt, pages, params, phys};
    if (fmt == FMT_MIXED) {
        if (phys < n16) {
            l.fmt = FMT_FP16;
        } else {
            l.fmt = FMT_INT8_TOKEN;
            l.pages = (const uint8_t *)pages + (size_t)n16 * H * PAGE * d * 2;
            l.idx = phys - n16;
        }
    }
    return l;
}

/* The key of token t of sequence b, channel ch, as attention reads it. */
static float key_decoded(int fmt, int n16, const void *k_pages, const float *params,
                         const int32_t *bt_row, int t, int h, int ch, int H, int d)
{
    PageLoc l = locate(fmt, n16, k_pages, params, bt_row[t / PAGE], H, d);
    fmt = l.fmt;
    k_pages = l.pages;
    params = l.params;
    int phys = l.idx, slot = t % PAGE;
    if (fmt == FMT_FP16)
        return half_bits_to_float(((const uint16_t *)k_pages)[tile_elem(phys, h, slot, ch, H, d)]);
    const uint8_t c = (uint8_t)get_code(fmt, k_pages, phys, h, slot, ch, H, d);
    if (per_token(fmt)) {
        const float *p = params + (((size_t)phys * H + h) * PAGE + slot) * 4;
        return dequant(c, p[0], p[1]);
    }
    const float *p = params + ((size_t)phys * H + h) * 4;
    return dequant(c, p[0], p[1]);
}

static float value_decoded(int fmt, int n16, const void *v_pages, const float *params,
                           const int32_t *bt_row, int t, int h, int ch, int H, int d)
{
    PageLoc l = locate(fmt, n16, v_pages, params, bt_row[t / PAGE], H, d);
    fmt = l.fmt;
    v_pages = l.pages;
    params = l.params;
    int phys = l.idx, slot = t % PAGE;
    if (fmt == FMT_FP16)
        return half_bits_to_float(((const uint16_t *)v_pages)[tile_elem(phys, h, slot, ch, H, d)]);
    const uint8_t c = (uint8_t)get_code(fmt, v_pages, phys, h, slot, ch, H, d);
    if (per_token(fmt)) {
        const float *p = params + (((size_t)phys * H + h) * PAGE + slot) * 4;
        return dequant(c, p[2], p[3]);
    }
    const float *p = params + ((size_t)phys * H + h) * 4;
    return dequant(c, p[2], p[3]);
}

/* ------------------------------------------------------------------------- */
/* One token row of one KV head into slot `slot` of page `idx` of a pool of   */
/* format fmt: an fp16 copy, or one (scale, zero) per token and per K / V     */
/* ([LY] section 2), codes of `levels` + 1 values.                            */
/* ------------------------------------------------------------------------- */
static void write_token(int fmt, void *k_pages, void *v_pages, float *params, int idx, int h, int slot,
                        const uint16_t *kr, const uint16_t *vr, int H, int d)
{
    if (fmt == FMT_FP16) {
        for (int ch = 0; ch < d; ++ch) {
            size_t e = tile_elem(idx, h, slot, ch, H, d);
            ((uint16_t *)k_pages)[e] = kr[ch];
            ((uint16_t *)v_pages)[e] = vr[ch];
        }
        return;
    }
    float klo = INFINITY, khi = -INFINITY, vlo = INFINITY, vhi = -INFINITY;
    for (int ch = 0; ch < d; ++ch) {
        float kx = half_bits_to_float(kr[ch]), vx = half_bits_to_float(vr[ch]);
        if (kx < klo) klo = kx;
        if (kx > khi) khi = kx;
        if (vx < vlo) vlo = vx;
        if (vx > vhi) vhi = vx;
    }
    float ks, kinv, vs, vinv;
    int levels = code_max(fmt);
    klo = zero_point(klo);
    vlo = zero_point(vlo);
    quant_scale_levels(klo, khi, levels, &ks, &kinv);
    quant_scale_levels(vlo, vhi, levels, &vs, &vinv);
    for (int ch = 0; ch < d; ++ch) {
        put_code(fmt, k_pages, idx, h, slot, ch, H, d, quant_code_levels(half_bits_to_float(kr[ch]), klo, kinv, levels));
        put_code(fmt, v_pages, idx, h, slot, ch, H, d, quant_code_levels(half_bits_to_float(vr[ch]), vlo, vinv, levels));
    }
    float *p = params + (((size_t)idx * H + h) * PAGE + slot) * 4;
    p[0] = ks; p[1] = klo; p[2] = vs; p[3] = vlo;
}

/* ------------------------------------------------------------------------- */
/* Append: write new tokens into their paged slots, quantizing as the format says.*/
/*                                                                            */
/* Sequence b receives rows new_off[b] .. new_off[b+1]-1 of k_new / v_new     */
/* ([N][H][d] fp16 bits) at logical positions start_pos[b], start_pos[b]+1, . */
/* Token t goes to physical page block_table[b][t/16], slot t%16 ([LY]        */
/* section 3); in a MIXED cache it takes the format of that page's pool.      */
/* For the per-group formats, start_pos[b] must be a multiple of 64 and the   */
/* rows must include every token of each group they touch.                   */
/* Returns 0, or -1 on a precondition violation.                              */
/* ------------------------------------------------------------------------- */
int kvqo_append(int fmt, int n16, int B, int H, int d, int max_pages,
                const int32_t *block_table, const int32_t *start_pos, const int32_t *new_off,
                const uint16_t *k_new, const uint16_t *v_new,
                void *k_pages, void *v_pages, float *params)
{
    for (int b = 0; b < B; ++b) {
        const int32_t *bt = block_table + (size_t)b * max_pages;
        int start = start_pos[b];
        int n = new_off[b + 1] - new_off[b];
        const uint16_t *kb = k_new + (size_t)new_off[b] * H * d;
        const uint16_t *vb = v_new + (size_t)new_off[b] * H * d;
        if (n < 0 || start < 0 || (start + n + PAGE - 1) / PAGE > max_pages)
            return -1;
        if (fmt == FMT_FP16 || per_token(fmt) || fmt == FMT_MIXED) {
            for (int i = 0; i < n; ++i) {
                int t = start + i;
                PageLoc kl = locate(fmt, n16, k_pages, params, bt[t / PAGE], H, d);
                PageLoc vl = locate(fmt, n16, v_pages, params, bt[t / PAGE], H, d);
                for (int h = 0; h < H; ++h)
                    write_token(kl.fmt, (void *)kl.pages, (void *)vl.pages, (float *)kl.params, kl.idx, h,
                                t % PAGE, kb + ((size_t)i * H + h) * d, vb + ((size_t)i * H + h) * d, H, d);
            }
        } else if (per_group(fmt)) {
            /* one (scale, zero) per 64-token logical group, KV head, and K / V */
            if (n > 0 && start % 64 != 0)
                return -1;
            for (int g0 = 0; g0 < n; g0 += 64) {
                int gn = n - g0 < 64 ? n - g0 : 64;      /* valid tokens of this group */
                for (int h = 0; h < H; ++h) {
                    float klo = INFINITY, khi = -INFINITY, vlo = INFINITY, vhi = -INFINITY;
                    for (int i = g0; i < g0 + gn; ++i)
                        for (int ch = 0; ch < d; ++ch) {
                            float kx = half_bits_to_float(kb[((size_t)i * H + h) * d + ch]);
                            float vx = half_bits_to_float(vb[((size_t)i * H + h) * d + ch]);
                            if (kx < klo) klo = kx;
                            if (kx > khi) khi = kx;
                            if (vx < vlo) vlo = vx;
                            if (vx > vhi) vhi = vx;
                        }
                    float ks, kinv, vs, vinv;
                    int levels = code_max(fmt);
                    klo = zero_point(klo);
                    vlo = zero_point(vlo);
                    quant_scale_levels(klo, khi, levels, &ks, &kinv);
                    quant_scale_levels(vlo, vhi, levels, &vs, &vinv);
                    for (int i = g0; i < g0 + gn; ++i) {
                        int t = start + i;
                        int phys = bt[t / PAGE], slot = t % PAGE;
                        for (int ch = 0; ch < d; ++ch) {
                            float kx = half_bits_to_float(kb[((size_t)i * H + h) * d + ch]);
                            float vx = half_bits_to_float(vb[((size_t)i * H + h) * d + ch]);
                            put_code(fmt, k_pages, phys, h, slot, ch, H, d, quant_code_levels(kx, klo, kinv, levels));
                            put_code(fmt, v_pages, phys, h, slot, ch, H, d, quant_code_levels(vx, vlo, vinv, levels));
                        }
                        float *p = params + ((size_t)phys * H + h) * 4;   /* every page of the group */
                        p[0] = ks; p[1] = klo; p[2] = vs; p[3] = vlo;
                    }
                }
            }
        } else {
            return -1;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Page metadata phi(K_j) = (m_j, M_j), the per-channel min and max of   */
/* the page's keys ([TS] section 2.1), in fp32 ([TS] section 5.2), over the   */
/* valid tokens of logical pages page_begin[b] .. P_b-1 (page_begin NULL: 0). */
/* ------------------------------------------------------------------------- */
void kvqo_page_meta(int fmt, int n16, int B, int H, int d, int max_pages,
                    const int32_t *block_table, const int32_t *seq_lens, const int32_t *page_begin,
                    const void *k_pages, const float *params, float *meta)
{
    for (int b = 0; b < B; ++b) {
        const int32_t *bt = block_table + (size_t)b * max_pages;
        int L = seq_lens[b];
        int P = (L + PAGE - 1) / PAGE;
        for (int j = page_begin ? page_begin[b] : 0; j < P; ++j) {
            int t0 = j * PAGE, t1 = (j + 1) * PAGE < L ? (j + 1) * PAGE : L;
            int phys = bt[j];
            for (int h = 0; h < H; ++h) {
                float *mn = meta + ((size_t)phys * H + h) * 2 * d;
                float *mx = mn + d;
                for (int ch = 0; ch < d; ++ch) {
                    float lo = INFINITY, hi = -INFINITY;
                    for (int t = t0; t < t1; ++t) {
                        float k = key_decoded(fmt, n16, k_pages, params, bt, t, h, ch, H, d);
                        if (k < lo) lo = k;
                        if (k > hi) hi = k;
                    }
                    mn[ch] = lo;
                    mx[ch] = hi;
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Page relevance r(q, phi) = sum_i (q_i >= 0 ? q_i M_i : q_i m_i)        */
/* ([TS] section 2.1), fp64, summed in channel order.  The KV group's score   */
/* is the max over its G = Hq/H query heads.  Pages j >= P_b score -inf.      */
/* scores: [B][H][max_pages] double.                                          */
/* ------------------------------------------------------------------------- */
static double page_score_one(const uint16_t *q, const float *mn, const float *mx, int d)
{
    double r = 0.0;
    for (int i = 0; i < d; ++i) {
        double qi = (double)half_bits_to_float(q[i]);
        r += qi >= 0.0 ? qi * (double)mx[i] : qi * (double)mn[i];
    }
    return r;
}

static void scores_unit(int b, int g, int Hq, int H, int d, int max_pages,
                        const int32_t *block_table, const int32_t *seq_lens,
                        const uint16_t *q, const float *meta, double *scores)
{
    int G = Hq / H;
    int P = (seq_lens[b] + PAGE - 1) / PAGE;
    const int32_t *bt = block_table + (size_t)b * max_pages;
    double *row = scores + ((size_t)b * H + g) * max_pages;
    for (int j = 0; j < max_pages; ++j) {
        if (j >= P) { row[j] = -INFINITY; continue; }
        const float *mn = meta + ((size_t)bt[j] * H + g) * 2 * d;
        double best = -INFINITY;
        for (int hh = 0; hh < G; ++hh) {
            int h = g * G + hh;
            double r = page_score_one(q + ((size_t)b * Hq + h) * d, mn, mn + d, d);
            if (r > best) best = r;
        }
        row[j] = best;
    }
}

void kvqo_page_scores(int B, int Hq, int H, int d, int max_pages,
                      const int32_t *block_table, const int32_t *seq_lens,
                      const uint16_t *q, const float *meta, double *scores)
{
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < H; ++g)
            scores_unit(b, g, Hq, H, d, max_pages, block_table, seq_lens, q, meta, scores);
}

/* ------------------------------------------------------------------------- */
/* Top-K pages per (sequence, KV head) ([TS] section 3.1 phase 2 and      */
/* section 5.1 selection_ratio).                                              */
/* ------------------------------------------------------------------------- */
int kvqo_num_selected(int P, int ratio_num, int ratio_den, int k_fixed)
{
    long long k;
    if (P <= 0) return 0;
    if (k_fixed > 0)
        k = k_fixed;
    else
        k = ((long long)ratio_num * P + ratio_den - 1) / ratio_den;   /* ceil(num*P/den) */
    if (k < 1) k = 1;
    if (k > P) k = P;
    return (int)k;
}

typedef struct { double score; int page; } scored_page;

static int by_score_desc_then_page(const void *a, const void *b)
{
    const scored_page *x = a, *y = b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->page > y->page) - (x->page < y->page);
}

static int by_page_asc(const void *a, const void *b)
{
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

static void topk_unit(int b, int g, int H, int max_pages, const int32_t *seq_lens, const double *scores,
                      int ratio_num, int ratio_den, int k_fixed, int k_cap,
                      int32_t *sel_pages, int32_t *sel_count)
{
    int P = (seq_lens[b] + PAGE - 1) / PAGE;
    int K = kvqo_num_selected(P, ratio_num, ratio_den, k_fixed);
    const double *row = scores + ((size_t)b * H + g) * max_pages;
    int32_t *out = sel_pages + ((size_t)b * H + g) * k_cap;
    scored_page *order = malloc(sizeof(scored_page) * (P > 0 ? P : 1));
    int *chosen = malloc(sizeof(int) * (K > 0 ? K : 1));
    for (int j = 0; j < P; ++j) { order[j].score = row[j]; order[j].page = j; }
    qsort(order, P, sizeof(scored_page), by_score_desc_then_page);
    for (int i = 0; i < K; ++i) chosen[i] = order[i].page;
    qsort(chosen, K, sizeof(int), by_page_asc);
    for (int i = 0; i < k_cap; ++i) out[i] = i < K ? chosen[i] : -1;
    sel_count[(size_t)b * H + g] = K;
    free(order);
    free(chosen);
}

int kvqo_topk(int B, int H, int max_pages, const int32_t *seq_lens, const double *scores,
              int ratio_num, int ratio_den, int k_fixed, int k_cap,
              int32_t *sel_pages, int32_t *sel_count)
{
    for (int b = 0; b < B; ++b) {
        int P = (seq_lens[b] + PAGE - 1) / PAGE;
        if (kvqo_num_selected(P, ratio_num, ratio_den, k_fixed) > k_cap) return -1;
    }
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < H; ++g)
            topk_unit(b, g, H, max_pages, seq_lens, scores, ratio_num, ratio_den, k_fixed, k_cap,
                      sel_pages, sel_count);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Hierarchical selection, coarse then fine ([TS] section 6: for large       */
/* models, screen coarsely first, then finely).  Reading: a super-page is     */
/* `group` consecutive logical pages of a sequence; its bounding box is the   */
/* channel-wise min of the member pages' minima and max of their maxima, so   */
/* its score (the page score formula on that box) is at least every member    */
/* page's score.  The top kc super-pages by that score survive, and only      */
/* their pages keep their fine scores; every other page scores -inf before    */
/* the usual top-K.                                                           */
/*                                                                            */
/* Coarse boxes: coarse[b * pc_max + jc][h] = (min row, max row) over the     */
/* valid pages j of super-page jc (group jc <= j < group (jc+1), j < P_b).    */
/* The layout is that of page metadata with "physical page" b * pc_max + jc,  */
/* so page scores on it are the coarse scores.  Super-pages past the          */
/* sequence's pages are left untouched.                                       */
/* ------------------------------------------------------------------------- */
void kvqo_coarse_meta(int B, int H, int d, int max_pages, const int32_t *block_table,
                      const int32_t *seq_lens, int group, const float *meta, float *coarse)
{
    int pc_max = (max_pages + group - 1) / group;
    for (int b = 0; b < B; ++b) {
        const int32_t *bt = block_table + (size_t)b * max_pages;
        int P = (seq_lens[b] + PAGE - 1) / PAGE;
        int Pc = (P + group - 1) / group;
        for (int jc = 0; jc < Pc; ++jc)
            for (int h = 0; h < H; ++h) {
                float *out = coarse + (((size_t)b * pc_max + jc) * H + h) * 2 * d;
                for (int ch = 0; ch < d; ++ch) {
                    float lo = INFINITY, hi = -INFINITY;
                    for (int j = jc * group; j < (jc + 1) * group && j < P; ++j) {
                        const float *m = meta + ((size_t)bt[j] * H + h) * 2 * d;
                        if (m[ch] < lo) lo = m[ch];
                        if (m[d + ch] > hi) hi = m[d + ch];
                    }
                    out[ch] = lo;
                    out[d + ch] = hi;
                }
            }
    }
}

/* The fine scores kept after the coarse screen: scores[b][h][j] stays for     */
/* pages j whose super-page j / group is among sel_super[b][h][0 .. count),    */
/* and becomes -inf for every other page (in place).                          */
void kvqo_mask_scores(int B, int H, int max_pages, int group, const int32_t *sel_super,
                      const int32_t *sel_super_count, int kc_cap, double *scores)
{
    int pc_max = (max_pages + group - 1) / group;
    char *keep = malloc((size_t)pc_max + 1);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            memset(keep, 0, (size_t)pc_max + 1);
            const int32_t *sel = sel_super + ((size_t)b * H + h) * kc_cap;
            for (int i = 0; i < sel_super_count[(size_t)b * H + h]; ++i)
                if (sel[i] >= 0 && sel[i] < pc_max) keep[sel[i]] = 1;
            double *row = scores + ((size_t)b * H + h) * max_pages;
            for (int j = 0; j < max_pages; ++j)
                if (!keep[j / group]) row[j] = -INFINITY;
        }
    free(keep);
}

/* ------------------------------------------------------------------------- */
/* Attention of each query head over every valid token of the selected   */
/* pages of its KV group: softmax(q k^T * sm_scale) v ([KV] section 2.1;      */
/* [TS] section 3.1 phases 3-4), fp64.  sel_pages NULL: all pages.            */
/* out: [B][Hq][d] double.                                                    */
/* ------------------------------------------------------------------------- */
static void attention_unit(int fmt, int n16, int b, int g, int Hq, int H, int d, int max_pages,
                           const int32_t *block_table, const int32_t *seq_lens, const uint16_t *q,
                           const void *k_pages, const void *v_pages, const float *params,
                           const int32_t *sel_pages, const int32_t *sel_count, int k_cap,
                           double sm_scale, double *out)
{
    int G = Hq / H;
    int L = seq_lens[b];
    int P = (L + PAGE - 1) / PAGE;
    const int32_t *bt = block_table + (size_t)b * max_pages;
    int npages = sel_pages ? sel_count[(size_t)b * H + g] : P;
    /* the tokens U of the selected pages */
    int *tok = malloc(sizeof(int) * ((size_t)npages * PAGE + 1));
    int ntok = 0;
    for (int s = 0; s < npages; ++s) {
        int j = sel_pages ? sel_pages[((size_t)b * H + g) * k_cap + s] : s;
        for (int t = j * PAGE; t < (j + 1) * PAGE && t < L; ++t) tok[ntok++] = t;
    }
    double *logit = malloc(sizeof(double) * (ntok + 1));
    for (int hh = 0; hh < G; ++hh) {
        int h = g * G + hh;
        const uint16_t *qh = q + ((size_t)b * Hq + h) * d;
        double *o = out + ((size_t)b * Hq + h) * d;
        double mu = -INFINITY;
        for (int u = 0; u < ntok; ++u) {
            double dot = 0.0;
            for (int i = 0; i < d; ++i)
                dot += (double)half_bits_to_float(qh[i]) *
                       (double)key_decoded(fmt, n16, k_pages, params, bt, tok[u], g, i, H, d);
            logit[u] = dot * sm_scale;
            if (logit[u] > mu) mu = logit[u];
        }
        double denom = 0.0;
        for (int i = 0; i < d; ++i) o[i] = 0.0;
        for (int u = 0; u < ntok; ++u) {
            double w = exp(logit[u] - mu);
            denom += w;
            for (int i = 0; i < d; ++i)
                o[i] += w * (double)value_decoded(fmt, n16, v_pages, params, bt, tok[u], g, i, H, d);
        }
        for (int i = 0; i < d; ++i) o[i] = ntok ? o[i] / denom : 0.0;
    }
    free(logit);
    free(tok);
}

void kvqo_attention(int fmt, int n16, int B, int Hq, int H, int d, int max_pages,
                    const int32_t *block_table, const int32_t *seq_lens, const uint16_t *q,
                    const void *k_pages, const void *v_pages, const float *params,
                    const int32_t *sel_pages, const int32_t *sel_count, int k_cap,
                    double sm_scale, double *out)
{
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < H; ++g)
            attention_unit(fmt, n16, b, g, Hq, H, d, max_pages, block_table, seq_lens, q, k_pages, v_pages,
                           params, sel_pages, sel_count, k_cap, sm_scale, out);
}

/* ------------------------------------------------------------------------- */
/* Selection quality: the share of dense attention that the selected pages    */
/* carry.  For (b, h): the softmax weights w_t = exp(l_t - mu) / sum_t' ... of */
/* every valid token t of sequence b (l_t = q.k_t * sm_scale, the dense       */
/* attention of [KV] section 2.1), summed over the tokens of the pages        */
/* selected for (b, h / G).  1 when every page is selected.  fp64.            */
/* out: [B][Hq] double; 0 for an empty sequence.                              */
/* ------------------------------------------------------------------------- */
void kvqo_attention_mass(int fmt, int n16, int B, int Hq, int H, int d, int max_pages,
                         const int32_t *block_table, const int32_t *seq_lens, const uint16_t *q,
                         const void *k_pages, const float *params,
                         const int32_t *sel_pages, const int32_t *sel_count, int k_cap,
                         double sm_scale, double *out)
{
    int G = Hq / H;
    for (int b = 0; b < B; ++b) {
        int L = seq_lens[b];
        int P = (L + PAGE - 1) / PAGE;
        const int32_t *bt = block_table + (size_t)b * max_pages;
        double *logit = malloc(sizeof(double) * ((size_t)L + 1));
        char *chosen = calloc((size_t)P + 1, 1);
        for (int h = 0; h < Hq; ++h) {
            int g = h / G;
            const uint16_t *qh = q + ((size_t)b * Hq + h) * d;
            memset(chosen, 0, (size_t)P + 1);
            for (int s = 0; s < sel_count[(size_t)b * H + g]; ++s) {
                int j = sel_pages[((size_t)b * H + g) * k_cap + s];
                if (j >= 0 && j < P) chosen[j] = 1;
            }
            double mu = -INFINITY;
            for (int t = 0; t < L; ++t) {
                double dot = 0.0;
                for (int i = 0; i < d; ++i)
                    dot += (double)half_bits_to_float(qh[i]) *
                           (double)key_decoded(fmt, n16, k_pages, params, bt, t, g, i, H, d);
                logit[t] = dot * sm_scale;
                if (logit[t] > mu) mu = logit[t];
            }
            double all = 0.0, sel = 0.0;
            for (int t = 0; t < L; ++t) {
                double w = exp(logit[t] - mu);
                all += w;
                if (chosen[t / PAGE]) sel += w;
            }
            out[(size_t)b * Hq + h] = L ? sel / all : 0.0;
        }
        free(chosen);
        free(logit);
    }
}

/* ------------------------------------------------------------------------- */
/* One decode step: scores -> top-K -> attention, over the (sequence, KV head) units,   */
/* which are independent; nthreads host threads take whole units.             */
/* scores / sel_pages / sel_count / out are outputs as above.                 */
/* ------------------------------------------------------------------------- */
int kvqo_decode_step(int fmt, int n16, int B, int Hq, int H, int d, int max_pages,
                     const int32_t *block_table, const int32_t *seq_lens, const uint16_t *q,
                     const void *k_pages, const void *v_pages, const float *params, const float *meta,
                     int ratio_num, int ratio_den, int k_fixed, int k_cap, double sm_scale,
                     double *scores, int32_t *sel_pages, int32_t *sel_count, double *out, int nthreads)
{
    for (int b = 0; b < B; ++b) {
        int P = (seq_lens[b] + PAGE - 1) / PAGE;
        if (kvqo_num_selected(P, ratio_num, ratio_den, k_fixed) > k_cap) return -1;
    }
    long units = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (long u = 0; u < units; ++u) {
        int b = (int)(u / H), g = (int)(u % H);
        scores_unit(b, g, Hq, H, d, max_pages, block_table, seq_lens, q, meta, scores);
        topk_unit(b, g, H, max_pages, seq_lens, scores, ratio_num, ratio_den, k_fixed, k_cap,
                  sel_pages, sel_count);
        attention_unit(fmt, n16, b, g, Hq, H, d, max_pages, block_table, seq_lens, q, k_pages, v_pages,
                       params, sel_pages, sel_count, k_cap, sm_scale, out);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Demotion in a MIXED cache ([TS] section 6: pages that are no longer of     */
/* high importance leave FP16 for INT8).  Item i moves logical page page[i]   */
/* of sequence seq[i] from its FP16 page to INT8 page dst[i]: every valid     */
/* token of the page is quantized per token from its fp16 rows (as an append  */
/* of those rows to dst would), the block-table entry becomes dst[i], and the */
/* page's metadata is rebuilt from the new decoded keys.  Slots at or past    */
/* the sequence's length are not written.  Returns 0, or -1 if an item does   */
/* not move an FP16 page of the sequence to an INT8 page.                     */
/* ------------------------------------------------------------------------- */
int kvqo_demote(int n16, int n_phys, int B, int H, int d, int max_pages, int32_t *block_table,
                const int32_t *seq_lens, int n, const int32_t *seq, const int32_t *page, const int32_t *dst,
                void *k_pages, void *v_pages, float *params, float *meta)
{
    for (int i = 0; i < n; ++i) {
        int b = seq[i], j = page[i];
        if (b < 0 || b >= B || j < 0 || j >= max_pages) return -1;
        int L = seq_lens[b];
        int32_t *bt = block_table + (size_t)b * max_pages;
        int src = bt[j];
        if (j * PAGE >= L || src < 0 || src >= n16 || dst[i] < n16 || dst[i] >= n_phys) return -1;
        PageLoc from = locate(FMT_MIXED, n16, k_pages, params, src, H, d);
        PageLoc kto = locate(FMT_MIXED, n16, k_pages, params, dst[i], H, d);
        PageLoc vto = locate(FMT_MIXED, n16, v_pages, params, dst[i], H, d);
        for (int t = j * PAGE; t < (j + 1) * PAGE && t < L; ++t)
            for (int h = 0; h < H; ++h) {
                const uint16_t *kr = (const uint16_t *)k_pages + tile_elem(from.idx, h, t % PAGE, 0, H, d);
                const uint16_t *vr = (const uint16_t *)v_pages + tile_elem(from.idx, h, t % PAGE, 0, H, d);
                write_token(FMT_INT8_TOKEN, (void *)kto.pages, (void *)vto.pages, (float *)kto.params, kto.idx, h,
                            t % PAGE, kr, vr, H, d);
            }
        bt[j] = dst[i];
        int32_t begin = j;
        int32_t lens1 = (j + 1) * PAGE < L ? (j + 1) * PAGE : L;   /* the page's tokens only */
        kvqo_page_meta(FMT_MIXED, n16, 1, H, d, max_pages, bt, &lens1, &begin, k_pages, params, meta);
    }
    return 0;
}

/* Exported element helpers, so tests can probe single values. */
float kvqo_half_to_float(uint16_t h) { return half_bits_to_float(h); }
float kvqo_dequant(uint8_t c, float scale, float zero) { return dequant(c, scale, zero); }
void kvqo_quant_scale(float lo, float hi, float *scale, float *inv) { quant_scale(lo, hi, scale, inv); }
uint8_t kvqo_quant_code(float x, float zero, float inv) { return quant_code(x, zero, inv); }
void kvqo_quant_scale_levels(float lo, float hi, int levels, float *scale, float *inv)
{
    quant_scale_levels(lo, hi, levels, scale, inv);
}
uint8_t kvqo_quant_code_levels(float x, float zero, float inv, int levels)
{
    return quant_code_levels(x, zero, inv, levels);
}
