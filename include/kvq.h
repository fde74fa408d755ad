/*
 * kvq.h -- C ABI of the MI355X (gfx950) decode-step library for paged,
 * quantized, query-aware sparse attention (libkvq.so).
 *
 * The decode step it implements, cited by page title and section:
 *   - KV cache in 16-token pages reached through a per-sequence block table
 *     ("KV-cache layout from the HBM-bandwidth viewpoint", pzsr.cn, section 2
 *     layout C and section 3 block tables; "TinyServe", lpnh.cn, section 5.1
 *     page_size 16);
 *   - storage as fp16, INT8 per token (same pzsr.cn page, section 2: each
 *     token's vector quantized with its own min/max) or INT8 per 64-token group
 *     ("Gemini KV cache: FlashAttention-3 adaptation", uyd888.cn, chapter 1),
 *     4-bit codes, or mixed precision (FP16 for the pages of high importance,
 *     INT8 for the rest: "TinyServe", section 6);
 *   - per-page fp32 metadata phi(K_j) = (per-channel min, per-channel max) of
 *     the page's keys, page score r = sum_i (q_i >= 0 ? q_i M_i : q_i m_i),
 *     top-K page selection, attention over the selected pages only
 *     ("TinyServe", sections 2.1, 3.1, 5.1, 5.2);
 *   - Attention(Q,K,V) = softmax(Q K^T / sqrt(d)) V ("KV-cache optimization and
 *     memory management", intelliparadigm.com, section 2.1).
 *
 * Conventions shared by every entry point:
 *   - Every array pointer is DEVICE memory owned by the caller, unless a
 *     comment says otherwise.  The library never allocates or frees memory and
 *     keeps no state between calls beyond a one-time, read-only lookup of
 *     each device's occupancy limits (on the first launch on that device);
 *     calls are reentrant.
 *   - Each call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *     default stream) and returns.  Nothing synchronizes.  The caller keeps the
 *     buffers alive until the stream has drained.
 *   - Host-checkable arguments are validated before anything is enqueued; a
 *     rejected call enqueues nothing and returns the status.  A failed launch
 *     returns KVQ_ERR_HIP.  Contents of device arrays are preconditions, listed
 *     per call, that the library does not check.
 *   - Page size is 16 tokens, head_dim is 64 or 128, H_q is a multiple of
 *     H_kv with group size G = H_q / H_kv in {1, 2, 4, 8}; query head h reads
 *     KV head h / G.
 *
 * Storage layout of one layer's cache (all C-contiguous):
 *   k_pages, v_pages   [P_phys][H_kv][16][d]  fp16 bits (KVQ_FP16) or uint8 codes (INT8);
 *                      [P_phys][H_kv][16][d/2] packed 4-bit codes (INT4: channel 2i in
 *                      the low nibble of byte i, 2i+1 in its high nibble)
 *   kv_params          *_TOKEN  : [P_phys][H_kv][16][4] fp32
 *                                 (k_scale, k_zero, v_scale, v_zero) per token slot
 *                      *_GROUP64: [P_phys][H_kv][4] fp32, the 64-token
 *                                 group's values repeated in each of its pages
 *                      KVQ_FP16 : unused (may be NULL)
 *   KVQ_MIXED_FP16_INT8: physical pages 0 .. n16-1 (n16 = num_fp16_pages) are
 *                      the FP16 pool and pages n16 .. P_phys-1 the INT8-per-token
 *                      pool.  k_pages (v_pages) is one array: the FP16 pool
 *                      [n16][H_kv][16][d] fp16 bits, then, at byte
 *                      n16 * H_kv * 16 * d * 2, the INT8 pool [P_phys-n16][H_kv][16][d];
 *                      kv_params is [P_phys-n16][H_kv][16][4] for the INT8 pool
 *                      (its page p - n16).  Which pages are important is the
 *                      caller's choice: it allocates them from the FP16 pool and
 *                      moves them later with kvq_demote_pages.
 *   page_meta          [P_phys][H_kv][2][d] fp32: row 0 per-channel min, row 1 max
 * A stored key or value decodes to fmaf(code, scale, zero) (INT8) or to the
 * fp16 value (FP16).  Codes are unsigned 0..255 (INT8) or 0..15 (INT4, the
 * 4-bit row of the quantization table on the KV-cache optimization page,
 * section 3.2) with zero = the quantized row's minimum (a minimum of -0 is
 * stored as +0) and scale = (max - min) / 255 (or / 15); a constant row has
 * scale 1.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 8
#define KVQ_PAGE_SIZE 16
#define KVQ_SELECT_MAX_PAGES 2048 /* longest row (pages) kvq_select_decode_attn takes */

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = 1,   /* null pointer, negative size, inconsistent shape */
    KVQ_ERR_UNSUPPORTED = 2,   /* page size, head_dim, group size or row length not built */
    KVQ_ERR_WORKSPACE = 3,     /* workspace missing or smaller than kvq_attn_workspace_bytes() */
    KVQ_ERR_HIP = 4            /* a HIP launch failed */
} kvq_status;

typedef enum {
    KVQ_FP16 = 0,
    KVQ_INT8_TOKEN = 1,
    KVQ_INT8_GROUP64 = 2,
    KVQ_INT4_TOKEN = 3,    /* 4-bit codes, head_dim 128 only */
    KVQ_INT4_GROUP64 = 4,  /* 4-bit codes, head_dim 128 only */
    KVQ_MIXED_FP16_INT8 = 5 /* FP16 pool + INT8-per-token pool (layout above) */
} kvq_format;

/* Non-owning view of one layer's paged cache (host struct, device pointers). */
typedef struct {
    int32_t format;            /* kvq_format */
    int32_t num_phys_pages;    /* P_phys */
    int32_t page_size;         /* must be 16 */
    int32_t num_kv_heads;      /* H_kv */
    int32_t head_dim;          /* d: 64 or 128 */
    void *k_pages;
    void *v_pages;
    float *kv_params;
    float *page_meta;
    int32_t num_fp16_pages;    /* KVQ_MIXED_FP16_INT8: n16, 0 <= n16 <= P_phys; otherwise ignored */
} kvq_cache;

/* The batch of sequences (host struct, device pointers). */
typedef struct {
    int32_t batch;                 /* B >= 1 */
    int32_t max_pages;             /* block-table row stride, >= ceil(L_b / 16) for every b */
    const int32_t *seq_lens;       /* [B] tokens in each sequence, 1 <= L_b <= 16 * max_pages */
    const int32_t *block_table;    /* [B][max_pages] physical page of each logical page;
                                      entries j < ceil(L_b/16) lie in [0, P_phys) */
} kvq_seqs;

/*
 * kvq_append_quant -- write new tokens into their paged slots.
 * (pzsr.cn layout page, sections 2-3: token t of sequence b goes to physical
 * page block_table[b][t/16], slot t%16; per-token INT8 from the token's own
 * min/max.  uyd888.cn Gemini page, chapter 1: 64 tokens share one
 * scale/zero-point.)
 *
 * Sequence b receives rows new_off[b] .. new_off[b+1]-1 of k_new / v_new
 * (fp16 bits, [N][H_kv][d]) at logical positions start_pos[b], start_pos[b]+1, ...
 *   KVQ_FP16        : the rows are copied.
 *   KVQ_INT8_TOKEN  : every (token, KV head) row of d values, K and V apart,
 *                     is quantized with its own (scale, zero).
 *   KVQ_INT8_GROUP64: every (64-token group aligned to logical position 64g,
 *                     KV head), K and V apart, shares one (scale, zero) over
 *                     the group's rows in this call; start_pos[b] must be a
 *                     multiple of 64 whenever sequence b receives rows, and the
 *                     rows must hold every token of each group they touch
 *                     (an open group is re-supplied whole and re-quantized).
 * Quantization arithmetic is IEEE fp32 with round-to-nearest-even, no fused
 * operations: range = max - min, scale = range / 255, inv = 1 / scale,
 * code = clamp(rint((x - zero) * inv), 0, 255).
 *
 * seqs->seq_lens is not read.  max_new (host) is an upper bound on the rows
 * of any one sequence; it sizes the grid.  Rows beyond it are not written.
 * Preconditions: new_off non-decreasing from 0; block-table entries of every
 * written page valid.
 */
kvq_status kvq_append_quant(const kvq_cache *cache, const kvq_seqs *seqs,
                            const int32_t *start_pos, const int32_t *new_off, int32_t max_new,
                            const uint16_t *k_new, const uint16_t *v_new, void *stream);

/*
 * kvq_append_decode -- the decode-time append: kvq_append_quant followed by
 * kvq_build_page_meta on exactly the pages the new rows land in, in one
 * kernel.  Each sequence's rows are its newest tokens: after the call the
 * sequence holds start_pos[b] + rows tokens, and page metadata covers the
 * valid tokens below that.  At most KVQ_DECODE_MAX_ROWS rows per sequence
 * (max_new larger: KVQ_ERR_UNSUPPORTED); INT8_GROUP64 rows re-supply the open
 * group from its aligned start, as in kvq_append_quant.  seqs->seq_lens is
 * not read; cache->page_meta is required.  Codes, scales, zero-points and
 * metadata are bit-identical to the two separate calls.
 */
#define KVQ_DECODE_MAX_ROWS 64
kvq_status kvq_append_decode(const kvq_cache *cache, const kvq_seqs *seqs,
                             const int32_t *start_pos, const int32_t *new_off, int32_t max_new,
                             const uint16_t *k_new, const uint16_t *v_new, void *stream);

/*
 * kvq_build_page_meta -- per (logical page j, KV head) of each sequence, for
 * page_begin[b] <= j < ceil(L_b/16): page_meta[block_table[b][j]][h] = the
 * per-channel min and max over the page's valid tokens (t < L_b) of the keys
 * as decoded ("TinyServe", section 2.1 direction-aware bounding box; section
 * 5.2 fp32 metadata).  Results are exact (min/max of fmaf-decoded values).
 * page_begin NULL means 0.  max_span (host, > 0) is the expected number of
 * pages per sequence and only sizes the grid; 0 means max_pages.
 */
kvq_status kvq_build_page_meta(const kvq_cache *cache, const kvq_seqs *seqs,
                               const int32_t *page_begin, int32_t max_span, void *stream);

/*
 * kvq_demote_pages -- a mixed-precision cache moves pages out of its FP16
 * pool ("TinyServe", section 6: high-importance pages stay FP16, the rest
 * are INT8; a page that is no longer important leaves FP16).  Item i moves
 * logical page page[i] of sequence seq[i] from its FP16-pool page to
 * INT8-pool page dst[i]: every valid token of the page (t < L_b) is quantized
 * per token from its fp16 rows, exactly as kvq_append_quant writes an INT8
 * page; the page's metadata is rebuilt from the new decoded keys (as
 * kvq_build_page_meta); and block_table[seq[i]][page[i]] becomes dst[i]
 * (the block table is written: seqs->block_table must point to writable
 * memory).  Slots at or past L_b are not written; the old FP16 page is left
 * as it was, for the caller to reuse.
 * seq, page, dst: [n] int32 device arrays.  Preconditions (not checked):
 * each item's page is below ceil(L_b / 16) and lives in the FP16 pool, each
 * dst lies in the INT8 pool, and no two items name the same page or the same
 * dst.  Only KVQ_MIXED_FP16_INT8 (else KVQ_ERR_UNSUPPORTED); n = 0 enqueues
 * nothing.
 */
kvq_status kvq_demote_pages(const kvq_cache *cache, const kvq_seqs *seqs, int32_t n, const int32_t *seq,
                            const int32_t *page, const int32_t *dst, void *stream);

/*
 * kvq_page_scores -- page relevance of every logical page ("TinyServe",
 * section 2.1): r(q, phi) = sum_i (q_i >= 0 ? q_i M_i : q_i m_i) with q the
 * unscaled fp16 query, summed in fp32.  The KV group's score is the max over
 * its G query heads.
 *   q      : [B][H_q][d] fp16 bits
 *   scores : [B][H_kv][max_pages] fp32 out; pages j >= ceil(L_b/16) get -inf.
 * Reads page_meta through the block table; page_meta must be current.
 */
kvq_status kvq_page_scores(const kvq_cache *cache, const kvq_seqs *seqs,
                           const uint16_t *q, int32_t num_q_heads, float *scores, void *stream);

/*
 * kvq_append_decode_scores -- kvq_append_decode followed by kvq_page_scores,
 * in one kernel (same arguments as the two calls).  For every sequence that
 * receives rows, seq_lens[b] must equal start_pos[b] + rows (the rows are its
 * newest tokens).  Codes, scale/zero, metadata and scores are bit-identical to
 * the two separate calls.
 */
kvq_status kvq_append_decode_scores(const kvq_cache *cache, const kvq_seqs *seqs,
                                    const int32_t *start_pos, const int32_t *new_off, int32_t max_new,
                                    const uint16_t *k_new, const uint16_t *v_new,
                                    const uint16_t *q, int32_t num_q_heads, float *scores, void *stream);

/*
 * Coarse-then-fine selection ("TinyServe", section 6: for large models,
 * screen coarsely first, then finely).  A super-page is group_pages
 * consecutive logical pages of a sequence (1 <= group_pages <= 64; pc_max =
 * ceil(max_pages / group_pages) super-pages per row).
 *
 * kvq_build_coarse_meta -- each super-page's box: the channel-wise min of its
 * valid pages' metadata minima and max of their maxima, exact (min/max of
 * page_meta, which must be current).  Written for super-pages
 * super_begin[b] <= jc < ceil(P_b / group_pages) (super_begin NULL: all);
 * max_span (host, >= 0), when super_begin is given, bounds how many of them
 * each sequence needs refreshed and only sizes the grid (0: all of them,
 * e.g. 1 + the pages a decode-time append touches / group_pages), as
 *   coarse_meta  [B * pc_max][H_kv][2][d] fp32 (the page_meta layout with
 *                "physical page" b * pc_max + jc),
 *   coarse_lens  [B] int32: 16 * ceil(P_b / group_pages), and
 *   coarse_table [B][pc_max] int32: b * pc_max + jc.
 * With these as a cache view (page_meta = coarse_meta, num_phys_pages =
 * B * pc_max) and a kvq_seqs view (max_pages = pc_max, seq_lens =
 * coarse_lens, block_table = coarse_table), kvq_page_scores gives the coarse
 * scores (each at least every member page's score) and kvq_topk_pages with
 * k_fixed = kc the kept super-pages.
 */
kvq_status kvq_build_coarse_meta(const kvq_cache *cache, const kvq_seqs *seqs, int32_t group_pages,
                                 const int32_t *super_begin, int32_t max_span, float *coarse_meta,
                                 int32_t *coarse_lens, int32_t *coarse_table, void *stream);

/*
 * kvq_page_scores_masked -- kvq_page_scores restricted to the kept
 * super-pages: for row (b, g), pages of the super-pages
 * sel_super[b][g][0 .. sel_super_count[b][g]) (ascending, as kvq_topk_pages
 * writes them; kc_cap is the row stride) get their page score, bit for bit
 * what kvq_page_scores writes, and every other page j < max_pages gets -inf.
 * Only the kept pages' metadata is read.
 */
kvq_status kvq_page_scores_masked(const kvq_cache *cache, const kvq_seqs *seqs, const uint16_t *q,
                                  int32_t num_q_heads, int32_t group_pages, const int32_t *sel_super,
                                  const int32_t *sel_super_count, int32_t kc_cap, float *scores, void *stream);

/*
 * kvq_topk_pages -- per (sequence b, KV head) row of `scores`, select K_b of
 * the P_b = ceil(L_b/16) pages ("TinyServe", section 3.1 phase 2; section 5.1
 * selection_ratio):
 *   K_b = min(P_b, k_fixed) if k_fixed > 0, else
 *   K_b = clamp(ceil(ratio_num * P_b / ratio_den), 1, P_b) in integers.
 * The K_b largest scores win; equal scores go to the lower logical page.
 * -0.0 and +0.0 compare equal.  Scores must not be NaN.
 *   sel_pages : [B][H_kv][k_cap] int32 out: selected logical pages, ascending,
 *               then -1 up to k_cap.
 *   sel_count : [B][H_kv] int32 out: K_b.
 * k_cap must be >= K for P = max_pages (else KVQ_ERR_INVALID_ARG), and
 * max_pages <= 12000 (else KVQ_ERR_UNSUPPORTED).
 */
kvq_status kvq_topk_pages(const float *scores, const kvq_seqs *seqs, int32_t num_kv_heads,
                          int32_t ratio_num, int32_t ratio_den, int32_t k_fixed, int32_t k_cap,
                          int32_t *sel_pages, int32_t *sel_count, void *stream);

/*
 * kvq_sparse_decode_attn -- single-token attention of every query head over
 * the valid tokens of the selected pages of its KV head ("TinyServe", section
 * 3.1 phases 3-4; intelliparadigm.com, section 2.1):
 *   out[b][h] = sum_t softmax_t(sm_scale * q.k_t) v_t
 * over t in the pages sel_pages[b][h/G][0 .. sel_count[b][h/G]) (logical page
 * ids, any order, no repeats), or over every page when sel_pages is NULL
 * (sel_count is then ignored).  Computed split-K: each split of
 * pages_per_split selected pages keeps an online (max, sum, acc) in fp32, and
 * a second kernel merges the splits with log-sum-exp weights (when no row
 * has more than one split, the split kernel writes out itself and no merge
 * runs; the output is the same bit for bit).  For a query
 * group (G = 2, 4, 8) over INT8 or 4-bit codes (a mixed cache's INT8 pages
 * included) the products run on the matrix cores:
 * q.k as fp16 x fp16 with fp32 accumulation, p.v with the weights split into
 * three bf16 parts (~2^-21 relative) against exact bf16 codes, fp32
 * accumulation.  A mixed cache's fp16 pages take the matrix cores too for a
 * query group: q.k as fp16 x fp16, p.v with the weights (times 2^7) split into
 * two fp16 parts against the fp16 values, fp32 accumulation.  A whole fp16
 * cache runs on the vector units.
 *   q   : [B][H_q][d] fp16 bits
 *   out : [B][H_q][d] fp32
 *   ws  : workspace of at least kvq_attn_workspace_bytes(...) bytes (the
 *         per-split partial results); ws_bytes is its size.  Calls that share
 *         a workspace must not overlap in time (one stream, or synchronized).
 * pages_per_split 0 picks a default; otherwise 1..4096.  k_cap is the row
 * stride of sel_pages and bounds sel_count (ignored when sel_pages is NULL).
 */
kvq_status kvq_sparse_decode_attn(const kvq_cache *cache, const kvq_seqs *seqs,
                                  const uint16_t *q, int32_t num_q_heads,
                                  const int32_t *sel_pages, const int32_t *sel_count, int32_t k_cap,
                                  float sm_scale, int32_t pages_per_split,
                                  float *out, void *ws, size_t ws_bytes, void *stream);

/*
 * kvq_select_decode_attn -- kvq_topk_pages and kvq_sparse_decode_attn in one
 * call: every attention block selects the top-K pages of its (sequence, KV
 * head) row from `scores` by exactly the rule of kvq_topk_pages and attends
 * to its share of them, so the selection costs no launch of its own.  out
 * equals, bit for bit, kvq_sparse_decode_attn over the selection
 * kvq_topk_pages makes from the same scores, with the same pages_per_split.
 *   scores    : [B][H_kv][max_pages] fp32 (as kvq_page_scores writes them)
 *   sel_pages : [B][H_kv][k_cap] int32 out, or NULL: the selection, as
 *               kvq_topk_pages writes it; sel_count [B][H_kv] out likewise
 *               (both NULL or both given).
 * k_cap must be >= K for P = max_pages (KVQ_ERR_INVALID_ARG); ws is sized by
 * kvq_attn_workspace_bytes(..., k_cap, pages_per_split).  max_pages <=
 * KVQ_SELECT_MAX_PAGES, and the block's LDS (pages_per_split * 4 bytes on top
 * of its fixed use) must fit the device (else KVQ_ERR_UNSUPPORTED); longer
 * rows take kvq_topk_pages and kvq_sparse_decode_attn.
 */
kvq_status kvq_select_decode_attn(const kvq_cache *cache, const kvq_seqs *seqs,
                                  const uint16_t *q, int32_t num_q_heads, const float *scores,
                                  int32_t ratio_num, int32_t ratio_den, int32_t k_fixed, int32_t k_cap,
                                  int32_t *sel_pages, int32_t *sel_count,
                                  float sm_scale, int32_t pages_per_split,
                                  float *out, void *ws, size_t ws_bytes, void *stream);

/*
 * kvq_decode_step -- the whole decode step in ONE persistent launch
 * ("TinyServe", section 3.1: score, top-K, sparse load and reduce fused into
 * one kernel; section 5.2: kernel-launch overhead): kvq_append_decode_scores
 * (append the newest rows, refresh the touched pages' metadata, score every
 * page) followed by kvq_select_decode_attn (top-K inside the attention,
 * split-K attention, split combine), with the same arguments.  Rows, their
 * scores and splits are items of one work list that the blocks of a grid of
 * resident blocks take in turn; a row's splits wait for its scores.
 *   - Codes, scale/zero, metadata, the selection (sel_pages/sel_count, if
 *     given), the scores of every page below ceil(L_b/16) and `out` equal,
 *     bit for bit, the two calls above with the same pages_per_split.
 *     scores past a row's pages are left unspecified (not -inf).
 *   - ws: at least kvq_step_workspace_bytes(...) bytes.  Its first
 *     kvq_step_counter_bytes(batch, num_kv_heads) bytes are counters that
 *     must be zero before the first call on this workspace (zero the buffer
 *     when allocating it); every call leaves them zero.  Calls sharing a
 *     workspace must not overlap in time.  The second 32-bit word of ws is
 *     set to 1, and stays 1, if a wait inside a launch ever ran out of its
 *     bound (the launch then still ends, with wrong results, and may leave
 *     counters set); a correct launch never does that.
 *   - Limits (else KVQ_ERR_UNSUPPORTED): max_pages <= KVQ_SELECT_MAX_PAGES,
 *     batch <= KVQ_STEP_MAX_SEQS, pages_per_split <= KVQ_STEP_MAX_SPLIT_PAGES,
 *     fp16 or INT8 storage.
 * max_new may be 0 (no rows appended; k_new / v_new may then be NULL).
 */
#define KVQ_STEP_MAX_SEQS 512
#define KVQ_STEP_MAX_SPLIT_PAGES 512
kvq_status kvq_decode_step(const kvq_cache *cache, const kvq_seqs *seqs,
                           const int32_t *start_pos, const int32_t *new_off, int32_t max_new,
                           const uint16_t *k_new, const uint16_t *v_new,
                           const uint16_t *q, int32_t num_q_heads, float *scores,
                           int32_t ratio_num, int32_t ratio_den, int32_t k_fixed, int32_t k_cap,
                           int32_t *sel_pages, int32_t *sel_count,
                           float sm_scale, int32_t pages_per_split,
                           float *out, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of kvq_decode_step (counters, then the per-split partials),
 * and the leading counter bytes that must start zero; 0 for invalid sizes. */
size_t kvq_step_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_pages, int32_t k_cap, int32_t pages_per_split);
size_t kvq_step_counter_bytes(int32_t batch, int32_t num_kv_heads);

/*
 * kvq_select_decode_attn_noalloc -- kvq_select_decode_attn without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The per-split partials go to a scratch array the library
 * holds in device memory, KVQ_NOALLOC_SCRATCH_BYTES per GPU it runs on, kept
 * until the process ends; its address is looked up on the first call on each
 * device (that device current).  The call allocates nothing and otherwise
 * behaves, and computes bit for bit, as kvq_select_decode_attn with the same
 * arguments.  Sizes whose kvq_attn_workspace_bytes(...) exceeds
 * KVQ_NOALLOC_SCRATCH_BYTES return KVQ_ERR_WORKSPACE before anything is
 * enqueued; a failed lookup returns KVQ_ERR_HIP.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialized by the caller.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_select_decode_attn_noalloc(const kvq_cache *cache, const kvq_seqs *seqs,
                                          const uint16_t *q, int32_t num_q_heads, const float *scores,
                                          int32_t ratio_num, int32_t ratio_den, int32_t k_fixed, int32_t k_cap,
                                          int32_t *sel_pages, int32_t *sel_count,
                                          float sm_scale, int32_t pages_per_split,
                                          float *out, void *stream);

/* Workspace bytes kvq_sparse_decode_attn needs for these sizes; k_cap 0
 * means every page (sel_pages NULL).  Returns 0 for invalid sizes. */
size_t kvq_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_pages, int32_t k_cap, int32_t pages_per_split);

/*
 * kvq_num_selected -- K for a row of P pages under the selection rule of
 * kvq_topk_pages ("TinyServe", section 5.1 selection_ratio): min(P, k_fixed)
 * if k_fixed > 0, else clamp(ceil(ratio_num * P / ratio_den), 1, P) in
 * integers; 0 for P <= 0.  A caller sizes sel_pages with it (k_cap =
 * kvq_num_selected(max_pages, ...)).  Host function, no device work.
 */
int32_t kvq_num_selected(int32_t num_pages, int32_t ratio_num, int32_t ratio_den, int32_t k_fixed);

/* The pages_per_split kvq_sparse_decode_attn uses when given 0. */
int32_t kvq_default_pages_per_split(int32_t batch, int32_t num_kv_heads, int32_t max_pages, int32_t k_cap);

/*
 * kvq_read_probe -- measurement helper, not a step of the method: reads
 * `bytes` of device memory at `buf` once with a plain streaming kernel (one
 * contiguous 64 KiB run per block, nontemporal 16-byte loads), so a caller
 * can time the bandwidth an HBM-bound kernel can reach on this GPU.
 * buf 16-byte aligned, bytes a multiple of 16 (else KVQ_ERR_INVALID_ARG);
 * sink is one device uint32 the kernel may write (in practice never does).
 */
kvq_status kvq_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Static description of a status code (never NULL). */
const char *kvq_status_string(kvq_status status);

/* KVQ_ABI_VERSION of the built library. */
int32_t kvq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
