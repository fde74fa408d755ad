// kvq_api.hip -- the extern "C" entry points of libkvq: argument validation,
// workspace sizing and launches on the caller's stream.  No allocation, no
// synchronization, no state between calls.
#include <hip/hip_runtime.h>

#include "../../include/kvq.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

kvq_status check_cache(const kvq_cache* c, bool need_meta) {
  if (!c) return KVQ_ERR_INVALID_ARG;
  if (c->page_size != KVQ_PAGE_SIZE) return KVQ_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (c->format < KVQ_FP16 || c->format > KVQ_MIXED_FP16_INT8) return KVQ_ERR_UNSUPPORTED;
  if ((c->format == KVQ_INT4_TOKEN || c->format == KVQ_INT4_GROUP64) && c->head_dim != 128)
    return KVQ_ERR_UNSUPPORTED;
  if (c->num_kv_heads < 1 || c->num_kv_heads > 65535 || c->num_phys_pages < 1) return KVQ_ERR_INVALID_ARG;
  if (c->format == KVQ_MIXED_FP16_INT8 && (c->num_fp16_pages < 0 || c->num_fp16_pages > c->num_phys_pages))
    return KVQ_ERR_INVALID_ARG;
  if (!c->k_pages || !c->v_pages || !aligned16(c->k_pages) || !aligned16(c->v_pages)) return KVQ_ERR_INVALID_ARG;
  if (c->format != KVQ_FP16 && (!c->kv_params || !aligned16(c->kv_params))) return KVQ_ERR_INVALID_ARG;
  if (need_meta && (!c->page_meta || !aligned16(c->page_meta))) return KVQ_ERR_INVALID_ARG;
  return KVQ_OK;
}

kvq_status check_seqs(const kvq_seqs* s) {
  if (!s || !s->seq_lens || !s->block_table) return KVQ_ERR_INVALID_ARG;
  if (s->batch < 1 || s->batch > 65535 || s->max_pages < 1) return KVQ_ERR_INVALID_ARG;
  return KVQ_OK;
}

kvq_status check_heads(const kvq_cache* c, int32_t num_q_heads) {
  if (num_q_heads < 1 || num_q_heads % c->num_kv_heads != 0) return KVQ_ERR_INVALID_ARG;
  const int G = num_q_heads / c->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

kvq_status from_hip(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

int32_t splits_for(int32_t max_pages, int32_t k_cap, int32_t pps) {
  const int32_t cap = k_cap > 0 ? k_cap : max_pages;
  return (cap + pps - 1) / pps;
}

// Validation and launch shared by kvq_select_decode_attn and its variant
// without a workspace argument (ws NULL there: the library's scratch).
kvq_status select_decode_attn(const kvq_cache* cache, const kvq_seqs* seqs, const uint16_t* q, int32_t num_q_heads,
                              const float* scores, int32_t ratio_num, int32_t ratio_den, int32_t k_fixed,
                              int32_t k_cap, int32_t* sel_pages, int32_t* sel_count, float sm_scale,
                              int32_t pages_per_split, float* out, void* ws, size_t ws_bytes, bool scratch,
                              void* stream) {
  kvq_status st = check_cache(cache, false);
  if (st != KVQ_OK) return st;
  if ((st = check_seqs(seqs)) != KVQ_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != KVQ_OK) return st;
  if (!q || !out || !scores || !aligned16(q)) return KVQ_ERR_INVALID_ARG;
  if (k_fixed < 0 || (k_fixed == 0 && (ratio_num < 1 || ratio_den < 1))) return KVQ_ERR_INVALID_ARG;
  if ((sel_pages == nullptr) != (sel_count == nullptr)) return KVQ_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale)) return KVQ_ERR_INVALID_ARG;
  if (pages_per_split < 0 || pages_per_split > 4096) return KVQ_ERR_INVALID_ARG;
  if (seqs->max_pages > kvq::kSelMaxPages) return KVQ_ERR_UNSUPPORTED;
  if (k_cap < kvq::num_selected(seqs->max_pages, ratio_num, ratio_den, k_fixed)) return KVQ_ERR_INVALID_ARG;
  const int32_t pps = pages_per_split ? pages_per_split
                                      : kvq_default_pages_per_split(seqs->batch, cache->num_kv_heads,
                                                                    seqs->max_pages, k_cap);
  const int32_t max_splits = splits_for(seqs->max_pages, k_cap, pps);
  const size_t need = kvq_attn_workspace_bytes(seqs->batch, num_q_heads, cache->head_dim, seqs->max_pages, k_cap,
                                               pps);
  if (scratch) {
    if (need == 0 || need > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
    const hipError_t e = kvq::noalloc_scratch(&ws);
    if (e != hipSuccess || !ws) return KVQ_ERR_HIP;
  } else if (!ws || ws_bytes < need || !aligned16(ws)) {
    return KVQ_ERR_WORKSPACE;
  }
  const kvq::InKernelSelect ks{scores, ratio_num, ratio_den, k_fixed, sel_pages, sel_count};
  const hipError_t e = kvq::launch_decode_attn(*cache, *seqs, q, num_q_heads, nullptr, nullptr, &ks, k_cap, sm_scale,
                                               pps, max_splits, out, ws, (hipStream_t)stream);
  if (e == hipErrorInvalidConfiguration) return KVQ_ERR_UNSUPPORTED;  // LDS of this row length and split
  return from_hip(e);
}


}  // namespace

extern "C" {

kvq_status kvq_append_quant(const kvq_cache* cache, const kvq_seqs* seqs, const int32_t* start_pos,
                            const int32_t* new_off, int32_t max_new, const uint16_t* k_new,
                            const uint16_t* v_new, void* stream) {
  kvq_status st = check_cache(cache, false);
  if (st != KVQ_OK) return st;
  if (!seqs || !seqs->block_table || seqs->batch < 1 || seqs->batch > 65535 || seqs->max_pages < 1)
    return KVQ_ERR_INVALID_ARG;
  if (!start_pos || !new_off || max_new < 0) return KVQ_ERR_INVALID_ARG;
  if (max_new > 0 && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))) return KVQ_ERR_INVALID_ARG;
  if ((long long)max_new * cache->num_kv_heads > 0x7FFFFFFFLL) return KVQ_ERR_UNSUPPORTED;
  return from_hip(kvq::launch_append(*cache, *seqs, start_pos, new_off, max_new, k_new, v_new,
                                     (hipStream_t)stream));
}

kvq_status kvq_append_decode(const kvq_cache* cache, const kvq_seqs* seqs, const int32_t* start_pos,
                             const int32_t* new_off, int32_t max_new, const uint16_t* k_new,
                             const uint16_t* v_new, void* stream) {
  kvq_status st = check_cache(cache, true);
  if (st != KVQ_OK) return st;
  if (!seqs || !seqs->block_table || seqs->batch < 1 || seqs->batch > 65535 || seqs->max_pages < 1)
    return KVQ_ERR_INVALID_ARG;
  if (!start_pos || !new_off || max_new < 0) return KVQ_ERR_INVALID_ARG;
  if (max_new > KVQ_DECODE_MAX_ROWS) return KVQ_ERR_UNSUPPORTED;
  if (max_new == 0) return KVQ_OK;
  if (!k_new || !v_new) return KVQ_ERR_INVALID_ARG;
  if (cache->num_kv_heads > 65535) return KVQ_ERR_UNSUPPORTED;
  return from_hip(kvq::launch_append_decode(*cache, *seqs, start_pos, new_off, k_new, v_new, (hipStream_t)stream));
}

kvq_status kvq_append_decode_scores(const kvq_cache* cache, const kvq_seqs* seqs, const int32_t* start_pos,
                                    const int32_t* new_off, int32_t max_new, const uint16_t* k_new,
                                    const uint16_t* v_new, const uint16_t* q, int32_t num_q_heads, float* scores,
                                    void* stream) {
  kvq_status st = check_cache(cache, true);
  if (st != KVQ_OK) return st;
  if ((st = check_seqs(seqs)) != KVQ_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != KVQ_OK) return st;
  if (!q || !scores || !aligned16(q)) return KVQ_ERR_INVALID_ARG;
  if (!start_pos || !new_off || max_new < 0) return KVQ_ERR_INVALID_ARG;
  if (max_new > KVQ_DECODE_MAX_ROWS) return KVQ_ERR_UNSUPPORTED;
  if (max_new > 0 && (!k_new || !v_new)) return KVQ_ERR_INVALID_ARG;
  return from_hip(kvq::launch_append_scores(*cache, *seqs, start_pos, new_off, k_new, v_new, q, num_q_heads, scores,
                                            (hipStream_t)stream));
}

kvq_status kvq_build_page_meta(const kvq_cache* cache, const kvq_seqs* seqs, const int32_t* page_begin,
                               int32_t max_span, void* stream) {
  kvq_status st = check_cache(cache, true);
  if (st != KVQ_OK) return st;
  if ((st = check_seqs(seqs)) != KVQ_OK) return st;
  if (max_span < 0) return KVQ_ERR_INVALID_ARG;
  return from_hip(kvq::launch_page_meta(*cache, *seqs, page_begin, max_span, (hipStream_t)stream));
}

kvq_status kvq_demote_pages(const kvq_cache* cache, const kvq_seqs* seqs, int32_t n, const int32_t* seq,
                            const int32_t* page, const int32_t* dst, void* stream) {
  kvq_status st = check_cache(cache, true);
  if (st != KVQ_OK) return st;
  if ((st = check_seqs(seqs)) != KVQ_OK) return st;
  if (cache->format != KVQ_MIXED_FP16_INT8) return KVQ_ERR_UNSUPPORTED;
  if (n < 0) return KVQ_ERR_INVALID_ARG;
  if (n == 0) return KVQ_OK;
  if (!seq || !page || !dst) return KVQ_ERR_INVALID_ARG;
  return from_hip(kvq::launch_demote(*cache, *seqs, n, seq, page, dst, (hipStream_t)stream));
}

kvq_status kvq_page_scores(const kvq_cache* cache, const kvq_seqs* seqs, const uint16_t* q,
                           int32_t num_q_heads, float* scores, void* stream) {
  kvq_status st = check_cache(cache, true);
  if (st != KVQ_OK) return st;
  if ((st = check_seqs(seqs)) != KVQ_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != KVQ_OK) return st;
  if (!q || !scores || !aligned16(q)) return KVQ_ERR_INVALID_ARG;
  return from_hip(kvq::launch_page_scores(*cache, *seqs, q, num_q_heads, scores, (hipStream_t)stream));
}

kvq_status kvq_build_coarse_meta(const kvq_cache* cache, const kvq_seqs* seqs, int32_t group_pages,
                                 const int32_t* super_begin, int32_t max_span, float* coarse_meta,
                                 int32_t* coarse_lens, int32_t* coarse_table, void* stream) {
  kvq_status st = check_cache(cache, true);
  if (st != KVQ_OK) return st;
  if ((st = check_seqs(seqs)) != KVQ_OK) return st;
  if (group_pages < 1 || group_pages > 64 || max_span < 0) return KVQ_ERR_INVALID_ARG;
  if (!coarse_meta || !coarse_lens || !coarse_table || !aligned16(coarse_meta)) return KVQ_ERR_INVALID_ARG;
  if ((long long)seqs->batch * ((seqs->max_pages + group_pages - 1) / group_pages) > 0x7FFFFFFFLL)
    return KVQ_ERR_UNSUPPORTED;
  return from_hip(kvq::launch_coarse_meta(*cache, *seqs, group_pages, super_begin, max_span, coarse_meta,
                                          coarse_lens, coarse_table, (hipStream_t)stream));
}

kvq_status kvq_page_scores_masked(const kvq_cache* cache, const kvq_seqs* seqs, const uint16_t* q,
                                  int32_t num_q_heads, int32_t group_pages, const int32_t* sel_super,
                                  const int32_t* sel_super_count, int32_t kc_cap, float* scores, void* stream) {
  kvq_status st = check_cache(cache, true);
  if (st != KVQ_OK) return st;
  if ((st = check_seqs(seqs)) != KVQ_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != KVQ_OK) return st;
  if (!q || !scores || !sel_super || !sel_super_count || !aligned16(q)) return KVQ_ERR_INVALID_ARG;
  if (group_pages < 1 || group_pages > 64 || kc_cap < 1) return KVQ_ERR_INVALID_ARG;
  if ((long long)seqs->batch * cache->num_kv_heads * kc_cap > 0x7FFFFFFFLL) return KVQ_ERR_UNSUPPORTED;
  return from_hip(kvq::launch_page_scores_masked(*cache, *seqs, q, num_q_heads, group_pages, sel_super,
                                                 sel_super_count, kc_cap, scores, (hipStream_t)stream));
}

kvq_status kvq_topk_pages(const float* scores, const kvq_seqs* seqs, int32_t num_kv_heads, int32_t ratio_num,
                          int32_t ratio_den, int32_t k_fixed, int32_t k_cap, int32_t* sel_pages,
                          int32_t* sel_count, void* stream) {
  kvq_status st = check_seqs(seqs);
  if (st != KVQ_OK) return st;
  if (!scores || !sel_pages || !sel_count || num_kv_heads < 1) return KVQ_ERR_INVALID_ARG;
  if (k_fixed < 0 || (k_fixed == 0 && (ratio_num < 1 || ratio_den < 1))) return KVQ_ERR_INVALID_ARG;
  if ((long long)seqs->batch * num_kv_heads > 0x7FFFFFFFLL) return KVQ_ERR_INVALID_ARG;
  if (seqs->max_pages > kvq::kTopkMaxPages) return KVQ_ERR_UNSUPPORTED;
  if (k_cap < kvq::num_selected(seqs->max_pages, ratio_num, ratio_den, k_fixed)) return KVQ_ERR_INVALID_ARG;
  return from_hip(kvq::launch_topk(scores, *seqs, num_kv_heads, ratio_num, ratio_den, k_fixed, k_cap,
                                   sel_pages, sel_count, (hipStream_t)stream));
}

size_t kvq_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t max_pages,
                                int32_t k_cap, int32_t pages_per_split) {
  if (batch < 1 || num_q_heads < 1 || head_dim < 1 || max_pages < 1 || k_cap < 0 || pages_per_split < 1)
    return 0;
  const size_t splits = (size_t)splits_for(max_pages, k_cap, pages_per_split);
  return (size_t)batch * num_q_heads * splits * ((size_t)head_dim + 2) * sizeof(float);
}

int32_t kvq_num_selected(int32_t num_pages, int32_t ratio_num, int32_t ratio_den, int32_t k_fixed) {
  if (k_fixed <= 0 && (ratio_num < 1 || ratio_den < 1)) return num_pages > 0 ? 1 : 0;
  return kvq::num_selected(num_pages, ratio_num, ratio_den, k_fixed);
}

int32_t kvq_default_pages_per_split(int32_t batch, int32_t num_kv_heads, int32_t max_pages, int32_t k_cap) {
  // Few, long splits: each block streams its pages with the next tile in
  // flight, and every split adds a partial to merge.  Aim for about two
  // blocks per CU (512 on 256 CUs), 24..128 pages each (measured: 40 pages
  // at 32K x 32 heads; 96-128 beat 64 and 192 on 64 ragged GQA sequences;
  // 16 x 308 selected pages at 16K: 24 pages per split beat 12, 16, 32, 48).
  const long long cap = k_cap > 0 ? k_cap : max_pages;
  const long long total = (long long)batch * num_kv_heads * cap;
  long long pps = (total + 511) / 512;
  if (pps < 24) pps = 24;
  if (pps > 128) pps = 128;
  return (int32_t)((pps + 3) / 4 * 4);
}

kvq_status kvq_sparse_decode_attn(const kvq_cache* cache, const kvq_seqs* seqs, const uint16_t* q,
                                  int32_t num_q_heads, const int32_t* sel_pages, const int32_t* sel_count,
                                  int32_t k_cap, float sm_scale, int32_t pages_per_split, float* out, void* ws,
                                  size_t ws_bytes, void* stream) {
  kvq_status st = check_cache(cache, false);
  if (st != KVQ_OK) return st;
  if ((st = check_seqs(seqs)) != KVQ_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != KVQ_OK) return st;
  if (!q || !out || !aligned16(q)) return KVQ_ERR_INVALID_ARG;
  if (sel_pages && (!sel_count || k_cap < 1)) return KVQ_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale)) return KVQ_ERR_INVALID_ARG;
  if (pages_per_split < 0 || pages_per_split > 4096) return KVQ_ERR_INVALID_ARG;
  const int32_t cap = sel_pages ? k_cap : 0;
  const int32_t pps = pages_per_split ? pages_per_split
                                      : kvq_default_pages_per_split(seqs->batch, cache->num_kv_heads,
                                                                    seqs->max_pages, cap);
  const int32_t max_splits = splits_for(seqs->max_pages, cap, pps);
  const size_t need = kvq_attn_workspace_bytes(seqs->batch, num_q_heads, cache->head_dim, seqs->max_pages, cap, pps);
  if (!ws || ws_bytes < need || !aligned16(ws)) return KVQ_ERR_WORKSPACE;
  return from_hip(kvq::launch_decode_attn(*cache, *seqs, q, num_q_heads, sel_pages, sel_count, nullptr, k_cap,
                                          sm_scale, pps,
                                          max_splits, out, ws, (hipStream_t)stream));
}

kvq_status kvq_select_decode_attn(const kvq_cache* cache, const kvq_seqs* seqs, const uint16_t* q,
                                  int32_t num_q_heads, const float* scores, int32_t ratio_num, int32_t ratio_den,
                                  int32_t k_fixed, int32_t k_cap, int32_t* sel_pages, int32_t* sel_count,
                                  float sm_scale, int32_t pages_per_split, float* out, void* ws, size_t ws_bytes,
                                  void* stream) {
  return select_decode_attn(cache, seqs, q, num_q_heads, scores, ratio_num, ratio_den, k_fixed, k_cap, sel_pages,
                            sel_count, sm_scale, pages_per_split, out, ws, ws_bytes, false, stream);
}

kvq_status kvq_select_decode_attn_noalloc(const kvq_cache* cache, const kvq_seqs* seqs, const uint16_t* q,
                                          int32_t num_q_heads, const float* scores, int32_t ratio_num,
                                          int32_t ratio_den, int32_t k_fixed, int32_t k_cap, int32_t* sel_pages,
                                          int32_t* sel_count, float sm_scale, int32_t pages_per_split, float* out,
                                          void* stream) {
  return select_decode_attn(cache, seqs, q, num_q_heads, scores, ratio_num, ratio_den, k_fixed, k_cap, sel_pages,
                            sel_count, sm_scale, pages_per_split, out, nullptr, 0, true, stream);
}

size_t kvq_step_counter_bytes(int32_t batch, int32_t num_kv_heads) {
  if (batch < 1 || num_kv_heads < 1 || (long long)batch * num_kv_heads > (1LL << 24)) return 0;
  return kvq::step_counter_bytes(batch, batch * num_kv_heads);
}

size_t kvq_step_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_pages, int32_t k_cap, int32_t pages_per_split) {
  const size_t ctr = kvq_step_counter_bytes(batch, num_kv_heads);
  const size_t part = kvq_attn_workspace_bytes(batch, num_q_heads, head_dim, max_pages, k_cap, pages_per_split);
  if (ctr == 0 || part == 0) return 0;
  return ctr + part;
}

kvq_status kvq_decode_step(const kvq_cache* cache, const kvq_seqs* seqs, const int32_t* start_pos,
                           const int32_t* new_off, int32_t max_new, const uint16_t* k_new, const uint16_t* v_new,
                           const uint16_t* q, int32_t num_q_heads, float* scores, int32_t ratio_num,
                           int32_t ratio_den, int32_t k_fixed, int32_t k_cap, int32_t* sel_pages,
                           int32_t* sel_count, float sm_scale, int32_t pages_per_split, float* out, void* ws,
                           size_t ws_bytes, void* stream) {
  kvq_status st = check_cache(cache, true);
  if (st != KVQ_OK) return st;
  if ((st = check_seqs(seqs)) != KVQ_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != KVQ_OK) return st;
  if (!q || !out || !scores || !aligned16(q)) return KVQ_ERR_INVALID_ARG;
  if (!start_pos || !new_off || max_new < 0) return KVQ_ERR_INVALID_ARG;
  if (max_new > KVQ_DECODE_MAX_ROWS) return KVQ_ERR_UNSUPPORTED;
  if (max_new > 0 && (!k_new || !v_new)) return KVQ_ERR_INVALID_ARG;
  if (k_fixed < 0 || (k_fixed == 0 && (ratio_num < 1 || ratio_den < 1))) return KVQ_ERR_INVALID_ARG;
  if ((sel_pages == nullptr) != (sel_count == nullptr)) return KVQ_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale)) return KVQ_ERR_INVALID_ARG;
  if (pages_per_split < 0 || pages_per_split > 4096) return KVQ_ERR_INVALID_ARG;
  if (seqs->max_pages > kvq::kSelMaxPages || seqs->batch > kvq::kStepMaxSeqs) return KVQ_ERR_UNSUPPORTED;
  if (cache->format != KVQ_FP16 && cache->format != KVQ_INT8_TOKEN && cache->format != KVQ_INT8_GROUP64)
    return KVQ_ERR_UNSUPPORTED;
  if (k_cap < kvq::num_selected(seqs->max_pages, ratio_num, ratio_den, k_fixed)) return KVQ_ERR_INVALID_ARG;
  const int32_t pps = pages_per_split ? pages_per_split
                                      : kvq_default_pages_per_split(seqs->batch, cache->num_kv_heads,
                                                                    seqs->max_pages, k_cap);
  if (pps > kvq::kStepMaxSplitPages) return KVQ_ERR_UNSUPPORTED;
  const int32_t max_splits = splits_for(seqs->max_pages, k_cap, pps);
  const size_t need = kvq_step_workspace_bytes(seqs->batch, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                               seqs->max_pages, k_cap, pps);
  if (!ws || need == 0 || ws_bytes < need || !aligned16(ws)) return KVQ_ERR_WORKSPACE;
  const hipError_t e = kvq::launch_decode_step(*cache, *seqs, start_pos, new_off, k_new, v_new, q, num_q_heads,
                                               scores, ratio_num, ratio_den, k_fixed, k_cap, sel_pages, sel_count,
                                               sm_scale, pps, max_splits, out, ws, (hipStream_t)stream);
  if (e == hipErrorInvalidConfiguration) return KVQ_ERR_UNSUPPORTED;
  return from_hip(e);
}

kvq_status kvq_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || !aligned16(buf) || bytes % 16 != 0) return KVQ_ERR_INVALID_ARG;
  return from_hip(kvq::launch_read_probe(buf, bytes, sink, (hipStream_t)stream));
}

const char* kvq_status_string(kvq_status status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

}  // extern "C"
