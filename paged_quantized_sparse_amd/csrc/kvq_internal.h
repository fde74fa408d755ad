// kvq_internal.h -- launchers behind the C ABI of libkvq (host side).
// Each launcher assumes its arguments were validated by kvq_api.hip and
// returns the HIP error of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "../../include/kvq.h"

namespace kvq {

// A host-side lookup of a device property (occupancy, LDS room) memoized per
// device: computed on the first launch on each device (the current one) and
// reused after.  `memo` starts zeroed and holds value + 1; concurrent first
// calls compute the same value, so the race is benign.
constexpr int kMaxDevices = 64;
template <class F>
long long per_device(std::atomic<long long> (&memo)[kMaxDevices], F compute) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return compute();
  long long v = memo[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    v = compute() + 1;
    memo[dev].store(v, std::memory_order_relaxed);
  }
  return v - 1;
}

// The FP16 pool size of a mixed-precision cache (its physical pages below
// this are FP16); 0 for every other format.
inline int fp16_pool(const kvq_cache& c) { return c.format == KVQ_MIXED_FP16_INT8 ? c.num_fp16_pages : 0; }

hipError_t launch_append(const kvq_cache& c, const kvq_seqs& s, const int32_t* start_pos,
                         const int32_t* new_off, int max_new, const uint16_t* k_new,
                         const uint16_t* v_new, hipStream_t st);
hipError_t launch_demote(const kvq_cache& c, const kvq_seqs& s, int n, const int32_t* seq, const int32_t* page,
                         const int32_t* dst, hipStream_t st);

hipError_t launch_append_decode(const kvq_cache& c, const kvq_seqs& s, const int32_t* start_pos,
                                const int32_t* new_off, const uint16_t* k_new, const uint16_t* v_new,
                                hipStream_t st);

hipError_t launch_append_scores(const kvq_cache& c, const kvq_seqs& s, const int32_t* start_pos,
                                const int32_t* new_off, const uint16_t* k_new, const uint16_t* v_new,
                                const uint16_t* q, int num_q_heads, float* scores, hipStream_t st);

hipError_t launch_page_meta(const kvq_cache& c, const kvq_seqs& s, const int32_t* page_begin,
                            int max_span, hipStream_t st);

hipError_t launch_page_scores(const kvq_cache& c, const kvq_seqs& s, const uint16_t* q, int num_q_heads,
                              float* scores, hipStream_t st);

constexpr int kTopkMaxPages = 12000;  // keys in LDS beside 16.9 KB of histograms, within 64 KB
hipError_t launch_topk(const float* scores, const kvq_seqs& s, int num_kv_heads, int rnum, int rden,
                       int k_fixed, int k_cap, int32_t* sel_pages, int32_t* sel_count, hipStream_t st);

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);

// Longest row (pages) the attention kernel selects in itself: each of its
// 256 threads holds the keys of 8 consecutive pages in registers.  (More keys
// per thread would cost registers, and unrolled code that every launch
// fetches again, for all rows.)
constexpr int kSelMaxPages = KVQ_SELECT_MAX_PAGES;

// Selection done inside the attention kernel: the scores, the rule, and
// optional copies of the selection (NULL: not wanted).
struct InKernelSelect {
  const float* scores;
  int rnum, rden, k_fixed;
  int32_t* sel_out;
  int32_t* cnt_out;
};

// Coarse-then-fine selection (hier_select.hip).
hipError_t launch_coarse_meta(const kvq_cache& c, const kvq_seqs& s, int group, const int32_t* super_begin,
                              int max_span, float* coarse, int32_t* coarse_lens, int32_t* coarse_table,
                              hipStream_t st);
hipError_t launch_page_scores_masked(const kvq_cache& c, const kvq_seqs& s, const uint16_t* q, int num_q_heads,
                                     int group, const int32_t* sel_super, const int32_t* sel_count, int kc_cap,
                                     float* scores, hipStream_t st);

// The fused decode step (decode_step.hip): rows of at most kSelMaxPages
// pages, at most kStepMaxSeqs sequences, splits of at most kStepMaxSplitPages.
constexpr int kStepMaxSeqs = KVQ_STEP_MAX_SEQS;
constexpr int kStepMaxSplitPages = KVQ_STEP_MAX_SPLIT_PAGES;
// bytes of the step's counters at the start of its workspace (the partials follow)
size_t step_counter_bytes(int batch, int rows);
hipError_t launch_decode_step(const kvq_cache& c, const kvq_seqs& s, const int32_t* start_pos,
                              const int32_t* new_off, const uint16_t* k_new, const uint16_t* v_new,
                              const uint16_t* q, int num_q_heads, float* scores, int rnum, int rden, int k_fixed,
                              int k_cap, int32_t* sel_pages, int32_t* sel_count, float sm_scale,
                              int pages_per_split, int max_splits, float* out, void* ws, hipStream_t st);

// The device address of the library's scratch array on the current device
// (looked up on the first call per device; KVQ_NOALLOC_SCRATCH_BYTES long).
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_decode_attn(const kvq_cache& c, const kvq_seqs& s, const uint16_t* q, int num_q_heads,
                              const int32_t* sel_pages, const int32_t* sel_count, const InKernelSelect* ks,
                              int k_cap, float sm_scale,
                              int pages_per_split, int max_splits, float* out, void* ws, hipStream_t st);

}  // namespace kvq
