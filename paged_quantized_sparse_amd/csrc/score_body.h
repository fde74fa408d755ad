// score_body.h -- the wave-level page scorer shared by page_scores.hip and the
// fused append + scores kernel.
//
// Page relevance ("TinyServe", lpnh.cn, section 2.1):
//   r(q, phi_j) = sum_i (q_i >= 0 ? q_i M_j[i] : q_i m_j[i]),
// which never underestimates q.k for any key of page j; written as
// sum_i max(q_i, 0) M_j[i] + min(q_i, 0) m_j[i], the same terms without a
// per-channel select.  For GQA the KV group's score is the max over its query
// heads, so it still bounds every member head's q.k.
//
// Layout per (physical page, KV head): meta[2][d] fp32 (min row, max row) =
// 8d bytes, read as one contiguous wave load: lanes 0-31 hold min-row
// channels, lanes 32-63 the max-row channels.  The query stays in registers.
#pragma once

#include "kvq_device.h"

namespace kvq {

// Scoring kernels run at 8 waves per SIMD (at most 64 VGPRs), so a launch of
// 256 CUs x 8 blocks streams the metadata in a single round of blocks.
#define KVQ_SCORE_OCC_ATTR __attribute__((amdgpu_waves_per_eu(8, 8)))

constexpr int kScoreWaves = 4;
constexpr int kScorePagesPerWave = 8;

struct ScoreView {
  const float* meta;
  const int32_t* block_table;
  const uint16_t* q;
  float* scores;
  int H;
  int Hq;
  int max_pages;
};

// This lane's query coefficients: max(q, 0) on the max row, min(q, 0) on the min row.
template <int D, int G>
struct ScoreQuery {
  static constexpr int E = 2 * D / 64;  // floats per lane (4 for d = 128, 2 for d = 64)
  float qc[G][E];
  __device__ __forceinline__ void load(const ScoreView& a, int b, int g) {
    const int lane = lane_id();
    const bool max_row = lane >= 32;
    const int ch0 = (lane & 31) * E;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint16_t* qh = a.q + ((size_t)b * a.Hq + g * G + hh) * D + ch0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float x = half_bits_to_float(qh[e]);
        qc[hh][e] = max_row ? fmaxf(x, 0.0f) : fminf(x, 0.0f);
      }
    }
  }
};

// Score of one page from this lane's E metadata values: per head, an fma
// chain over the lane's values, a 64-lane sum, then the max over the G heads.
template <int D, int G>
__device__ __forceinline__ float score_from_values(const ScoreQuery<D, G>& q, const float* vals) {
  constexpr int E = ScoreQuery<D, G>::E;
  float best = -INFINITY;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float r = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) r = __builtin_fmaf(q.qc[hh][e], vals[e], r);
    r = sum_contig<64>(r);
    best = fmaxf(best, r);
  }
  return best;
}

// Block-table entries of pages j0 .. j0+7 of sequence b in one vector load:
// lane k (mod 8) holds page j0 + k's entry (the index clamped into the row).
__device__ __forceinline__ int score_table_load(const ScoreView& a, int b, int j0) {
  const int j = min(max(j0 + (lane_id() & 7), 0), a.max_pages - 1);
  return a.block_table[(size_t)b * a.max_pages + j];
}

// The calling wave scores pages j0 .. j0+7 of row (b, g), given their table
// entries bt_v from score_table_load: pages below min(P, skip_from) get their
// score, pages at or past P (and below max_pages) get -inf, pages in
// [skip_from, P) are left to another writer.  P and skip_from come from
// `bounds(P, skip_from)`, called only here, so the caller's loads of them and
// the table load are in flight together.  A page that is not scored reads
// physical page 0's metadata instead of its own, so every load is
// unconditional.  All loads are issued before any page is reduced.
template <int D, int G, typename Bounds>
__device__ __forceinline__ void score_pages(const ScoreView& a, const ScoreQuery<D, G>& q, int b, int g, int j0,
                                            int bt_v, Bounds bounds) {
  constexpr int E = ScoreQuery<D, G>::E;
  const int lane = lane_id();
  float* out = a.scores + ((size_t)b * a.H + g) * a.max_pages;
  __builtin_amdgcn_sched_barrier(0);
  int P, skip_from;
  bounds(P, skip_from);
  const int live = min(P, skip_from);
  float vals[kScorePagesPerWave][E];
#pragma unroll
  for (int k = 0; k < kScorePagesPerWave; ++k) {
    const int ph = j0 + k < live ? __builtin_amdgcn_readlane(bt_v, k) : 0;
    const float* m = a.meta + ((size_t)ph * a.H + g) * 2 * D + lane * E;
    if constexpr (E == 4) {
      const float4 v = *(const float4*)m;
      vals[k][0] = v.x; vals[k][1] = v.y; vals[k][2] = v.z; vals[k][3] = v.w;
    } else {
      const float2 v = *(const float2*)m;
      vals[k][0] = v.x; vals[k][1] = v.y;
    }
  }
#pragma unroll
  for (int k = 0; k < kScorePagesPerWave; ++k) {
    const int j = j0 + k;
    if (j >= a.max_pages) break;
    if (j >= live && j < P) continue;
    const float best = j < live ? score_from_values<D, G>(q, vals[k]) : -INFINITY;
    if (lane == 0) out[j] = best;
  }
}

}  // namespace kvq
