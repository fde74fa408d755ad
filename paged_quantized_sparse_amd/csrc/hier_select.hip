// hier_select.hip -- the coarse-then-fine page selection ("TinyServe",
// lpnh.cn, section 6: for large models, screen coarsely first, then finely).
//
// A super-page is `group` consecutive logical pages of a sequence.  Its box
// is the channel-wise min of the member pages' minima and max of their maxima
// (coarse_meta_kernel), laid out like page metadata with "physical page"
// b * pc_max + jc, so kvq_page_scores and kvq_topk_pages on that view are the
// coarse screen.  The box contains every member page's box, so the coarse
// score is at least every member page's score.  page_scores_masked_kernel
// then scores only the pages of the kept super-pages and writes -inf for all
// others, and the usual top-K (kvq_topk_pages or the in-kernel selection)
// finishes the selection.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "score_body.h"

namespace kvq {
namespace {

struct CoarseArgs {
  const float* meta;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* super_begin;  // [B] or NULL
  int from_begin;              // 1: the grid covers super-pages from super_begin[b] on
  float* coarse;               // [B * pc_max][H][2][D]
  int32_t* coarse_lens;        // [B]: 16 * super-pages of the sequence
  int32_t* coarse_table;       // [B][pc_max]: b * pc_max + jc
  int H, max_pages, group, pc_max, B;
};

// One wave per (super-page slot jc, KV head, sequence): lanes 0-31 hold
// min-row channels and lanes 32-63 max-row channels, E each, as the scorer
// reads a page's metadata; the wave folds the member pages' rows with min
// (lanes < 32) or max.  Grid (ceil(span / 4), H, B), 4 waves per block; the
// slots start at 0, or at super_begin[b] when the grid covers only the
// super-pages from there (from_begin).
template <int D>
__global__ __launch_bounds__(256) void coarse_meta_kernel(CoarseArgs a) {
  constexpr int E = 2 * D / 64;
  const int b = blockIdx.z, h = blockIdx.y;
  const int first = a.super_begin ? max(a.super_begin[b], 0) : 0;
  const int jc = (a.from_begin ? first : 0) + blockIdx.x * 4 + wave_id();
  const int lane = lane_id();
  if (h == 0 && jc < a.pc_max && lane == 0) a.coarse_table[(size_t)b * a.pc_max + jc] = b * a.pc_max + jc;
  const int P = min((a.seq_lens[b] + kPage - 1) / kPage, a.max_pages);
  const int Pc = (P + a.group - 1) / a.group;
  if (h == 0 && blockIdx.x == 0 && threadIdx.x == 0) a.coarse_lens[b] = kPage * Pc;
  if (jc >= Pc || jc < first) return;  // wave-uniform
  const bool max_row = lane >= 32;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = max_row ? -INFINITY : INFINITY;
  // member pages 8 at a time: their block-table entries in one load (lane i
  // takes page j0 + i%8), then their 8 rows, all in flight together; a slot
  // past the super-page's last page re-reads the last (min and max do not
  // change)
  const int j_end = min((jc + 1) * a.group, P);
  for (int j0 = jc * a.group; j0 < j_end; j0 += 8) {  // wave-uniform
    const int phys_v = a.block_table[(size_t)b * a.max_pages + min(j0 + (lane & 7), j_end - 1)];
    float v[8][E];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const float* m = a.meta + ((size_t)__builtin_amdgcn_readlane(phys_v, p) * a.H + h) * 2 * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) v[p][e] = m[e];
    }
#pragma unroll
    for (int p = 0; p < 8; ++p)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = max_row ? fmaxf(acc[e], v[p][e]) : fminf(acc[e], v[p][e]);
  }
  float* out = a.coarse + (((size_t)b * a.pc_max + jc) * a.H + h) * 2 * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) out[e] = acc[e];
}

struct MaskedArgs {
  ScoreView v;
  const int32_t* seq_lens;
  const int32_t* sel_super;   // [B][H][kc_cap] ascending
  const int32_t* sel_count;   // [B][H]
  int kc_cap, group;
};

// -inf over pages [lo, hi) of a row (lane-parallel stores).
__device__ __forceinline__ void fill_neg_inf(float* row, int lo, int hi) {
  for (int j = lo + lane_id(); j < hi; j += kWave) row[j] = -INFINITY;
}

// One wave per (row, kept slot k): scores the pages of super-page
// sel_super[row][k] below the sequence's length (8 at a time, as the scorer
// does), and writes -inf over the pages between the previous kept super-page
// and this one, over this super-page's pages past the length, and -- for the
// last kept slot -- over every page after it.  A row with nothing kept is
// all -inf (slot 0 writes it).  Grid ceil(rows * kc_cap / 4), 4 waves per block.
template <int D, int G>
__global__ __launch_bounds__(256) void page_scores_masked_kernel(MaskedArgs a, int rows) {
  constexpr int E = ScoreQuery<D, G>::E;
  const long long item = (long long)blockIdx.x * kScoreWaves + wave_id();
  if (item >= (long long)rows * a.kc_cap) return;
  const int row = (int)(item / a.kc_cap), k = (int)(item % a.kc_cap);
  const int b = row / a.v.H, g = row % a.v.H;
  const int lane = lane_id();
  float* out = a.v.scores + (size_t)row * a.v.max_pages;
  const int cnt = min(__builtin_amdgcn_readfirstlane(vload_i32(a.sel_count, row)), a.kc_cap);
  if (k >= cnt) {
    if (k == 0) fill_neg_inf(out, 0, a.v.max_pages);
    return;
  }
  const int32_t* sel = a.sel_super + (size_t)row * a.kc_cap;
  const int jc = __builtin_amdgcn_readfirstlane(vload_i32(sel, k));
  const int prev = k > 0 ? __builtin_amdgcn_readfirstlane(vload_i32(sel, k - 1)) : -1;
  const int P = min((__builtin_amdgcn_readfirstlane(vload_i32(a.seq_lens, b)) + kPage - 1) / kPage, a.v.max_pages);
  const int j_lo = min(jc * a.group, a.v.max_pages), j_hi = min((jc + 1) * a.group, a.v.max_pages);
  fill_neg_inf(out, min((prev + 1) * a.group, a.v.max_pages), j_lo);
  fill_neg_inf(out, max(min(P, j_hi), j_lo), j_hi);
  if (k == cnt - 1) fill_neg_inf(out, j_hi, a.v.max_pages);
  const int live = min(P, j_hi);
  const ScoreSeqs ss{a.seq_lens, nullptr, nullptr, rows};
  for (int j0 = j_lo; j0 < live; j0 += kScorePagesPerWave) {  // wave-uniform
    const ScoreHead<D, G> h = score_head_load<D, G, false>(a.v, ss, b, g, j0);
    float vals[kScorePagesPerWave][E];
#pragma unroll
    for (int p = 0; p < kScorePagesPerWave; ++p) {
      const int ph = j0 + p < live ? __builtin_amdgcn_readlane(h.bt, p) : 0;
      const float* m = a.v.meta + ((size_t)ph * a.v.H + g) * 2 * D + lane * E;
      if constexpr (E == 4) {
        const float4 v = load_stream_f4(m);
        vals[p][0] = v.x; vals[p][1] = v.y; vals[p][2] = v.z; vals[p][3] = v.w;
      } else {
        const float2 v = load_stream_f2(m);
        vals[p][0] = v.x; vals[p][1] = v.y;
      }
    }
    const ScoreQuery<D, G> q = score_query_of<D, G>(h);
#pragma unroll
    for (int p = 0; p < kScorePagesPerWave; ++p) {
      const int j = j0 + p;
      if (j >= live) break;
      const float best = score_from_values<D, G>(q, vals[p]);
      if (lane == 0) out[j] = best;
    }
  }
}

template <int D>
hipError_t masked_d(const MaskedArgs& a, int rows, int G, hipStream_t st) {
  const long long items = (long long)rows * a.kc_cap;
  const dim3 grid((unsigned)((items + kScoreWaves - 1) / kScoreWaves));
  switch (G) {
    case 1: hipLaunchKernelGGL((page_scores_masked_kernel<D, 1>), grid, dim3(256), 0, st, a, rows); break;
    case 2: hipLaunchKernelGGL((page_scores_masked_kernel<D, 2>), grid, dim3(256), 0, st, a, rows); break;
    case 4: hipLaunchKernelGGL((page_scores_masked_kernel<D, 4>), grid, dim3(256), 0, st, a, rows); break;
    default: hipLaunchKernelGGL((page_scores_masked_kernel<D, 8>), grid, dim3(256), 0, st, a, rows); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_coarse_meta(const kvq_cache& c, const kvq_seqs& s, int group, const int32_t* super_begin,
                              int max_span, float* coarse, int32_t* coarse_lens, int32_t* coarse_table,
                              hipStream_t st) {
  const int pc_max = (s.max_pages + group - 1) / group;
  const bool from_begin = super_begin && max_span > 0 && max_span < pc_max;
  const int span = from_begin ? max_span : pc_max;
  CoarseArgs a{c.page_meta, s.block_table, s.seq_lens, super_begin, from_begin ? 1 : 0, coarse, coarse_lens,
               coarse_table, c.num_kv_heads, s.max_pages, group, pc_max, s.batch};
  const dim3 grid((span + 3) / 4, c.num_kv_heads, s.batch);
  if (c.head_dim == 64)
    hipLaunchKernelGGL(coarse_meta_kernel<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(coarse_meta_kernel<128>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_page_scores_masked(const kvq_cache& c, const kvq_seqs& s, const uint16_t* q, int num_q_heads,
                                     int group, const int32_t* sel_super, const int32_t* sel_count, int kc_cap,
                                     float* scores, hipStream_t st) {
  MaskedArgs a{{c.page_meta, s.block_table, q, scores, c.num_kv_heads, num_q_heads, s.max_pages}, s.seq_lens,
               sel_super, sel_count, kc_cap, group};
  const int rows = s.batch * c.num_kv_heads;
  const int G = num_q_heads / c.num_kv_heads;
  return c.head_dim == 64 ? masked_d<64>(a, rows, G, st) : masked_d<128>(a, rows, G, st);
}

}  // namespace kvq
