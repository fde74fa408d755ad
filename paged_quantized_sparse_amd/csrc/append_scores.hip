// append_scores.hip -- the decode-time append fused into page scoring.
//
// The scoring of page_scores.hip, with one change per (sequence, KV head)
// row that received rows: the scoring blocks skip the pages the rows touch,
// and one extra block per row appends the rows and rebuilds those pages'
// metadata (append_body.h), then scores them from the metadata it still holds
// in LDS with the same per-page arithmetic as the scorer (score_body.h), so
// every score equals what kvq_append_decode followed by kvq_page_scores gives.
// The append blocks come first in the grid, so they are dispatched first and
// their dependent loads run while the scoring blocks stream metadata.
#include "append_body.h"
#include "kvq_internal.h"
#include "score_body.h"

namespace kvq {
namespace {

struct AppendScoreArgs {
  AppendView ap;
  ScoreView sc;
  const int32_t* seq_lens;
};

// 1-D grid of (1 + ceil(max_pages / 32)) * B * H_kv blocks of 256 threads:
// block L < B * H_kv appends for row L; the others score 32 pages each.
template <int FMT, int D, int G>
__global__ __launch_bounds__(256) KVQ_SCORE_OCC_ATTR void append_scores_kernel(AppendScoreArgs a, int rows) {
  __shared__ float sm_meta[kMaxTouched][2][D];
  const int L = blockIdx.x;
  const int row = L % rows, c = L / rows - 1;  // c = -1: the row's append block
  const int b = row / a.sc.H, g = row % a.sc.H;
  const int j0 = (c * kScoreWaves + wave_id()) * kScorePagesPerWave;
  const int bt_v = score_table_load(a.sc, b, j0);  // issued first; unused by the append block
  // per-sequence values as pending vector loads (see vload_i32)
  const int len_v = vload_i32(a.seq_lens, b);
  const int off0_v = vload_i32(a.ap.new_off, b), off1_v = vload_i32(a.ap.new_off, b + 1);
  const int start_v = vload_i32(a.ap.start_pos, b);
  ScoreQuery<D, G> q;
  q.load(a.sc, b, g);
  __builtin_amdgcn_sched_barrier(0);
  // the touched pages [first, first + count) of the rows (count 0: no rows); at most 64 rows,
  // as the append itself clamps them
  auto touched = [&](int& P, int& first, int& count) {
    P = (__builtin_amdgcn_readfirstlane(len_v) + kPage - 1) / kPage;
    const int n = min(__builtin_amdgcn_readfirstlane(off1_v) - __builtin_amdgcn_readfirstlane(off0_v), 64);
    const int start = __builtin_amdgcn_readfirstlane(start_v);
    first = start / kPage;
    count = n > 0 ? (start + n - 1) / kPage - first + 1 : 0;
  };
  if (c < 0) {  // block-uniform
    int P, first, count;
    touched(P, first, count);
    if (count == 0 || P == 0) return;
    append_rows_and_meta<FMT, D>(a.ap, b, g, sm_meta);
    if (wave_id() == 0) {
      constexpr int E = ScoreQuery<D, G>::E;
      float* out = a.sc.scores + ((size_t)b * a.sc.H + g) * a.sc.max_pages;
      for (int p = 0; p < count && first + p < P; ++p) {
        const float best = score_from_values<D, G>(q, &sm_meta[p][0][0] + lane_id() * E);
        if (lane_id() == 0) out[first + p] = best;
      }
    }
    return;
  }
  score_pages<D, G>(a.sc, q, b, g, j0, bt_v, [&](int& P, int& skip_from) {
    int first, count;
    touched(P, first, count);
    skip_from = count > 0 ? first : P;  // the rows touch pages [first, P)
  });
}

template <int FMT, int D>
hipError_t launch_g(const AppendScoreArgs& a, int rows, int G, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1: hipLaunchKernelGGL((append_scores_kernel<FMT, D, 1>), grid, dim3(256), 0, st, a, rows); break;
    case 2: hipLaunchKernelGGL((append_scores_kernel<FMT, D, 2>), grid, dim3(256), 0, st, a, rows); break;
    case 4: hipLaunchKernelGGL((append_scores_kernel<FMT, D, 4>), grid, dim3(256), 0, st, a, rows); break;
    default: hipLaunchKernelGGL((append_scores_kernel<FMT, D, 8>), grid, dim3(256), 0, st, a, rows); break;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_d(const AppendScoreArgs& a, int d, int rows, int G, dim3 grid, hipStream_t st) {
  return d == 64 ? launch_g<FMT, 64>(a, rows, G, grid, st) : launch_g<FMT, 128>(a, rows, G, grid, st);
}

}  // namespace

hipError_t launch_append_scores(const kvq_cache& c, const kvq_seqs& s, const int32_t* start_pos,
                                const int32_t* new_off, const uint16_t* k_new, const uint16_t* v_new,
                                const uint16_t* q, int num_q_heads, float* scores, hipStream_t st) {
  AppendScoreArgs a{{c.k_pages, c.v_pages, c.kv_params, c.page_meta, s.block_table, start_pos, new_off, k_new,
                     v_new, c.num_kv_heads, s.max_pages},
                    {c.page_meta, s.block_table, q, scores, c.num_kv_heads, num_q_heads, s.max_pages},
                    s.seq_lens};
  const int per_block = kScoreWaves * kScorePagesPerWave;
  const int rows = s.batch * c.num_kv_heads;
  const long long blocks = (1LL + (s.max_pages + per_block - 1) / per_block) * rows;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks);
  const int G = num_q_heads / c.num_kv_heads;
  if (c.format == KVQ_FP16) return launch_d<kFp16>(a, c.head_dim, rows, G, grid, st);
  if (c.format == KVQ_INT8_TOKEN) return launch_d<kInt8Token>(a, c.head_dim, rows, G, grid, st);
  return launch_d<kInt8Group>(a, c.head_dim, rows, G, grid, st);
}

}  // namespace kvq
