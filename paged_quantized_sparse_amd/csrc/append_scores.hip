// append_scores.hip -- the decode-time append fused into page scoring.
//
// The scoring of page_scores.hip, with one change per (sequence, KV head)
// row that received rows: the scoring waves skip the pages the rows touch,
// and one extra block per row appends the rows and rebuilds those pages'
// metadata (append_body.h), then scores them from the metadata it still holds
// in LDS with the same per-page arithmetic as the scorer (score_body.h), so
// every score equals what kvq_append_decode followed by kvq_page_scores gives.
// The append blocks come first in the grid, so they are dispatched first and
// their dependent loads run while the persistent scoring grid, sized to the
// slots they leave, streams metadata.
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

// 1-D grid: blocks 0 .. rows-1 append for row b * H_kv + g (then exit); the
// rest are a persistent scoring grid whose waves take 8-page items (BAL:
// balanced over the live items, for a persistent grid over a ragged batch).
template <int FMT, int D, int G, bool BAL>
__global__ __launch_bounds__(256) void append_scores_kernel(AppendScoreArgs a, int rows) {
  const int L = blockIdx.x;
  if (L >= rows) {  // block-uniform
    const ScoreSeqs ss{a.seq_lens, a.ap.new_off, a.ap.start_pos, rows};
    const int gw = (L - rows) * kScoreWaves + wave_id(), TW = ((int)gridDim.x - rows) * kScoreWaves;
    if constexpr (BAL) {
      __shared__ int sm_pref[kScoreMaxSeqs + 1];
      __shared__ int sm_wsum[kScoreWaves];
      score_items_balanced<D, G, true>(a.sc, ss, gw, TW, ScoreShared{sm_pref, sm_wsum});
    } else {
      score_items<D, G, true>(a.sc, ss, gw, TW);
    }
    return;
  }
  __shared__ float sm_meta[kMaxTouched][2][D];
  const int b = L / a.sc.H, g = L % a.sc.H;
  const int len = vload_i32(a.seq_lens, b);
  const int off0 = vload_i32(a.ap.new_off, b), off1 = vload_i32(a.ap.new_off, b + 1);
  const int start = __builtin_amdgcn_readfirstlane(vload_i32(a.ap.start_pos, b));
  ScoreQuery<D, G> q;
  q.load(a.sc, b, g);
  // the touched pages [first, first + count) of the rows (count 0: no rows);
  // at most 64 rows, as the append itself clamps them
  const int P = (__builtin_amdgcn_readfirstlane(len) + kPage - 1) / kPage;
  const int n = min(__builtin_amdgcn_readfirstlane(off1) - __builtin_amdgcn_readfirstlane(off0), 64);
  const int first = start / kPage;
  const int count = n > 0 ? (start + n - 1) / kPage - first + 1 : 0;
  if (count == 0 || P == 0) return;  // block-uniform
  append_rows_and_meta<FMT, D>(a.ap, b, g, sm_meta);
  if (wave_id() == 0) {
    constexpr int E = ScoreQuery<D, G>::E;
    float* out = a.sc.scores + ((size_t)b * a.sc.H + g) * a.sc.max_pages;
    for (int p = 0; p < count && first + p < P; ++p) {
      const float best = score_from_values<D, G>(q, &sm_meta[p][0][0] + lane_id() * E);
      if (lane_id() == 0) out[first + p] = best;
    }
  }
}

template <int FMT, int D, int G>
hipError_t launch_k(const AppendScoreArgs& a, int rows, hipStream_t st) {
  static std::atomic<long long> memo[kMaxDevices], memo_bal[kMaxDevices];
  const int capacity = (int)per_device(
      memo, [] { return resident_blocks(reinterpret_cast<const void*>(&append_scores_kernel<FMT, D, G, false>)); });
  const int capacity_bal = (int)per_device(
      memo_bal, [] { return resident_blocks(reinterpret_cast<const void*>(&append_scores_kernel<FMT, D, G, true>)); });
  const int items = rows * ((a.sc.max_pages + kScorePagesPerWave - 1) / kScorePagesPerWave);
  int blocks = score_grid_blocks(capacity, items, rows);
  if (blocks < 1) return hipErrorInvalidConfiguration;
  const bool bal = score_balanced(rows, a.sc.H, a.sc.max_pages, blocks * kScoreWaves);
  if (bal) blocks = score_grid_blocks(capacity_bal, items, rows);
  if (blocks < 1 || (long long)blocks + rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (bal)
    hipLaunchKernelGGL((append_scores_kernel<FMT, D, G, true>), dim3(rows + blocks), dim3(256), 0, st, a, rows);
  else
    hipLaunchKernelGGL((append_scores_kernel<FMT, D, G, false>), dim3(rows + blocks), dim3(256), 0, st, a, rows);
  return hipGetLastError();
}

template <int FMT, int D>
hipError_t launch_g(const AppendScoreArgs& a, int rows, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_k<FMT, D, 1>(a, rows, st);
    case 2: return launch_k<FMT, D, 2>(a, rows, st);
    case 4: return launch_k<FMT, D, 4>(a, rows, st);
    default: return launch_k<FMT, D, 8>(a, rows, st);
  }
}

template <int FMT>
hipError_t launch_d(const AppendScoreArgs& a, int d, int rows, int G, hipStream_t st) {
  if constexpr (fmt_int4(FMT))
    return launch_g<FMT, 128>(a, rows, G, st);
  else
    return d == 64 ? launch_g<FMT, 64>(a, rows, G, st) : launch_g<FMT, 128>(a, rows, G, st);
}

}  // namespace

hipError_t launch_append_scores(const kvq_cache& c, const kvq_seqs& s, const int32_t* start_pos,
                                const int32_t* new_off, const uint16_t* k_new, const uint16_t* v_new,
                                const uint16_t* q, int num_q_heads, float* scores, hipStream_t st) {
  AppendScoreArgs a{{c.k_pages, c.v_pages, c.kv_params, c.page_meta, s.block_table, start_pos, new_off, k_new,
                     v_new, c.num_kv_heads, s.max_pages, fp16_pool(c)},
                    {c.page_meta, s.block_table, q, scores, c.num_kv_heads, num_q_heads, s.max_pages},
                    s.seq_lens};
  const int rows = s.batch * c.num_kv_heads;
  const int G = num_q_heads / c.num_kv_heads;
  if (c.format == KVQ_FP16) return launch_d<kFp16>(a, c.head_dim, rows, G, st);
  if (c.format == KVQ_INT8_TOKEN) return launch_d<kInt8Token>(a, c.head_dim, rows, G, st);
  if (c.format == KVQ_INT8_GROUP64) return launch_d<kInt8Group>(a, c.head_dim, rows, G, st);
  if (c.format == KVQ_INT4_TOKEN) return launch_d<kInt4Token>(a, c.head_dim, rows, G, st);
  if (c.format == KVQ_MIXED_FP16_INT8) return launch_d<kMixed>(a, c.head_dim, rows, G, st);
  return launch_d<kInt4Group>(a, c.head_dim, rows, G, st);
}

}  // namespace kvq
