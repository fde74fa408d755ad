// page_scores.hip -- query-aware page relevance of every logical page
// ("TinyServe", lpnh.cn, section 2.1); the scorer itself is score_body.h.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "score_body.h"

namespace kvq {
namespace {

struct ScoreArgs {
  ScoreView v;
  ScoreSeqs ss;
};

// Persistent grid of 256-thread blocks; each wave scores 8-page items
// (balanced over the live items for a persistent grid over a ragged batch).
template <int D, int G, bool BAL>
__global__ __launch_bounds__(256) void page_scores_kernel(ScoreArgs a) {
  const int gw = blockIdx.x * kScoreWaves + wave_id(), TW = gridDim.x * kScoreWaves;
  if constexpr (BAL) {
    __shared__ int sm_pref[kScoreMaxSeqs + 1];
    __shared__ int sm_wsum[kScoreWaves];
    score_items_balanced<D, G, false>(a.v, a.ss, gw, TW, ScoreShared{sm_pref, sm_wsum});
  } else {
    score_items<D, G, false>(a.v, a.ss, gw, TW);
  }
}

template <int D, int G>
hipError_t launch_g(const ScoreArgs& a, hipStream_t st) {
  static std::atomic<long long> memo[kMaxDevices], memo_bal[kMaxDevices];
  const int capacity = (int)per_device(
      memo, [] { return resident_blocks(reinterpret_cast<const void*>(&page_scores_kernel<D, G, false>)); });
  const int capacity_bal = (int)per_device(
      memo_bal, [] { return resident_blocks(reinterpret_cast<const void*>(&page_scores_kernel<D, G, true>)); });
  const int items = a.ss.rows * ((a.v.max_pages + kScorePagesPerWave - 1) / kScorePagesPerWave);
  int blocks = score_grid_blocks(capacity, items, 0);
  if (blocks < 1) return hipErrorInvalidConfiguration;
  if (score_balanced(a.ss.rows, a.v.H, a.v.max_pages, blocks * kScoreWaves)) {
    blocks = score_grid_blocks(capacity_bal, items, 0);
    if (blocks < 1) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((page_scores_kernel<D, G, true>), dim3(blocks), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((page_scores_kernel<D, G, false>), dim3(blocks), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const ScoreArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_g<D, 1>(a, st);
    case 2: return launch_g<D, 2>(a, st);
    case 4: return launch_g<D, 4>(a, st);
    default: return launch_g<D, 8>(a, st);
  }
}

}  // namespace

hipError_t launch_page_scores(const kvq_cache& c, const kvq_seqs& s, const uint16_t* q, int num_q_heads,
                              float* scores, hipStream_t st) {
  ScoreArgs a{{c.page_meta, s.block_table, q, scores, c.num_kv_heads, num_q_heads, s.max_pages},
              {s.seq_lens, nullptr, nullptr, s.batch * c.num_kv_heads}};
  const int G = num_q_heads / c.num_kv_heads;
  return c.head_dim == 64 ? launch_d<64>(a, G, st) : launch_d<128>(a, G, st);
}

}  // namespace kvq
