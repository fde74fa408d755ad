// page_scores.hip -- query-aware page relevance of every logical page
// ("TinyServe", lpnh.cn, section 2.1); the scorer itself is score_body.h.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "score_body.h"

namespace kvq {
namespace {

struct ScoreArgs {
  ScoreView v;
  const int32_t* seq_lens;
};

// grid (ceil(max_pages / 32), H_kv, B), 256 threads; each wave scores 8 pages.
template <int D, int G>
__global__ __launch_bounds__(256) KVQ_SCORE_OCC_ATTR void page_scores_kernel(ScoreArgs a) {
  const int b = blockIdx.z, g = blockIdx.y;
  const int j0 = (blockIdx.x * kScoreWaves + wave_id()) * kScorePagesPerWave;
  const int bt_v = score_table_load(a.v, b, j0);
  const int len_v = vload_i32(a.seq_lens, b);
  ScoreQuery<D, G> q;
  q.load(a.v, b, g);
  score_pages<D, G>(a.v, q, b, g, j0, bt_v, [&](int& P, int& skip_from) {
    P = (__builtin_amdgcn_readfirstlane(len_v) + kPage - 1) / kPage;
    skip_from = P;
  });
}

template <int D>
hipError_t launch_d(const ScoreArgs& a, int G, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1: hipLaunchKernelGGL((page_scores_kernel<D, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((page_scores_kernel<D, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((page_scores_kernel<D, 4>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((page_scores_kernel<D, 8>), grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_page_scores(const kvq_cache& c, const kvq_seqs& s, const uint16_t* q, int num_q_heads,
                              float* scores, hipStream_t st) {
  ScoreArgs a{{c.page_meta, s.block_table, q, scores, c.num_kv_heads, num_q_heads, s.max_pages}, s.seq_lens};
  const int per_block = kScoreWaves * kScorePagesPerWave;
  dim3 grid((s.max_pages + per_block - 1) / per_block, c.num_kv_heads, s.batch);
  const int G = num_q_heads / c.num_kv_heads;
  return c.head_dim == 64 ? launch_d<64>(a, G, grid, st) : launch_d<128>(a, G, grid, st);
}

}  // namespace kvq
