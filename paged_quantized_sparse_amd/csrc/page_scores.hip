// page_scores.hip -- query-aware page relevance ("TinyServe", lpnh.cn,
// section 2.1): r(q, phi_j) = sum_i (q_i >= 0 ? q_i M_j[i] : q_i m_j[i]),
// which never underestimates q.k for any key of page j.  Written as
// sum_i max(q_i, 0) M_j[i] + min(q_i, 0) m_j[i], which takes the same terms
// without a per-channel select.  For GQA the KV group's score is the max over
// its query heads, so it still bounds every member head's q.k.
//
// Layout per (physical page, KV head): meta[2][d] fp32 (min row, max row) =
// 8d bytes, read as one contiguous wave load: lanes 0-31 hold min-row channels,
// lanes 32-63 the max-row channels.  The query stays in registers.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

struct ScoreArgs {
  const float* meta;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint16_t* q;
  float* scores;
  int H;
  int Hq;
  int max_pages;
};

constexpr int kScoreWaves = 4;
constexpr int kScorePagesPerWave = 8;

// grid (ceil(max_pages / 32), H_kv, B), 256 threads; each wave scores 8 pages.
template <int D, int G>
__global__ __launch_bounds__(256) void page_scores_kernel(ScoreArgs a) {
  constexpr int E = 2 * D / 64;  // floats per lane (4 for d = 128, 2 for d = 64)
  const int b = blockIdx.z, g = blockIdx.y;
  const int lane = lane_id();
  const int P = (a.seq_lens[b] + kPage - 1) / kPage;
  const int jbase = (blockIdx.x * kScoreWaves + wave_id()) * kScorePagesPerWave;
  float* out = a.scores + ((size_t)b * a.H + g) * a.max_pages;

  // this lane's query coefficients: max(q, 0) on the max row, min(q, 0) on the min row
  const bool max_row = lane >= 32;
  const int ch0 = (lane & 31) * E;
  float qc[G][E];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint16_t* qh = a.q + ((size_t)b * a.Hq + g * G + hh) * D + ch0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = half_bits_to_float(qh[e]);
      qc[hh][e] = max_row ? fmaxf(x, 0.0f) : fminf(x, 0.0f);
    }
  }

  float vals[kScorePagesPerWave][E];
#pragma unroll
  for (int k = 0; k < kScorePagesPerWave; ++k) {
    const int j = jbase + k;
    if (j < P) {
      const int phys = a.block_table[(size_t)b * a.max_pages + j];
      const float* m = a.meta + ((size_t)phys * a.H + g) * 2 * D + lane * E;
      if constexpr (E == 4) {
        const float4 v = *(const float4*)m;
        vals[k][0] = v.x; vals[k][1] = v.y; vals[k][2] = v.z; vals[k][3] = v.w;
      } else {
        const float2 v = *(const float2*)m;
        vals[k][0] = v.x; vals[k][1] = v.y;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kScorePagesPerWave; ++k) {
    const int j = jbase + k;
    if (j >= a.max_pages) break;
    float best = -INFINITY;
    if (j < P) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float r = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) r = __builtin_fmaf(qc[hh][e], vals[k][e], r);
        r = sum_contig<64>(r);
        best = fmaxf(best, r);
      }
    }
    if (lane == 0) out[j] = best;
  }
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
  ScoreArgs a{c.page_meta, s.block_table, s.seq_lens, q, scores, c.num_kv_heads, num_q_heads, s.max_pages};
  const int per_block = kScoreWaves * kScorePagesPerWave;
  dim3 grid((s.max_pages + per_block - 1) / per_block, c.num_kv_heads, s.batch);
  const int G = num_q_heads / c.num_kv_heads;
  return c.head_dim == 64 ? launch_d<64>(a, G, grid, st) : launch_d<128>(a, G, grid, st);
}

}  // namespace kvq
