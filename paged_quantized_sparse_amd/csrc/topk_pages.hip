// topk_pages.hip -- per (sequence, KV head) row, select the K_b pages with the
// largest scores ("TinyServe", lpnh.cn, section 3.1 phase 2; section 5.1
// selection_ratio), ties to the lower logical page, output ascending.
//
// One 1024-thread block per row.  Scores become order-preserving uint32 keys
// in LDS.  All keys share the bits above the highest bit where the row's
// minimum and maximum key differ; radix passes of up to 11 bits (MSB first,
// LDS histograms) over the bits below it find the K-th largest key T and how
// many keys equal to T are still needed.  (Starting at the top bit instead
// would put nearly every score of similar magnitude into one or two bins of
// the first pass and serialize its LDS atomics.)  Block-wide scans over
// 1024-key rounds, in page order, then write every key > T and the first
// `need` keys == T, ascending.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

struct TopkArgs {
  const float* scores;
  const int32_t* seq_lens;
  int32_t* sel_pages;
  int32_t* sel_count;
  int H;
  int max_pages;
  int rnum, rden, k_fixed, k_cap;
};

// Inclusive scan of one value per thread over the 1024-thread block.
__device__ __forceinline__ int block_inclusive_scan(int v, int* wsum) {
  const int lane = lane_id(), w = wave_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  if (w == 0) {
    int x = lane < kTopkWaves ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < kTopkWaves; off <<= 1) {
      const int t = __shfl_up(x, off, 64);
      if (lane >= off) x += t;
    }
    if (lane < kTopkWaves) wsum[kTopkWaves + lane] = x - wsum[lane];  // exclusive wave offsets
  }
  __syncthreads();
  v += wsum[kTopkWaves + w];
  __syncthreads();
  return v;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ uint32_t keys[];  // [max_pages]
  __shared__ int hist[2048];
  __shared__ int wsum[2 * kTopkWaves];
  __shared__ int pick[2];

  const int row = blockIdx.x;  // b * H + g
  const int b = row / a.H;
  const int tid = threadIdx.x;
  const int P = (a.seq_lens[b] + kPage - 1) / kPage;
  const int K = num_selected(P, a.rnum, a.rden, a.k_fixed);
  int32_t* out = a.sel_pages + (size_t)row * a.k_cap;
  if (tid == 0) a.sel_count[row] = K;

  if (K >= P) {  // every page
    for (int i = tid; i < a.k_cap; i += kTopkThreads) out[i] = i < P ? i : -1;
    return;
  }

  const float* sc = a.scores + (size_t)row * a.max_pages;
  for (int j0 = 0; j0 < P; j0 += 4 * kTopkThreads) {  // four loads in flight per thread
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * kTopkThreads + tid;
      v[u] = j < P ? sc[j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * kTopkThreads + tid;
      if (j < P) keys[j] = float_key(v[u]);
    }
  }

  // the row's key range: every key shares the bits above `lead`
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int j = tid; j < P; j += kTopkThreads) {
    const uint32_t k = keys[j];
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off, 64));
  }
  if (lane_id() == 0) {
    wsum[wave_id()] = (int)kmin;
    wsum[kTopkWaves + wave_id()] = (int)kmax;
  }
  __syncthreads();
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
#pragma unroll
  for (int v = 0; v < kTopkWaves; ++v) {
    kmin = min(kmin, (uint32_t)wsum[v]);
    kmax = max(kmax, (uint32_t)wsum[kTopkWaves + v]);
  }
  __syncthreads();
  const int lead = kmax == kmin ? -1 : 31 - __builtin_clz(kmax ^ kmin);  // highest differing bit
  uint32_t mask = lead < 0 ? 0xFFFFFFFFu : (lead >= 31 ? 0u : ~((2u << lead) - 1u));
  uint32_t prefix = kmax & mask;
  int need = K;  // keys still to take among those matching the prefix
  int hi_bit = lead;  // next bit to resolve
#pragma unroll 1
  while (hi_bit >= 0) {
    const int bits = hi_bit + 1 < 11 ? hi_bit + 1 : 11;
    const int shift = hi_bit + 1 - bits;
    const int nbins = 1 << bits;
    for (int i = tid; i < 2048; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < P; j += kTopkThreads) {
      const uint32_t k = keys[j];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & (nbins - 1)], 1);
    }
    __syncthreads();
    // thread t owns bins 2047-2t and 2046-2t of a 2048-bin view (bins at or
    // above nbins are empty), counted from the top
    const int top = 2047 - 2 * tid;
    const int c0 = hist[top], c1 = hist[top - 1];
    const int own = c0 + c1;
    const int incl = block_inclusive_scan(own, wsum);  // keys in bins above mine, plus mine
    int above = incl - own;
    if (above < need && above + c0 >= need) { pick[0] = top; pick[1] = need - above; }
    above += c0;
    if (above < need && above + c1 >= need) { pick[0] = top - 1; pick[1] = need - above; }
    __syncthreads();
    prefix |= (uint32_t)pick[0] << shift;
    mask |= (uint32_t)(nbins - 1) << shift;
    need = pick[1];
    hi_bit = shift - 1;
    __syncthreads();
  }
  const uint32_t T = prefix;

  // rounds of 1024 consecutive pages keep the output ascending
  int gt_base = 0, eq_base = 0;
  for (int j0 = 0; j0 < P; j0 += kTopkThreads) {
    const int j = j0 + tid;
    const uint32_t k = j < P ? keys[j] : 0u;
    const int is_gt = j < P && k > T, is_eq = j < P && k == T;
    const int packed = block_inclusive_scan(is_gt | (is_eq << 16), wsum);  // both counts <= 1024
    const int gt_before = gt_base + (packed & 0xFFFF) - is_gt;
    const int eq_before = eq_base + (packed >> 16) - is_eq;
    if (is_gt) out[gt_before + min(eq_before, need)] = j;
    else if (is_eq && eq_before < need) out[gt_before + eq_before] = j;
    if (tid == kTopkThreads - 1) {
      pick[0] = packed & 0xFFFF;
      pick[1] = packed >> 16;
    }
    __syncthreads();
    gt_base += pick[0];
    eq_base += pick[1];
    __syncthreads();
  }
  for (int i = K + tid; i < a.k_cap; i += kTopkThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_topk(const float* scores, const kvq_seqs& s, int num_kv_heads, int rnum, int rden,
                       int k_fixed, int k_cap, int32_t* sel_pages, int32_t* sel_count, hipStream_t st) {
  TopkArgs a{scores, s.seq_lens, sel_pages, sel_count, num_kv_heads, s.max_pages, rnum, rden, k_fixed, k_cap};
  const size_t lds = (size_t)s.max_pages * sizeof(uint32_t);
  hipLaunchKernelGGL(topk_kernel, dim3(s.batch * num_kv_heads), dim3(kTopkThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace kvq
