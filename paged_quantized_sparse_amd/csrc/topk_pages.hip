// topk_pages.hip -- per (sequence, KV head) row, select the K_b pages with the
// largest scores ("TinyServe", lpnh.cn, section 3.1 phase 2; section 5.1
// selection_ratio), ties to the lower logical page, output ascending.
//
// One 256-thread block per row.  Scores become order-preserving uint32 keys
// in LDS; a 4-pass 8-bit radix select (MSB first, LDS histograms) finds the
// K-th largest key T and how many keys equal to T are still needed.  A
// block-wide exclusive scan over contiguous index chunks then writes every
// key > T and the first `need` keys == T in ascending page order.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kTopkThreads = 256;

struct TopkArgs {
  const float* scores;
  const int32_t* seq_lens;
  int32_t* sel_pages;
  int32_t* sel_count;
  int H;
  int max_pages;
  int rnum, rden, k_fixed, k_cap;
};

// Exclusive scan of one value per thread over the block; returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int& total) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int off = 1; off < kTopkThreads; off <<= 1) {
    const int add = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  total = tmp[kTopkThreads - 1];
  const int excl = tmp[tid] - v;
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ uint32_t keys[];  // [max_pages]
  __shared__ int hist[256];
  __shared__ int scan_tmp[kTopkThreads];
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
  for (int j = tid; j < P; j += kTopkThreads) keys[j] = float_key(sc[j]);
  __syncthreads();

  uint32_t prefix = 0, mask = 0;
  int need = K;  // keys still to take among those matching the prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < P; j += kTopkThreads) {
      const uint32_t k = keys[j];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // suffix counts over digits: lane l owns digits 4l..4l+3
      int c[4], s = 0;
#pragma unroll
      for (int i = 3; i >= 0; --i) { c[i] = hist[4 * tid + i]; }
      const int own = c[0] + c[1] + c[2] + c[3];
      // inclusive suffix sum of `own` across lanes (lanes above me)
      int suf = own;
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_down(suf, off, 64);
        if (tid + off < 64) suf += o;
      }
      const int above = suf - own;  // count of digits > 4*tid+3
      // find the digit D with count(> D) < need <= count(>= D)
      s = above;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (s < need && s + c[i] >= need) { pick[0] = 4 * tid + i; pick[1] = need - s; }
        s += c[i];
      }
    }
    __syncthreads();
    const int digit = pick[0];
    need = pick[1];
    prefix |= (uint32_t)digit << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;

  // contiguous chunk of pages per thread keeps the output ascending
  const int chunk = (P + kTopkThreads - 1) / kTopkThreads;
  const int lo = min(P, tid * chunk), hi = min(P, lo + chunk);
  int n_gt = 0, n_eq = 0;
  for (int j = lo; j < hi; ++j) {
    const uint32_t k = keys[j];
    n_gt += k > T;
    n_eq += k == T;
  }
  int tot;
  int gt_before = block_exclusive_scan(n_gt, scan_tmp, tot);
  int eq_before = block_exclusive_scan(n_eq, scan_tmp, tot);
  for (int j = lo; j < hi; ++j) {
    const uint32_t k = keys[j];
    const int pos = gt_before + min(eq_before, need);
    if (k > T) {
      out[pos] = j;
      ++gt_before;
    } else if (k == T) {
      if (eq_before < need) out[pos] = j;
      ++eq_before;
    }
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
