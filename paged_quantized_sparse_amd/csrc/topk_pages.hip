// topk_pages.hip -- per (sequence, KV head) row, select the K_b pages with the
// largest scores ("TinyServe", lpnh.cn, section 3.1 phase 2; section 5.1
// selection_ratio), ties to the lower logical page, output ascending.
//
// One 1024-thread block per row.  Scores become order-preserving uint32 keys
// in LDS.  All keys share the bits above the highest bit where the row's
// minimum and maximum key differ; radix passes of up to 11 bits (MSB first)
// over the bits below it, with LDS histograms, find the K-th largest key T and
// how many keys equal to T are still needed.  (Starting at the top bit
// instead would put nearly every score of similar magnitude into one or two
// bins and serialize the histogram atomics.)  Selection is a chain of short
// dependent steps, so the block is built for latency: cross-lane work is DPP
// and ballots (no LDS shuffles), histograms are double-buffered so zeroing the
// next one overlaps the current pass, and every wave finds the chosen bin
// itself instead of waiting for a broadcast -- two barriers per pass.  The
// passes stop early once the chosen bin holds exactly the keys still needed:
// then every key of that bin is taken, whatever its unresolved low bits.
// Rounds of 1024 pages in page order then write every key above the chosen
// prefix (compared on the resolved bits) and the first `need` keys on it,
// ascending.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kHistBins = 2048;

struct TopkArgs {
  const float* scores;
  const int32_t* seq_lens;
  int32_t* sel_pages;
  int32_t* sel_count;
  int H;
  int max_pages;
  int rnum, rden, k_fixed, k_cap;
};

// The 16 per-wave values of an LDS array, one per lane of row 0 (lanes
// 16..63 read a copy of row 0 and are not used): a single LDS read instead of
// sixteen serialized ones.
__device__ __forceinline__ int per_wave_value(const int* arr, int lane) { return arr[lane & (kTopkWaves - 1)]; }

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ uint32_t keys[];  // [max_pages]
  __shared__ int hist[2][kHistBins];
  __shared__ int wtot[2][kTopkWaves];   // radix passes
  __shared__ int ctot[2][kTopkWaves];   // compaction rounds (a separate buffer: a slow wave may still
                                        // be reading wtot from the last pass)
  __shared__ uint32_t wrange[2][kTopkWaves];

  const int row = blockIdx.x;  // b * H + g
  const int b = row / a.H;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int P = (a.seq_lens[b] + kPage - 1) / kPage;
  const int K = num_selected(P, a.rnum, a.rden, a.k_fixed);
  int32_t* out = a.sel_pages + (size_t)row * a.k_cap;
  if (tid == 0) a.sel_count[row] = K;

  if (K >= P) {  // every page
    for (int i = tid; i < a.k_cap; i += kTopkThreads) out[i] = i < P ? i : -1;
    return;
  }

  // keys into LDS (four loads in flight per thread), the key range, and the
  // first histogram zeroed
  const float* sc = a.scores + (size_t)row * a.max_pages;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int j0 = 0; j0 < P; j0 += 4 * kTopkThreads) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * kTopkThreads + tid;
      v[u] = j < P ? sc[j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * kTopkThreads + tid;
      if (j < P) {
        const uint32_t k = float_key(v[u]);
        keys[j] = k;
        kmin = min(kmin, k);
        kmax = max(kmax, k);
      }
    }
  }
  for (int i = tid; i < kHistBins; i += kTopkThreads) hist[0][i] = 0;
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    wrange[0][w] = kmin;
    wrange[1][w] = kmax;
  }
  __syncthreads();
  kmin = wave_min_u32(wrange[0][lane & (kTopkWaves - 1)]);
  kmax = wave_max_u32(wrange[1][lane & (kTopkWaves - 1)]);
  const int lead = kmax == kmin ? -1 : 31 - __builtin_clz(kmax ^ kmin);  // highest differing bit
  uint32_t mask = lead < 0 ? 0xFFFFFFFFu : (lead >= 31 ? 0u : ~((2u << lead) - 1u));
  uint32_t prefix = kmax & mask;
  int need = K;  // keys still to take among those matching the prefix
  int hi_bit = lead;  // next bit to resolve
  int cur = 0;

#pragma unroll 1
  while (hi_bit >= 0) {
    const int bits = hi_bit + 1 < 11 ? hi_bit + 1 : 11;
    const int shift = hi_bit + 1 - bits;
    const int nbins = 1 << bits;
    int* h = hist[cur];
    for (int j = tid; j < P; j += kTopkThreads) {
      const uint32_t k = keys[j];
      if ((k & mask) == prefix) atomicAdd(&h[(k >> shift) & (nbins - 1)], 1);
    }
    __syncthreads();
    // thread t owns bins 2047-2t and 2046-2t, counted from the top (bins at
    // or above nbins stay empty); the next pass's histogram is zeroed now
    const int top = kHistBins - 1 - 2 * tid;
    const int c0 = h[top], c1 = h[top - 1];
    hist[cur ^ 1][tid] = 0;
    hist[cur ^ 1][tid + kTopkThreads] = 0;
    const int own = c0 + c1;
    const int incl = wave_incl_scan_add(own);
    if (lane == 63) wtot[cur][w] = incl;
    __syncthreads();
    // every wave finds the crossing wave (the first whose running total
    // reaches need), then the crossing bin, itself
    const int wt = per_wave_value(wtot[cur], lane);
    const int wrun = row16_incl_scan(wt);
    const uint64_t reach = __ballot(lane < kTopkWaves && wrun >= need);
    int wv = reach ? (int)__builtin_ctzll(reach) : kTopkWaves - 1;  // empty: unreachable, candidates cover need
    const int before = __builtin_amdgcn_readlane(wrun, wv) - __builtin_amdgcn_readlane(wt, wv);
    // lane l of the crossing wave covers bins 2047-2(64 wv + l) and below
    const int tb = kHistBins - 1 - 2 * (64 * wv + lane);
    const int d0 = h[tb], d1 = h[tb - 1];
    const int within = wave_incl_scan_add(d0 + d1);
    const int above = before + within - d0 - d1;
    const bool hit0 = above < need && above + d0 >= need;
    const bool hit1 = !hit0 && above + d0 < need && above + d0 + d1 >= need;
    const uint64_t m0 = __ballot(hit0), m1 = __ballot(hit1);
    const int src = m0 ? (int)__builtin_ctzll(m0) : (int)__builtin_ctzll(m1);
    const int src_above = __builtin_amdgcn_readlane(above, src);
    const int src_d0 = __builtin_amdgcn_readlane(d0, src);
    const int src_d1 = __builtin_amdgcn_readlane(d1, src);
    const int digit = m0 ? kHistBins - 1 - 2 * (64 * wv + src) : kHistBins - 2 - 2 * (64 * wv + src);
    need = m0 ? need - src_above : need - src_above - src_d0;
    prefix |= (uint32_t)digit << shift;
    mask |= (uint32_t)(nbins - 1) << shift;
    hi_bit = shift - 1;
    cur ^= 1;
    if ((m0 ? src_d0 : src_d1) == need) break;  // uniform: the whole bin is taken
  }
  // selected: every key whose resolved bits exceed the prefix, and the first
  // `need` keys whose resolved bits equal it
  const uint32_t T = prefix;

  // rounds of 1024 consecutive pages, in page order
  int gt_base = 0, eq_base = 0, par = 0;
  for (int j0 = 0; j0 < P; j0 += kTopkThreads, par ^= 1) {
    const int j = j0 + tid;
    const uint32_t k = j < P ? keys[j] & mask : 0u;
    const bool is_gt = j < P && k > T, is_eq = j < P && k == T;
    const uint64_t gm = __ballot(is_gt), em = __ballot(is_eq);
    if (lane == 0) ctot[par][w] = __builtin_popcountll(gm) | (__builtin_popcountll(em) << 16);
    __syncthreads();
    // both counts (< 2^16 each) scan together in one packed int
    const int ct = per_wave_value(ctot[par], lane);
    const int crun = row16_incl_scan(ct);
    const int excl = __builtin_amdgcn_readlane(crun, w) - __builtin_amdgcn_readlane(ct, w);
    const int total = __builtin_amdgcn_readlane(crun, kTopkWaves - 1);
    const int gt_w = excl & 0xFFFF, eq_w = excl >> 16, gt_r = total & 0xFFFF, eq_r = total >> 16;
    const int gt_before = gt_base + gt_w + lanes_below(gm);
    const int eq_before = eq_base + eq_w + lanes_below(em);
    // positions stay below K by construction; the guards keep every write
    // inside the row regardless
    const int pos_gt = gt_before + min(eq_before, need), pos_eq = gt_before + eq_before;
    if (is_gt && pos_gt < K) out[pos_gt] = j;
    else if (is_eq && eq_before < need && pos_eq < K) out[pos_eq] = j;
    gt_base += gt_r;
    eq_base += eq_r;
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
