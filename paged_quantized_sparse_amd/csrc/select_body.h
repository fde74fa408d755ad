// select_body.h -- the top-K page selection of one (sequence, KV head) row
// run by one block inside the attention kernel, so that selection costs no
// launch of its own.  It selects exactly what kvq_topk_pages selects
// ("TinyServe", lpnh.cn, section 3.1 phase 2; section 5.1 selection_ratio):
// the K largest scores, equal scores to the lower logical page, -0 == +0.
//
// Each block of the row repeats the selection (the row's scores are a few KB
// and stay in L2) and keeps only its own chunk: the selected pages of ranks
// first .. first+n-1 in ascending page order, which is exactly the slice of
// kvq_topk_pages' output the block would otherwise read.
//
// Method, as in topk_pages.hip but for a 256-thread block and with every key
// in registers: scores become order-preserving uint32 keys, thread t holding
// those of pages 8t .. 8t+7; all keys share the bits above the highest bit
// where the row's minimum and maximum key differ; MSB-first radix passes of
// up to 11 bits over the bits below (LDS histograms filled from the
// registers) find the K-th largest key's prefix and how many keys on it are
// still needed, stopping early once the chosen bin holds exactly that many.
// Every wave finds the chosen bin itself (two barriers per pass).  Ranks then
// come from each thread's counts of its 8 keys above and on the prefix, one
// wave scan and one block scan.  The code is kept short on purpose: it runs
// once per launch, so its instruction fetch is part of its latency.
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kSelBins = 2048;
static_assert(kSelMaxPages < 65536, "rank counts are packed in 16 bits");

constexpr int kSelKeys = kSelMaxPages / 256;  // keys per thread (pages 8t .. 8t+7)

// LDS of the selection (the caller allocates).
struct SelShared {
  int* hist;         // [2][kSelBins]
  int* wtot;         // [2][waves]
  uint32_t* wrange;  // [2][waves]
};

// Thread t's 8 scores (pages 8t .. 8t+7), loaded before the row length is
// known (indices clamped into the row of max_pages scores), so these loads
// are in flight with the kernel's other first loads; COH: at device scope,
// for scores other blocks of the same launch wrote.
template <int NT>
struct SelPrefetch {
  float v[kSelKeys];
  template <bool COH>
  __device__ __forceinline__ void load(const float* sc, int max_pages) {
#pragma unroll
    for (int u = 0; u < kSelKeys; ++u) v[u] = load_f<COH>(sc + min(kSelKeys * (int)threadIdx.x + u, max_pages - 1));
  }
};

// Writes out[0 .. n) = the selected pages of ranks first .. first+n-1, for a
// row of P <= kSelMaxPages pages of which K are selected (K < P; K >= P is
// the caller's).  Called by all NW * 64 threads of the block; ends with a
// barrier.
template <int NW>
__device__ __forceinline__ void select_chunk(const SelPrefetch<NW * 64>& pre, int P, int K, int first, int n,
                                             const SelShared& sm, int* out) {
  constexpr int NT = NW * 64;
  constexpr int BPT = kSelBins / NT;  // histogram bins per thread
  constexpr int U = kSelKeys;
  static_assert(BPT == 8 && NT * U == kSelMaxPages, "bins and keys per thread assume 256 threads");
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int j0 = U * tid;  // this thread's first page

  // ---- keys into registers, the key range, the first histogram zeroed
  uint32_t kr[U];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool valid = j0 + u < P;
    kr[u] = valid ? float_key(pre.v[u]) : 0u;
    kmin = valid ? min(kmin, kr[u]) : kmin;
    kmax = valid ? max(kmax, kr[u]) : kmax;
  }
  *(int4*)(sm.hist + BPT * tid) = make_int4(0, 0, 0, 0);
  *(int4*)(sm.hist + BPT * tid + 4) = make_int4(0, 0, 0, 0);
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    sm.wrange[w] = kmin;
    sm.wrange[NW + w] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    kmin = min(kmin, sm.wrange[x]);
    kmax = max(kmax, sm.wrange[NW + x]);
  }
  const int lead = kmax == kmin ? -1 : 31 - __builtin_clz(kmax ^ kmin);  // highest differing bit
  uint32_t mask = lead < 0 ? 0xFFFFFFFFu : (lead >= 31 ? 0u : ~((2u << lead) - 1u));
  uint32_t prefix = kmax & mask;
  int need = K;       // keys still to take among those on the prefix
  int hi_bit = lead;  // next bit to resolve
  int cur = 0;

#pragma unroll 1
  while (hi_bit >= 0) {
    const int bits = hi_bit + 1 < 11 ? hi_bit + 1 : 11;
    const int shift = hi_bit + 1 - bits;
    const int nbins = 1 << bits;
    int* h = sm.hist + cur * kSelBins;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j0 + u < P && (kr[u] & mask) == prefix) atomicAdd(&h[(kr[u] >> shift) & (nbins - 1)], 1);
    __syncthreads();
    // thread t owns bins lo .. lo+7 with lo = 2048 - 8(t+1): thread 0 the top
    // ones (bins at or above nbins stay empty); the next histogram is zeroed now
    const int lo = kSelBins - BPT * (tid + 1);
    const int4 a0 = *(const int4*)(h + lo), a1 = *(const int4*)(h + lo + 4);
    int* hn = sm.hist + (cur ^ 1) * kSelBins;
    *(int4*)(hn + lo) = make_int4(0, 0, 0, 0);
    *(int4*)(hn + lo + 4) = make_int4(0, 0, 0, 0);
    const int own = a0.x + a0.y + a0.z + a0.w + a1.x + a1.y + a1.z + a1.w;
    const int incl = wave_incl_scan_add(own);
    if (lane == 63) sm.wtot[cur * NW + w] = incl;
    __syncthreads();
    // every wave finds the crossing wave (the first whose running total
    // reaches need), then the crossing thread and bin, itself
    const int wt = lane < NW ? sm.wtot[cur * NW + lane] : 0;
    const int wrun = row16_incl_scan(wt);
    const uint64_t reach = __ballot(lane < NW && wrun >= need);
    const int wv = reach ? (int)__builtin_ctzll(reach) : NW - 1;
    const int before = __builtin_amdgcn_readlane(wrun, wv) - __builtin_amdgcn_readlane(wt, wv);
    const int lo2 = kSelBins - BPT * (64 * wv + lane + 1);  // this lane: bins of thread 64 wv + lane
    const int4 b0 = *(const int4*)(h + lo2), b1 = *(const int4*)(h + lo2 + 4);
    const int s2 = b0.x + b0.y + b0.z + b0.w + b1.x + b1.y + b1.z + b1.w;
    const int within = wave_incl_scan_add(s2);
    const int above = before + within - s2;
    const uint64_t hit = __ballot(above < need && above + s2 >= need);
    const int src = hit ? (int)__builtin_ctzll(hit) : 63;
    // the crossing thread's eight bins, from its top bin down (uniform values)
    const int cb[BPT] = {__builtin_amdgcn_readlane(b1.w, src), __builtin_amdgcn_readlane(b1.z, src),
                         __builtin_amdgcn_readlane(b1.y, src), __builtin_amdgcn_readlane(b1.x, src),
                         __builtin_amdgcn_readlane(b0.w, src), __builtin_amdgcn_readlane(b0.z, src),
                         __builtin_amdgcn_readlane(b0.y, src), __builtin_amdgcn_readlane(b0.x, src)};
    const int src_lo = kSelBins - BPT * (64 * wv + src + 1);
    int acc = __builtin_amdgcn_readlane(above, src);
    int digit = src_lo, cnt = cb[BPT - 1];
    bool found = false;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (!found && acc + cb[i] >= need) {
        found = true;
        digit = src_lo + BPT - 1 - i;
        cnt = cb[i];
      } else if (!found) {
        acc += cb[i];
      }
    }
    need -= acc;
    prefix |= (uint32_t)digit << shift;
    mask |= (uint32_t)(nbins - 1) << shift;
    hi_bit = shift - 1;
    cur ^= 1;
    if (cnt == need) break;  // uniform: the whole bin is taken
  }

  // ---- ranks.  Selected: every key whose resolved bits exceed the prefix,
  // and the first `need` (in page order) whose resolved bits equal it.  Each
  // thread counts both kinds among its 8 pages (packed in one int), a wave
  // scan and a block scan give the counts before its first page, and it walks
  // its pages in order.
  int gt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t k = kr[u] & mask;
    gt += j0 + u < P && k > prefix;
    eq += j0 + u < P && k == prefix;
  }
  const int packed = gt | (eq << 16);
  const int incl = wave_incl_scan_add(packed);
  if (lane == 63) sm.wtot[cur * NW + w] = incl;  // the buffer the last pass did not use
  __syncthreads();
  const int wt = lane < NW ? sm.wtot[cur * NW + lane] : 0;
  const int wrun = row16_incl_scan(wt);
  const int bef = __builtin_amdgcn_readlane(wrun, w) - __builtin_amdgcn_readlane(wt, w) + incl - packed;
  int gt_b = bef & 0xFFFF, eq_b = bef >> 16;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t k = kr[u] & mask;
    const bool valid = j0 + u < P;
    const bool is_gt = valid && k > prefix, is_eq = valid && k == prefix;
    const int rank = is_gt ? gt_b + min(eq_b, need) : (is_eq && eq_b < need ? gt_b + eq_b : -1);
    gt_b += is_gt;
    eq_b += is_eq;
    if (rank >= first && rank < first + n) out[rank - first] = j0 + u;
  }
  __syncthreads();
}

}  // namespace kvq
