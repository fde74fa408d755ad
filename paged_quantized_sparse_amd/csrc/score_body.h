// score_body.h -- the wave-level page scorer shared by page_scores.hip and the
// fused append + scores kernel.
//
// Page relevance ("TinyServe", lpnh.cn, section 2.1):
//   r(q, phi_j) = sum_i (q_i >= 0 ? q_i M_j[i] : q_i m_j[i]),
// which never underestimates q.k for any key of page j; written as
// sum_i max(q_i, 0) M_j[i] + min(q_i, 0) m_j[i], the same terms without a
// per-channel select.  For GQA the KV group's score is the max over its query
// heads, so it still bounds every member head's q.k.
//
// Layout per (physical page, KV head): meta[2][d] fp32 (min row, max row) =
// 8d bytes, read as one contiguous wave load: lanes 0-31 hold min-row
// channels, lanes 32-63 the max-row channels.  The query stays in registers.
#pragma once

#include "kvq_device.h"

namespace kvq {

constexpr int kScoreWaves = 4;
constexpr int kScorePagesPerWave = 8;

struct ScoreView {
  const float* meta;
  const int32_t* block_table;
  const uint16_t* q;
  float* scores;
  int H;
  int Hq;
  int max_pages;
};

// This lane's query coefficients: max(q, 0) on the max row, min(q, 0) on the min row.
template <int D, int G>
struct ScoreQuery {
  static constexpr int E = 2 * D / 64;  // floats per lane (4 for d = 128, 2 for d = 64)
  float qc[G][E];
  __device__ __forceinline__ void load(const ScoreView& a, int b, int g) {
    const int lane = lane_id();
    const bool max_row = lane >= 32;
    const int ch0 = (lane & 31) * E;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint16_t* qh = a.q + ((size_t)b * a.Hq + g * G + hh) * D + ch0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float x = half_bits_to_float(qh[e]);
        qc[hh][e] = max_row ? fmaxf(x, 0.0f) : fminf(x, 0.0f);
      }
    }
  }
};

// Score of one page from this lane's E metadata values: per head, an fma
// chain over the lane's values, a 64-lane sum, then the max over the G heads.
template <int D, int G>
__device__ __forceinline__ float score_from_values(const ScoreQuery<D, G>& q, const float* vals) {
  constexpr int E = ScoreQuery<D, G>::E;
  float best = -INFINITY;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float r = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) r = __builtin_fmaf(q.qc[hh][e], vals[e], r);
    r = sum_contig<64>(r);
    best = fmaxf(best, r);
  }
  return best;
}

// What one scoring item needs before its metadata can be loaded: the block-
// table entries of its 8 pages (lane k mod 8: page j0 + k, index clamped into
// the row), the sequence length, the append offsets and start (when rows are
// being appended) and this lane's raw fp16 query pairs.  All are vector loads
// left pending: a wave issues the next item's head while the current item's
// metadata loads are in flight.
template <int D, int G>
struct ScoreHead {
  static constexpr int E = ScoreQuery<D, G>::E;
  static constexpr int QW = G * E / 2;  // query dwords per lane
  int bt, len, o0, o1, start;
  uint32_t q[QW];
};

// Per-sequence arrays the scoring items read (new_off and start_pos only
// when rows are appended in the same launch).
struct ScoreSeqs {
  const int32_t* seq_lens;
  const int32_t* new_off;
  const int32_t* start_pos;
  int rows;  // B * H
};

template <int D, int G, bool APPEND>
__device__ __forceinline__ ScoreHead<D, G> score_head_load(const ScoreView& a, const ScoreSeqs& ss, int b, int g,
                                                           int j0) {
  constexpr int E = ScoreQuery<D, G>::E;
  ScoreHead<D, G> h;
  const int lane = lane_id();
  h.bt = a.block_table[(size_t)b * a.max_pages + min(j0 + (lane & 7), a.max_pages - 1)];
  h.len = vload_i32(ss.seq_lens, b);
  if constexpr (APPEND) {
    h.o0 = vload_i32(ss.new_off, b);
    h.o1 = vload_i32(ss.new_off, b + 1);
    h.start = vload_i32(ss.start_pos, b);
  } else {
    h.o0 = h.o1 = h.start = 0;
  }
  const int ch0 = (lane & 31) * E;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint16_t* qh = a.q + ((size_t)b * a.Hq + g * G + hh) * D + ch0;
    if constexpr (E == 4) {
      const uint2 v = *(const uint2*)qh;
      h.q[2 * hh] = v.x;
      h.q[2 * hh + 1] = v.y;
    } else {
      h.q[hh] = *(const uint32_t*)qh;
    }
  }
  return h;
}

// The query coefficients from a head's raw query, exactly as ScoreQuery::load.
template <int D, int G>
__device__ __forceinline__ ScoreQuery<D, G> score_query_of(const ScoreHead<D, G>& h) {
  constexpr int E = ScoreQuery<D, G>::E;
  ScoreQuery<D, G> q;
  const bool max_row = lane_id() >= 32;
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = half_bits_to_float((h.q[hh * E / 2 + e / 2] >> (16 * (e % 2))) & 0xFFFFu);
      q.qc[hh][e] = max_row ? fmaxf(x, 0.0f) : fminf(x, 0.0f);
    }
  return q;
}

// Persistent scoring: the calling wave takes items gw, gw + TW, ... of the
// rows * ceil(max_pages / 8) items (row-major: row = b * H + g, then 8-page
// chunks, so waves running at the same time read neighbouring pages).  For each item it scores pages below min(P, skip) (skip = the
// first page the appended rows touch, when APPEND), writes -inf for pages at
// or past P, and leaves pages in [skip, P) to the append block.  The next
// item's head is loaded while the current item's metadata is in flight, so a
// wave's loads never wait on a new block's first loads.  An item with no live
// page loads no metadata.
template <int D, int G, bool APPEND>
__device__ __forceinline__ void score_items(const ScoreView& a, const ScoreSeqs& ss, int gw, int TW) {
  constexpr int E = ScoreQuery<D, G>::E;
  const int nchunks = (a.max_pages + kScorePagesPerWave - 1) / kScorePagesPerWave;
  const int n_items = ss.rows * nchunks;
  if (gw >= n_items) return;
  const int lane = lane_id();
  auto head_of = [&](int item) {
    const int row = item / nchunks;
    return score_head_load<D, G, APPEND>(a, ss, row / a.H, row % a.H, (item % nchunks) * kScorePagesPerWave);
  };
  ScoreHead<D, G> nh = head_of(gw);
#pragma unroll 1
  for (int it = gw;;) {
    const ScoreHead<D, G> h = nh;
    const int row = it / nchunks, j0 = (it % nchunks) * kScorePagesPerWave;
    const int g = row % a.H;
    const int nxt = it + TW;
    const int nxt_c = min(nxt, n_items - 1);  // the last item's head is re-read, unused
    float* out = a.scores + (size_t)row * a.max_pages;
    const int P = (__builtin_amdgcn_readfirstlane(h.len) + kPage - 1) / kPage;
    int skip = P;
    if constexpr (APPEND) {
      const int n = min(__builtin_amdgcn_readfirstlane(h.o1) - __builtin_amdgcn_readfirstlane(h.o0), 64);
      const int st = __builtin_amdgcn_readfirstlane(h.start);
      skip = n > 0 ? min(st / kPage, P) : P;
    }
    const int live = skip;
    if (j0 < live) {  // wave-uniform
      float vals[kScorePagesPerWave][E];
#pragma unroll
      for (int k = 0; k < kScorePagesPerWave; ++k) {
        const int ph = j0 + k < live ? __builtin_amdgcn_readlane(h.bt, k) : 0;
        const float* m = a.meta + ((size_t)ph * a.H + g) * 2 * D + lane * E;
        if constexpr (E == 4) {
          const float4 v = load_stream_f4(m);
          vals[k][0] = v.x; vals[k][1] = v.y; vals[k][2] = v.z; vals[k][3] = v.w;
        } else {
          const float2 v = load_stream_f2(m);
          vals[k][0] = v.x; vals[k][1] = v.y;
        }
      }
      nh = head_of(nxt_c);
      const ScoreQuery<D, G> q = score_query_of<D, G>(h);
#pragma unroll
      for (int k = 0; k < kScorePagesPerWave; ++k) {
        const int j = j0 + k;
        if (j >= a.max_pages) break;
        if (j >= live && j < P) continue;
        const float best = j < live ? score_from_values<D, G>(q, vals[k]) : -INFINITY;
        if (lane == 0) out[j] = best;
      }
    } else {
      nh = head_of(nxt_c);
      const int j = j0 + lane;
      if (lane < kScorePagesPerWave && j >= P && j < a.max_pages) out[j] = -INFINITY;
    }
    if (nxt >= n_items) break;
    it = nxt;
  }
}

// Sequences the balanced mapping below indexes in LDS.
constexpr int kScoreMaxSeqs = 2048;

// LDS of the balanced mapping (the kernel declares it).
struct ScoreShared {
  int* pref;  // [kScoreMaxSeqs + 1]: live items before sequence b
  int* wsum;  // [kScoreWaves]
};

// Pages of sequence b the scoring waves score: those below its length P, or
// below the first page the rows appended in the same launch touch (exactly
// the `skip` of score_items), clamped into [0, max_pages] so that a length
// outside its documented range can neither write past the row nor break the
// prefix.
template <bool APPEND>
__device__ __forceinline__ int live_pages(const ScoreSeqs& ss, int b, int max_pages) {
  const int P = (ss.seq_lens[b] + kPage - 1) / kPage;
  int live = P;
  if constexpr (APPEND) {
    const int n = min(ss.new_off[b + 1] - ss.new_off[b], 64);
    live = n > 0 ? min(ss.start_pos[b] / kPage, P) : P;
  }
  return min(max(live, 0), max_pages);
}

// Whether a persistent scoring grid of TW waves over B = rows / H sequences
// takes the balanced mapping: a ragged batch leaves score_items' fixed
// stride with some waves all of whose items are live and others with none,
// and the most loaded waves set the launch's time.  Decided by the launcher.
__host__ __device__ __forceinline__ bool score_balanced(int rows, int H, int max_pages, int TW) {
  const int B = rows / H;
  const long long items = (long long)rows * ((max_pages + kScorePagesPerWave - 1) / kScorePagesPerWave);
  return B > 1 && B <= kScoreMaxSeqs && items > TW;
}

// Persistent scoring over the live items only.  Every block builds in LDS
// the prefix over sequences of (live 8-page chunks) x H items, sequence-
// major as score_items orders them; wave gw takes the contiguous items
// [gw T / TW, (gw+1) T / TW) of the T live ones, so waves get equal work
// however ragged the batch is.  Pages at or past each row's length get their
// -inf first, rows dealt round-robin to the waves; pages in [skip, P) are the
// append block's.  Each score is computed as in score_items.  Called by all
// threads of the block (it has barriers).
template <int D, int G, bool APPEND>
__device__ __forceinline__ void score_items_balanced(const ScoreView& a, const ScoreSeqs& ss, int gw, int TW,
                                                     const ScoreShared& sm) {
  constexpr int E = ScoreQuery<D, G>::E;
  constexpr int SPT = kScoreMaxSeqs / (kScoreWaves * 64);  // sequences per thread
  const int H = a.H;
  const int B = ss.rows / H;
  const int lane = lane_id(), w = wave_id();

  // ---- -inf past each row's length (stores only)
  for (int r = gw; r < ss.rows; r += TW) {
    const int P = (__builtin_amdgcn_readfirstlane(vload_i32(ss.seq_lens, r / H)) + kPage - 1) / kPage;
    float* out = a.scores + (size_t)r * a.max_pages;
    for (int j = max(P, 0) + lane; j < a.max_pages; j += kWave) out[j] = -INFINITY;
  }

  // ---- prefix of live items over the sequences (thread t: sequences
  // SPT t .. SPT t + SPT-1)
  int cnt[SPT];
  int own = 0;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int b = SPT * (int)threadIdx.x + i;
    cnt[i] = b < B ? (live_pages<APPEND>(ss, b, a.max_pages) + kScorePagesPerWave - 1) / kScorePagesPerWave * H : 0;
    own += cnt[i];
  }
  const int incl = wave_incl_scan_add(own);
  if (lane == kWave - 1) sm.wsum[w] = incl;
  __syncthreads();
  int run = incl - own;
#pragma unroll
  for (int x = 0; x < kScoreWaves; ++x) run += x < w ? sm.wsum[x] : 0;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int b = SPT * (int)threadIdx.x + i;
    if (b < B) sm.pref[b] = run;
    run += cnt[i];
  }
  if (threadIdx.x == kScoreWaves * kWave - 1) sm.pref[B] = run;  // the total
  __syncthreads();
  const int total = sm.pref[B];
  const int lo = (int)((long long)gw * total / TW), hi = (int)((long long)(gw + 1) * total / TW);
  if (lo >= hi) return;

  // ---- the sequence of item lo: the last b with pref[b] <= lo (pref is
  // non-decreasing), in two ballot rounds over B <= 64 * 64 entries
  const int stride = (B + kWave - 1) / kWave;
  const uint64_t r1 = __ballot(lane * stride < B && sm.pref[min(lane * stride, B - 1)] <= lo);
  const int seg = (63 - __builtin_clzll(r1)) * stride;  // r1 has lane 0 (pref[0] = 0 <= lo)
  const uint64_t r2 = __ballot(lane < stride && seg + lane < B && sm.pref[min(seg + lane, B - 1)] <= lo);
  int b = seg + (63 - __builtin_clzll(r2));
  auto chunks_of = [&](int bb) { return (sm.pref[bb + 1] - sm.pref[bb]) / H; };
  int nc = chunks_of(b);
  int g = (lo - sm.pref[b]) / nc, c = (lo - sm.pref[b]) % nc;
  // the item after (b, g, c) in the same order
  auto step = [&](int& bb, int& gg, int& cc, int& ncc) {
    if (++cc < ncc) return;
    cc = 0;
    if (++gg < H) return;
    gg = 0;
    do {
      ++bb;
    } while (bb < B - 1 && sm.pref[bb + 1] == sm.pref[bb]);
    ncc = chunks_of(min(bb, B - 1));
  };
  ScoreHead<D, G> nh = score_head_load<D, G, APPEND>(a, ss, b, g, c * kScorePagesPerWave);
#pragma unroll 1
  for (int it = lo; it < hi; ++it) {
    const ScoreHead<D, G> h = nh;
    const int cb = b, cg = g, j0 = c * kScorePagesPerWave;
    float* out = a.scores + ((size_t)cb * H + cg) * a.max_pages;
    const int P = (__builtin_amdgcn_readfirstlane(h.len) + kPage - 1) / kPage;
    int live = P;
    if constexpr (APPEND) {
      const int n = min(__builtin_amdgcn_readfirstlane(h.o1) - __builtin_amdgcn_readfirstlane(h.o0), 64);
      const int st = __builtin_amdgcn_readfirstlane(h.start);
      live = n > 0 ? min(st / kPage, P) : P;
    }
    live = min(max(live, 0), a.max_pages);  // as live_pages counts it
    float vals[kScorePagesPerWave][E];
#pragma unroll
    for (int k = 0; k < kScorePagesPerWave; ++k) {
      const int ph = j0 + k < live ? __builtin_amdgcn_readlane(h.bt, k) : 0;
      const float* m = a.meta + ((size_t)ph * H + cg) * 2 * D + lane * E;
      if constexpr (E == 4) {
        const float4 v = load_stream_f4(m);
        vals[k][0] = v.x; vals[k][1] = v.y; vals[k][2] = v.z; vals[k][3] = v.w;
      } else {
        const float2 v = load_stream_f2(m);
        vals[k][0] = v.x; vals[k][1] = v.y;
      }
    }
    // the next item's head (the last item re-reads its own, unused)
    if (it + 1 < hi) step(b, g, c, nc);
    nh = score_head_load<D, G, APPEND>(a, ss, b, g, c * kScorePagesPerWave);
    const ScoreQuery<D, G> q = score_query_of<D, G>(h);
#pragma unroll
    for (int k = 0; k < kScorePagesPerWave; ++k) {
      const int j = j0 + k;
      if (j >= live) break;
      const float best = score_from_values<D, G>(q, vals[k]);
      if (lane == 0) out[j] = best;
    }
  }
}

// Blocks of `kernel` (256 threads) the current device keeps resident at
// once, or 0 if that cannot be queried.  Launchers look it up once, into a
// function-local static (initialized once even with concurrent callers).
inline int resident_blocks(const void* kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kScoreWaves * 64, 0) != hipSuccess ||
      cus < 1 || per_cu < 1)
    return 0;
  return cus * per_cu;
}

// Blocks of a scoring grid: one wave per item when that fits in `capacity`
// resident blocks; otherwise a persistent grid of the capacity less
// `reserved` blocks launched ahead of it (but at least half the capacity).
// 0 if the capacity is unknown.
inline int score_grid_blocks(int capacity, int items, int reserved) {
  if (capacity < 1) return 0;
  const int want = (items + kScoreWaves - 1) / kScoreWaves;
  if (want <= capacity) return want;
  return capacity - reserved > capacity / 2 ? capacity - reserved : capacity / 2;
}

}  // namespace kvq
