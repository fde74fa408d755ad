// decode_step.hip -- the whole decode step in one persistent launch: append
// the newest rows and refresh their pages' metadata, score every page, select
// the top-K pages of every (sequence, KV head) row and attend to them, then
// merge the splits ("TinyServe", lpnh.cn, section 3.1: the four phases of the
// fused sparse-attention kernel; section 5.2: launch overhead).
//
// The work is a list of items over the rows r = b * H_kv + g:
//   the append item of row r: the rows appended to sequence b for head g,
//     the metadata of the pages they touch and those pages' scores
//     (append_body.h);
//   A items of row r: one scoring item per 32 pages below the first touched
//     page (4 waves x 8 pages: score_body.h's scorer);
//   B items of row r: one per split of the row's selected pages (the
//     in-kernel selection and the split's attention: attn_body.h); the block
//     that finishes a row's last split merges the row's splits.
// The list holds every append item first, then groups of rows in the order
// A(0) A(1) B(0) A(2) B(1) ... B(n-1), so a group's selections (latency, no
// HBM traffic) run while the next group's metadata streams.  Block i of the
// persistent grid takes items i, i + NB, i + 2 NB, ... in that order.  A B
// item waits (a bounded spin) until its row's append and A items, and every
// append item of its sequence, have finished.  Every item anyone waits for
// comes earlier in the list than the waiter, so the earliest unfinished item
// can always run and the grid (at most the resident capacity) drains.
//
// Data one block writes and another reads in the same launch -- scores,
// partials, the appended codes, scale/zero and metadata -- goes through
// device-scope (written-through) stores and device-scope loads; counters are
// device-scope atomics.  After its stores an append item invalidates its L2
// (an agent-scope acquire), so no line it read before another head's append
// of the same page stays stale there; B items of a sequence start only after
// all of its append items have finished.
//
// Counters live in the workspace, one 128-byte line per row and per sequence:
// atomics on one line are serialized (~50 ns each), so counters that share a
// line, or one counter every block bumps, would cost more than the step.  The
// block that merges a row resets that row's counters (every item that reads
// them is done by then), and the last row of a sequence to be merged resets
// the sequence's, so every launch finds them zero (the caller zeroes them
// once, when the workspace is allocated).
#include "append_body.h"
#include "attn_body.h"
#include "score_body.h"

namespace kvq {
namespace {

constexpr int kStepPagesPerItem = kScoreWaves * kScorePagesPerWave;  // 32 pages per scoring item
constexpr int kStepGroups = 8;            // row groups the item list interleaves (at most)
constexpr int kStepMaxSpins = 1 << 21;    // bound of a wait (each poll ~1 us): far beyond any real wait

struct StepArgs {
  AttnArgs at;       // attention: the row scores, selection rule, partials, output
  AppendView ap;     // append of the newest rows
  ScoreView sc;      // scoring
  int* ctr;          // line 0: [1] error (a wait ran out); then one line per row r
                     // (A_done, B_done) and one per sequence b (appended, rows_done)
  int B, R, rows_per_group, ngroups, nblocks;
};

constexpr int kCtrLine = 32;  // ints per 128-byte line

// Item counts of sequence b: A items per row (scoring chunks below the first
// touched page) and B items per row (splits).
struct SeqCounts {
  int nA, nB;
};

__device__ __forceinline__ SeqCounts seq_counts(const StepArgs& a, int b) {
  const int len = a.at.seq_lens[b];
  const int P = min(max((len + kPage - 1) / kPage, 0), a.at.max_pages);
  const int n = min(a.ap.new_off[b + 1] - a.ap.new_off[b], 64);
  const int live = n > 0 ? min(max(a.ap.start_pos[b] / kPage, 0), P) : P;
  const int K = num_selected(P, a.at.rnum, a.at.rden, a.at.k_fixed);
  return {(live + kStepPagesPerItem - 1) / kStepPagesPerItem, (K + a.at.pps - 1) / a.at.pps};
}

// Device-scope counter helpers.
__device__ __forceinline__ int ctr_load(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ctr_add(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int D, int G>
__global__ __launch_bounds__(256) void decode_step_kernel(StepArgs a) {
  constexpr int NW = kAttnWaves;
  __shared__ int sm_pa[kStepMaxSeqs + 1], sm_pb[kStepMaxSeqs + 1];  // A / B items before sequence b, x H
  __shared__ int sm_na[kStepMaxSeqs], sm_nb[kStepMaxSeqs];          // per row of sequence b
  __shared__ int sm_seg[2 * kStepGroups + 2];                       // item list: start of each segment
  __shared__ int sm_segk[2 * kStepGroups + 1];                      // its kind: group (+ 1 << 16: B; -1: appends)
  __shared__ int sm_flag;
  __shared__ int sm_list[kStepMaxSplitPages];                       // a B item's pages
  __shared__ float sm_meta[kMaxTouched][2][D];                      // an append item's new metadata
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int H = a.at.H;
  auto row_ctr = [&](int r) { return a.ctr + kCtrLine * (1 + r); };          // [0] A_done, [1] B_done
  auto seq_ctr = [&](int b) { return a.ctr + kCtrLine * (1 + a.R + b); };    // [0] appended, [1] rows_done

  // ---- item counts per sequence and their prefix (sequence-major; each of
  // a sequence's H rows has the same counts)
  for (int b = tid; b < a.B; b += NW * 64) {
    const SeqCounts c = seq_counts(a, b);
    sm_na[b] = c.nA;
    sm_nb[b] = c.nB;
  }
  __syncthreads();
  if (w == 0) {  // one wave scans the sequences, 64 at a time
    int runA = 0, runB = 0;
    for (int b0 = 0; b0 < a.B; b0 += kWave) {
      const int b = b0 + lane;
      const int xa = b < a.B ? sm_na[b] * H : 0, xb = b < a.B ? sm_nb[b] * H : 0;
      const int ia = wave_incl_scan_add(xa), ib = wave_incl_scan_add(xb);
      if (b < a.B) {
        sm_pa[b] = runA + ia - xa;
        sm_pb[b] = runB + ib - xb;
      }
      runA += __builtin_amdgcn_readlane(ia, kWave - 1);
      runB += __builtin_amdgcn_readlane(ib, kWave - 1);
    }
    if (lane == 0) {
      sm_pa[a.B] = runA;
      sm_pb[a.B] = runB;
    }
  }
  __syncthreads();
  // items before row r in A (or B) order: rows are sequence-major
  auto before = [&](const int* pref, const int* per, int r) {
    const int b = min(r / H, a.B);
    return pref[b] + (b < a.B ? (r - b * H) * per[b] : 0);
  };
  if (tid == 0) {  // segment starts of the list: appends, A(0) A(1) B(0) A(2) B(1) ... B(n-1)
    int pos = a.R, k = 1;
    sm_segk[0] = -1;
    sm_seg[0] = 0;
    for (int i = 0; i <= a.ngroups; ++i) {
      if (i < a.ngroups) {  // A(i)
        sm_segk[k] = i;
        sm_seg[k++] = pos;
        const int r0 = i * a.rows_per_group, r1 = min(a.R, r0 + a.rows_per_group);
        pos += before(sm_pa, sm_na, r1) - before(sm_pa, sm_na, r0);
      }
      if (i >= 1) {  // B(i-1)
        sm_segk[k] = (i - 1) | (1 << 16);
        sm_seg[k++] = pos;
        const int r0 = (i - 1) * a.rows_per_group, r1 = min(a.R, r0 + a.rows_per_group);
        pos += before(sm_pb, sm_nb, r1) - before(sm_pb, sm_nb, r0);
      }
    }
    sm_seg[k] = pos;
  }
  __syncthreads();
  const int nseg = 2 * a.ngroups + 1, total = sm_seg[nseg];

  // ---- the append item of row r: the rows, the touched pages' metadata and their scores
  auto append_item = [&](int r) {
    const int b = r / H, g = r % H;
    const int row = r;
    const int len = vload_i32(a.at.seq_lens, b);
    const int off0 = vload_i32(a.ap.new_off, b), off1 = vload_i32(a.ap.new_off, b + 1);
    const int start = __builtin_amdgcn_readfirstlane(vload_i32(a.ap.start_pos, b));
    ScoreQuery<D, G> q;
    q.load(a.sc, b, g);
    const int P = min((__builtin_amdgcn_readfirstlane(len) + kPage - 1) / kPage, a.sc.max_pages);
    const int n = min(__builtin_amdgcn_readfirstlane(off1) - __builtin_amdgcn_readfirstlane(off0), 64);
    const int first = start / kPage;
    const int count = n > 0 ? (start + n - 1) / kPage - first + 1 : 0;
    if (count > 0 && P > 0) {  // block-uniform
      append_rows_and_meta<FMT, D, true>(a.ap, b, g, sm_meta);
      if (w == 0) {
        constexpr int E = ScoreQuery<D, G>::E;
        float* out = a.sc.scores + (size_t)row * a.sc.max_pages;
        for (int p = 0; p < count && first + p < P; ++p) {
          const float best = score_from_values<D, G>(q, &sm_meta[p][0][0] + lane * E);
          if (lane == 0) store_f<true>(out + first + p, best);
        }
      }
    }
    if (P == 0) {  // an empty sequence: nothing selected, zero output
      for (int e = tid; e < G * D; e += NW * 64) a.at.out[((size_t)b * a.at.Hq + g * G) * D + e] = 0.0f;
      if (a.at.sel_out) {
        for (int i = tid; i < a.at.k_cap; i += NW * 64) a.at.sel_out[(size_t)row * a.at.k_cap + i] = -1;
        if (tid == 0) a.at.cnt_out[row] = 0;
      }
    }
    stores_done();
    // drop from this XCD's L2 any line read here before another head's
    // append of the same page wrote it (the readers wait for all heads)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
    if (tid == 0 && P > 0) {  // an empty sequence has no split waiting for it
      ctr_add(row_ctr(row), 1);
      ctr_add(seq_ctr(b), 1);
    }
  };

  for (int it = blockIdx.x; it < total; it += a.nblocks) {
    // ---- decode the item: segment, then (row, index) by a two-round ballot
    // search over the sequences' prefix
    int seg = 0;
    while (seg + 1 < nseg && sm_seg[seg + 1] <= it) ++seg;  // at most 2 * kStepGroups + 1 steps, uniform
    if (seg == 0) {
      append_item(it);
      continue;
    }
    const bool isA = sm_segk[seg] < (1 << 16);
    const int grp = sm_segk[seg] & 0xFFFF;
    const int* pref = isA ? sm_pa : sm_pb;
    const int* per = isA ? sm_na : sm_nb;
    const int x = before(pref, per, grp * a.rows_per_group) + (it - sm_seg[seg]);  // index in A (or B) order
    const int stride = (a.B + kWave - 1) / kWave;
    const uint64_t r1 = __ballot(lane * stride < a.B && pref[min(lane * stride, a.B - 1)] <= x);
    const int base = (63 - __builtin_clzll(r1)) * stride;
    const uint64_t r2 = __ballot(lane < stride && base + lane < a.B && pref[min(base + lane, a.B - 1)] <= x);
    int b = base + (63 - __builtin_clzll(r2));
    while (b + 1 < a.B && pref[b + 1] <= x) ++b;  // skip sequences with no items (uniform)
    const int n_row = per[b];
    const int g = (x - pref[b]) / n_row, idx = (x - pref[b]) % n_row;
    const int row = b * H + g;

    if (isA) {
      // ---- scoring item: pages [32 idx, 32 idx + 32) below the first touched page
      const ScoreSeqs ss{a.at.seq_lens, a.ap.new_off, a.ap.start_pos, a.R};
      const int j0 = idx * kStepPagesPerItem + w * kScorePagesPerWave;
      const ScoreHead<D, G> h = score_head_load<D, G, true>(a.sc, ss, b, g, j0);
      constexpr int E = ScoreQuery<D, G>::E;
      const int P = min((__builtin_amdgcn_readfirstlane(h.len) + kPage - 1) / kPage, a.sc.max_pages);
      const int nr = min(__builtin_amdgcn_readfirstlane(h.o1) - __builtin_amdgcn_readfirstlane(h.o0), 64);
      const int st = __builtin_amdgcn_readfirstlane(h.start);
      const int live = max(nr > 0 ? min(st / kPage, P) : P, 0);
      if (j0 < live) {  // wave-uniform
        float vals[kScorePagesPerWave][E];
#pragma unroll
        for (int k = 0; k < kScorePagesPerWave; ++k) {
          const int ph = j0 + k < live ? __builtin_amdgcn_readlane(h.bt, k) : 0;
          const float* m = a.sc.meta + ((size_t)ph * H + g) * 2 * D + lane * E;
          if constexpr (E == 4) {
            const float4 v = load_stream_f4(m);
            vals[k][0] = v.x; vals[k][1] = v.y; vals[k][2] = v.z; vals[k][3] = v.w;
          } else {
            const float2 v = load_stream_f2(m);
            vals[k][0] = v.x; vals[k][1] = v.y;
          }
        }
        const ScoreQuery<D, G> q = score_query_of<D, G>(h);
        float* out = a.sc.scores + (size_t)row * a.sc.max_pages;
#pragma unroll
        for (int k = 0; k < kScorePagesPerWave; ++k) {
          const int j = j0 + k;
          if (j >= live) break;
          const float best = score_from_values<D, G>(q, vals[k]);
          if (lane == 0) store_f<true>(out + j, best);
        }
      }
      stores_done();
      __syncthreads();
      if (tid == 0) ctr_add(row_ctr(row), 1);
    } else {
      // ---- split idx of row (b, g): wait for the row's scores and the
      // sequence's appends, then select, attend, and merge if last
      if (tid == 0) {
        const int needA = sm_na[b] + 1;  // the scoring items and the append item
        int spins = 0;
        while (ctr_load(row_ctr(row)) < needA || ctr_load(seq_ctr(b)) < H) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins > kStepMaxSpins) {
            __hip_atomic_store(a.ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      }
      __syncthreads();
      attend_split<FMT, D, G, NW, true, true>(a.at, g, b, idx, sm_list);
      if (tid == 0) sm_flag = ctr_add(row_ctr(row) + 1, 1) == sm_nb[b] - 1;
      __syncthreads();
      if (sm_flag) {  // this block finished the row's last split: merge them
#pragma unroll 1
        for (int hh = 0; hh < G; ++hh) combine_one<D, G, true>(a.at, b * a.at.Hq + g * G + hh);
        if (tid == 0) {  // every item that reads this row's counters is done: reset them
          store_u32<true>((uint32_t*)row_ctr(row), 0u);
          store_u32<true>((uint32_t*)row_ctr(row) + 1, 0u);
          if (ctr_add(seq_ctr(b) + 1, 1) == H - 1) {  // and the sequence's, after its last row
            store_u32<true>((uint32_t*)seq_ctr(b), 0u);
            store_u32<true>((uint32_t*)seq_ctr(b) + 1, 0u);
          }
        }
      }
    }
  }
}

template <int FMT, int D, int G>
hipError_t run(const StepArgs& a0, int total_rows, hipStream_t st) {
  static std::atomic<long long> memo[kMaxDevices];
  const int capacity = (int)per_device(
      memo, [] { return resident_blocks(reinterpret_cast<const void*>(&decode_step_kernel<FMT, D, G>)); });
  if (capacity < 1) return hipErrorInvalidConfiguration;
  StepArgs a = a0;
  a.nblocks = capacity;  // a persistent grid that is resident at once
  (void)total_rows;
  hipLaunchKernelGGL((decode_step_kernel<FMT, D, G>), dim3(a.nblocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int FMT, int D>
hipError_t run_g(const StepArgs& a, int R, int G, hipStream_t st) {
  switch (G) {
    case 1: return run<FMT, D, 1>(a, R, st);
    case 2: return run<FMT, D, 2>(a, R, st);
    case 4: return run<FMT, D, 4>(a, R, st);
    default: return run<FMT, D, 8>(a, R, st);
  }
}

template <int FMT>
hipError_t run_d(const StepArgs& a, int D, int R, int G, hipStream_t st) {
  return D == 64 ? run_g<FMT, 64>(a, R, G, st) : run_g<FMT, 128>(a, R, G, st);
}

}  // namespace

size_t step_counter_bytes(int batch, int rows) {
  return (size_t)(1 + rows + batch) * kCtrLine * sizeof(int);
}

hipError_t launch_decode_step(const kvq_cache& c, const kvq_seqs& s, const int32_t* start_pos,
                              const int32_t* new_off, const uint16_t* k_new, const uint16_t* v_new,
                              const uint16_t* q, int num_q_heads, float* scores, int rnum, int rden, int k_fixed,
                              int k_cap, int32_t* sel_pages, int32_t* sel_count, float sm_scale,
                              int pages_per_split, int max_splits, float* out, void* ws, hipStream_t st) {
  const int R = s.batch * c.num_kv_heads;
  int* ctr = (int*)ws;
  const size_t n_part = (size_t)s.batch * num_q_heads * max_splits;
  float* part_ml = (float*)((char*)ws + step_counter_bytes(s.batch, R));
  float* part_acc = part_ml + n_part * 2;
  StepArgs a{};
  a.at = AttnArgs{c.k_pages, c.v_pages, c.kv_params, s.block_table, s.seq_lens, q, nullptr, nullptr,
                  scores, sel_pages, sel_count, rnum, rden, k_fixed, part_acc, part_ml, out,
                  c.num_kv_heads, num_q_heads, s.max_pages, k_cap, pages_per_split, max_splits,
                  sm_scale * 1.4426950408889634f};
  a.ap = AppendView{c.k_pages, c.v_pages, c.kv_params, c.page_meta, s.block_table, start_pos, new_off,
                    k_new, v_new, c.num_kv_heads, s.max_pages};
  a.sc = ScoreView{c.page_meta, s.block_table, q, scores, c.num_kv_heads, num_q_heads, s.max_pages};
  a.ctr = ctr;
  a.B = s.batch;
  a.R = R;
  a.ngroups = R < kStepGroups ? R : kStepGroups;
  a.rows_per_group = (R + a.ngroups - 1) / a.ngroups;
  a.ngroups = (R + a.rows_per_group - 1) / a.rows_per_group;
  const int G = num_q_heads / c.num_kv_heads;
  if (c.format == KVQ_FP16) return run_d<kFp16>(a, c.head_dim, R, G, st);
  if (c.format == KVQ_INT8_TOKEN) return run_d<kInt8Token>(a, c.head_dim, R, G, st);
  return run_d<kInt8Group>(a, c.head_dim, R, G, st);
}

}  // namespace kvq
