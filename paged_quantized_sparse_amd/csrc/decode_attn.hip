// decode_attn.hip -- single-token attention over the selected pages of a
// paged, optionally INT8, KV cache ("TinyServe", lpnh.cn, section 3.1 phases
// 3-4: load only the selected pages' KV, then reduce; attention itself is
// softmax(q k^T / sqrt(d)) v, intelliparadigm.com KV-cache page, section 2.1).
//
// Split-K: block (split s, KV head g, sequence b) takes selected pages
// [s*PPS, (s+1)*PPS) of row (b, g); its waves take every NW-th page.  A wave
// holds a whole (page, KV head) tile in flight as 16-byte loads: for a token
// row of RB = d * elem bytes, LPT = RB/16 lanes share a token, so one load
// instruction covers TPL = 64/LPT tokens, and NL = 16/TPL loads cover the page.
// The next tile's loads are issued before the current tile is consumed.
//
// Keys: q.k runs on v_dot2_f32_f16 with the fp16 query.  An INT8 code c
// becomes the fp16 value 1024 + c with one byte permute (0x64 is the high byte
// of 1024.0h), so for per-token or per-group (scale s, zero z)
//   q.k = s * sum q_i (1024 + c_i) + (z - 1024 s) * sum q_i.
// Values: acc += (p s) * c per channel (byte converts + fma), plus p z once per
// token.  The G query heads of a KV group share every loaded tile.
//
// Online softmax per lane (exp2 domain): each lane keeps the running max m of
// the tokens it saw and rescales only when a logit exceeds m by more than
// kLazy (weights stay below 2^kLazy), so the inner loop needs no cross-lane
// max.  Lanes, then waves, merge with log-sum-exp weights; each block writes a
// partial (m, l, acc) per query head and split, and combine_kernel merges a
// row's splits.  (Merging in the last-arriving split block instead needs a
// device-scope release per block, which on gfx950 writes back the XCD's L2
// each time and costs far more than a second launch.)
//
// The SEL instances select the block's pages themselves (select_body.h) from
// the row's scores instead of reading a selection: every block of the row
// repeats the row's top-K and keeps the pages of its split's ranks.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "select_body.h"

namespace kvq {
namespace {

#ifndef KVQ_ATTN_PREFETCH
#define KVQ_ATTN_PREFETCH 2
#endif
constexpr int kAttnWaves = 4;
constexpr int kPrefetch = KVQ_ATTN_PREFETCH;  // tiles in flight ahead of the one being consumed
constexpr float kLazy = 8.0f;

struct AttnArgs {
  const void* k_pages;
  const void* v_pages;
  const float* params;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint16_t* q;
  const int32_t* sel_pages;  // NULL: all pages (or selection in the kernel, below)
  const int32_t* sel_count;
  const float* scores;       // [B][H][max_pages]: select in the kernel (the SEL instances)
  int32_t* sel_out;          // optional copies of that selection, as kvq_topk_pages writes it
  int32_t* cnt_out;
  int rnum, rden, k_fixed;   // its selection rule
  float* part_acc;    // [B][Hq][max_splits][D]
  float* part_ml;     // [B][Hq][max_splits][2]
  float* out;         // [B][Hq][D]
  int H;
  int Hq;
  int max_pages;
  int k_cap;
  int pps;  // pages per split
  int max_splits;
  float scale_log2;  // sm_scale * log2(e)
};

template <int FMT, int D>
struct Tile {
  static constexpr int ELEM = FMT == kFp16 ? 2 : 1;
  static constexpr int RB = D * ELEM;
  static constexpr int LPT = RB / 16;     // lanes per token
  static constexpr int TPL = 64 / LPT;    // tokens per load
  static constexpr int NL = kPage / TPL;  // loads per page
  static constexpr int CH = 16 / ELEM;    // channels per lane
};

__device__ __forceinline__ float byte_to_float(uint32_t w, int i) { return (float)((w >> (8 * i)) & 0xFFu); }

__device__ __forceinline__ half2v as_half2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// grid (B * Hq), 256 threads: out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
// with M = max_s m_s.  Thread (part, c) takes channel c of splits part,
// part + PARTS, ...: it loads eight splits' (m, l, acc) at once (indices past
// the row's splits re-read its last split and are masked), together with the
// split count, and merges them online; the PARTS partial merges then meet in
// LDS.  So the block waits on one round of loads, not two.
template <int D, int G>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  constexpr int PARTS = 256 / D;
  constexpr int U = 8;  // splits in flight per thread
  __shared__ float sm_m[PARTS][D], sm_num[PARTS][D], sm_den[PARTS][D];
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int row = b * a.H + h / G;
  const int tid = threadIdx.x;
  const int c = tid % D, part = tid / D;
  const float* ml = a.part_ml + (size_t)bh * a.max_splits * 2;
  const float* pa = a.part_acc + (size_t)bh * a.max_splits * D;
  const int32_t* cnt_p = a.sel_pages ? a.sel_count + row : a.seq_lens + b;  // a select, not a branch
  const int cnt_v = vload_i32(cnt_p, 0);
  float2 mlv[U];
  float av[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {  // speculative: the first U splits of this part
    const int sp = min(part + u * PARTS, a.max_splits - 1);
    mlv[u] = *(const float2*)(ml + 2 * sp);
    av[u] = pa[(size_t)sp * D + c];
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the count is waited for
  // with every page selected cnt_p points at the length, so K = P either way
  // (using the value on both paths keeps the load where it is issued)
  const int cnt = __builtin_amdgcn_readfirstlane(cnt_v);
  const int Pc = (cnt + kPage - 1) / kPage;
  const int K = a.sel_pages ? cnt : (a.scores ? num_selected(Pc, a.rnum, a.rden, a.k_fixed) : Pc);
  const int ns = (K + a.pps - 1) / a.pps;
  float M = -INFINITY, num = 0.0f, den = 0.0f;
  for (int s0 = 0;; s0 += U * PARTS) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float ms = s0 + part + u * PARTS < ns ? mlv[u].x : -INFINITY;
      const float Mn = fmaxf(M, ms);
      const float fo = M == -INFINITY ? 0.0f : exp2f(M - Mn);
      const float fs = ms == -INFINITY ? 0.0f : exp2f(ms - Mn);
      num = __builtin_fmaf(fs, av[u], num * fo);
      den = __builtin_fmaf(fs, mlv[u].y, den * fo);
      M = Mn;
    }
    if (s0 + U * PARTS >= ns) break;  // block-uniform
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = min(s0 + U * PARTS + part + u * PARTS, a.max_splits - 1);
      mlv[u] = *(const float2*)(ml + 2 * sp);
      av[u] = pa[(size_t)sp * D + c];
    }
  }
  sm_m[part][c] = M;
  sm_num[part][c] = num;
  sm_den[part][c] = den;
  __syncthreads();
  if (part == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int p = 0; p < PARTS; ++p) Mt = fmaxf(Mt, sm_m[p][c]);
    float n = 0.0f, dd = 0.0f;
#pragma unroll
    for (int p = 0; p < PARTS; ++p) {
      const float f = sm_m[p][c] == -INFINITY ? 0.0f : exp2f(sm_m[p][c] - Mt);
      n = __builtin_fmaf(f, sm_num[p][c], n);
      dd = __builtin_fmaf(f, sm_den[p][c], dd);
    }
    a.out[(size_t)bh * D + c] = dd > 0.0f ? n / dd : 0.0f;
  }
}

// SEL: the block selects its pages itself (select_body.h) from a.scores.
template <int FMT, int D, int G, int NW, bool SEL>
__global__ __launch_bounds__(NW * 64) void decode_attn_kernel(AttnArgs a) {
  static_assert(NW == 4, "the split merge and the combine assume 4 waves");
  using T = Tile<FMT, D>;
  constexpr int LPT = T::LPT, TPL = T::TPL, NL = T::NL, CH = T::CH;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int row = b * a.H + g;
  const int first = s * a.pps;
  const int w = wave_id();
  const int lane = lane_id();
  // Prologue, three levels of dependent loads.  Level 1, issued together and
  // unconditionally: this lane's selection slot (first + w + lane * NW, the
  // wave's first 64 pages), the sequence length, the selected count and the
  // query.  Level 2: the block-table entry of the slot's page.  Level 3: the
  // first tiles.  Indices are clamped into their arrays, so a slot past the
  // row's count reads some entry of the row and is never used; with no
  // selection (all pages) the slot load reads the block table and is replaced
  // by the slot index itself.
  // With in-kernel selection, level 1 carries the row's first scores
  // instead of the selection slot, and the slot comes from LDS after the
  // selection.
  const bool sparse = !SEL && a.sel_pages != nullptr;
  const int idx0 = first + w + lane * NW;
  SelPrefetch<NW * 64> pre;
  if constexpr (SEL) pre.load(a.scores + (size_t)row * a.max_pages, a.max_pages);
  const int slot_raw = SEL      ? 0
                       : sparse ? vload_i32(a.sel_pages, (size_t)row * a.k_cap + min(idx0, a.k_cap - 1))
                                : vload_i32(a.block_table, (size_t)b * a.max_pages + min(idx0, a.max_pages - 1));
  const int len_v = vload_i32(a.seq_lens, b);
  const int32_t* cnt_p = sparse ? a.sel_count + row : a.seq_lens + b;  // a select, not a branch
  const int cnt_v = vload_i32(cnt_p, 0);
  const int tg = lane / LPT;  // token group
  const int cc = lane % LPT;  // channel chunk
  const int ch0 = cc * CH;

  // ---- query chunk in registers: fp16 pairs for v_dot2, and its fp32 sum
  half2v qh[G][CH / 2];
  float qsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint32_t* qp = (const uint32_t*)(a.q + ((size_t)b * a.Hq + g * G + hh) * D + ch0);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CH / 8; ++i) {
      const uint4 raw = *(const uint4*)(qp + 4 * i);
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qh[hh][4 * i + j] = as_half2(wd[j]);
        acc += half_bits_to_float(wd[j] & 0xFFFFu) + half_bits_to_float(wd[j] >> 16);
      }
    }
    qsum[hh] = acc;
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every level-1 load ahead of the first use below

  const int L = __builtin_amdgcn_readfirstlane(len_v);
  const int P = (L + kPage - 1) / kPage;
  // with every page selected cnt_p points at the length, so K = P either way
  // (using the value on both paths keeps the load where it is issued)
  const int cnt = __builtin_amdgcn_readfirstlane(cnt_v);
  const int Pc = (cnt + kPage - 1) / kPage;
  const int K = SEL ? num_selected(Pc, a.rnum, a.rden, a.k_fixed) : (sparse ? cnt : Pc);
  if constexpr (SEL) {  // the selection's count and padding, once per row
    if (s == 0 && a.sel_out) {
      if (threadIdx.x == 0) a.cnt_out[row] = K;
      for (int i = K + threadIdx.x; i < a.k_cap; i += NW * 64) a.sel_out[(size_t)row * a.k_cap + i] = -1;
    }
  }
  if (first >= K) return;
  const int n = min(a.pps, K - first);
  int* list = nullptr;  // SEL: this block's pages, ascending
  int jlog0;
  if constexpr (SEL) {
    __shared__ int sm_hist[2 * kSelBins];
    __shared__ int sm_wtot[2 * NW];
    __shared__ uint32_t sm_wrange[2 * NW];
    extern __shared__ int sm_dyn[];  // the block's pages [pps]
    list = sm_dyn;
    if (K < P) {
      select_chunk<NW>(pre, P, K, first, n, SelShared{sm_hist, sm_wtot, sm_wrange}, list);
    } else {
      for (int i = threadIdx.x; i < n; i += NW * 64) list[i] = first + i;
      __syncthreads();
    }
    if (a.sel_out)
      for (int i = threadIdx.x; i < n; i += NW * 64) a.sel_out[(size_t)row * a.k_cap + first + i] = list[i];
    jlog0 = list[min(w + lane * NW, n - 1)];
  } else {
    jlog0 = sparse ? min(max(slot_raw, 0), a.max_pages - 1) : min(idx0, a.max_pages - 1);
  }
  // level 2 for the wave's first 64 pages
  const int phys0 = vload_i32(a.block_table, (size_t)b * a.max_pages + jlog0);

  // ---- per-lane online softmax state
  const int nw = n > w ? (n - w + NW - 1) / NW : 0;
  float m[G], l[G], acc[G][CH], zacc[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
    zacc[hh] = 0.0f;
#pragma unroll
    for (int i = 0; i < CH; ++i) acc[hh][i] = 0.0f;
  }

  const size_t tile_elems = (size_t)kPage * D;
  struct PageRegs {
    uint4 kr[NL], vr[NL];
    float4 pr[NL];
    int nvalid;
  };
  // issue every load of one (page, KV head) tile
  auto load_page = [&](int jl, int ph, PageRegs& r) {
    r.nvalid = min(kPage, L - jl * kPage);
    const size_t tile = ((size_t)ph * a.H + g) * tile_elems;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const size_t off = (tile + (size_t)(i * TPL + tg) * D + ch0) * T::ELEM;
      r.kr[i] = load_stream_u4((const char*)a.k_pages + off);
      r.vr[i] = load_stream_u4((const char*)a.v_pages + off);
      if constexpr (FMT == kInt8Token)
        r.pr[i] = load_stream_f4(a.params + ((size_t)ph * a.H + g) * (kPage * 4) + (i * TPL + tg) * 4);
    }
    if constexpr (FMT == kInt8Group) {
      const float4 gp = load_stream_f4(a.params + ((size_t)ph * a.H + g) * 4);
#pragma unroll
      for (int i = 0; i < NL; ++i) r.pr[i] = gp;
    }
  };
  // fold one loaded tile into the online softmax of the G heads
  auto consume_page = [&](PageRegs& r) {
    const int nvalid = r.nvalid;
    // Padding slots of a partial last page hold no data (possibly NaN bits):
    // zero their values and scale/zero with per-lane selects.  A branch that
    // rewrote the loaded registers would make the compiler wait for every
    // outstanding load, including the prefetched tiles, at its join.
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const bool pad = i * TPL + tg >= nvalid;
      r.vr[i].x = pad ? 0u : r.vr[i].x;
      r.vr[i].y = pad ? 0u : r.vr[i].y;
      r.vr[i].z = pad ? 0u : r.vr[i].z;
      r.vr[i].w = pad ? 0u : r.vr[i].w;
      if constexpr (FMT != kFp16) {
        r.pr[i].z = pad ? 0.0f : r.pr[i].z;
        r.pr[i].w = pad ? 0.0f : r.pr[i].w;
      }
    }
    // logits
    float lg[G][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t kw[4] = {r.kr[i].x, r.kr[i].y, r.kr[i].z, r.kr[i].w};
      float dot[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) dot[hh] = 0.0f;
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) {
        if constexpr (FMT == kFp16) {
#pragma unroll
          for (int hh = 0; hh < G; ++hh) dot[hh] = __builtin_amdgcn_fdot2(as_half2(kw[d4]), qh[hh][d4], dot[hh], false);
        } else {
          const half2v lo = as_half2(__builtin_amdgcn_perm(0x64646464u, kw[d4], 0x04010400u));
          const half2v hi = as_half2(__builtin_amdgcn_perm(0x64646464u, kw[d4], 0x04030402u));
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            dot[hh] = __builtin_amdgcn_fdot2(lo, qh[hh][2 * d4], dot[hh], false);
            dot[hh] = __builtin_amdgcn_fdot2(hi, qh[hh][2 * d4 + 1], dot[hh], false);
          }
        }
      }
      const bool valid = i * TPL + tg < nvalid;
      float zz = 0.0f;
      if constexpr (FMT != kFp16) zz = __builtin_fmaf(-1024.0f, r.pr[i].x, r.pr[i].y);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float part = dot[hh];
        if constexpr (FMT != kFp16) part = __builtin_fmaf(r.pr[i].x, dot[hh], zz * qsum[hh]);
        part = sum_contig<LPT>(part);
        lg[hh][i] = valid ? part * a.scale_log2 : -INFINITY;
      }
    }
    // values, decoded once for the G heads
    float vf[NL][CH];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t vw[4] = {r.vr[i].x, r.vr[i].y, r.vr[i].z, r.vr[i].w};
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if constexpr (FMT == kFp16)
          vf[i][c] = half_bits_to_float((vw[c / 2] >> (16 * (c % 2))) & 0xFFFFu);
        else
          vf[i][c] = byte_to_float(vw[c / 4], c % 4);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float mx = lg[hh][0];
#pragma unroll
      for (int i = 1; i < NL; ++i) mx = fmaxf(mx, lg[hh][i]);
      const bool need = mx > m[hh] + kLazy;
      if (__ballot(need)) {  // wave-uniform branch; rare once the max settles
        const float mn = need ? mx : m[hh];
        const float alpha = mn == m[hh] ? 1.0f : __builtin_amdgcn_exp2f(m[hh] - mn);
        l[hh] *= alpha;
        zacc[hh] *= alpha;
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[hh][c] *= alpha;
        m[hh] = mn;
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float p = lg[hh][i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(lg[hh][i] - m[hh]);
        l[hh] += p;
        if constexpr (FMT == kFp16) {
#pragma unroll
          for (int c = 0; c < CH; ++c) acc[hh][c] = __builtin_fmaf(p, vf[i][c], acc[hh][c]);
        } else {
          const float ps = p * r.pr[i].z;
          zacc[hh] = __builtin_fmaf(p, r.pr[i].w, zacc[hh]);
#pragma unroll
          for (int c = 0; c < CH; ++c) acc[hh][c] = __builtin_fmaf(ps, vf[i][c], acc[hh][c]);
        }
      }
    }
  };

  for (int k0 = 0; k0 < nw; k0 += 64) {
    // page ids with one lane each (the first 64 come from the prologue)
    int jlog_v = jlog0, phys_v = phys0;
    if (k0 > 0) {  // wave-uniform; only when a split gives a wave more than 64 pages
      const int idx = min(first + w + (k0 + lane) * NW, K - 1);
      if constexpr (SEL)
        jlog_v = list[idx - first];
      else
        jlog_v = sparse ? min(max(a.sel_pages[(size_t)row * a.k_cap + idx], 0), a.max_pages - 1) : idx;
      phys_v = a.block_table[(size_t)b * a.max_pages + jlog_v];
    }
    const int cnt = min(64, nw - k0);
    // Software pipeline over a ring of R = kPrefetch + 1 register tiles: the
    // loads of tiles k+1 .. k+kPrefetch are in flight while tile k is consumed.
    // Every load is unconditional (an index past the chunk re-reads its last
    // tile, which is cached), so the compiler's wait counts stay exact; a
    // conditional load would make it wait for all outstanding loads.  The main
    // loop is unrolled by R so ring indices are compile-time constants.
    constexpr int R = kPrefetch + 1;
    PageRegs ring[R];
    auto load_idx = [&](int k, PageRegs& r) {
      const int kk = min(k, cnt - 1);
      load_page(__builtin_amdgcn_readlane(jlog_v, kk), __builtin_amdgcn_readlane(phys_v, kk), r);
    };
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u) load_idx(u, ring[u]);
    int k = 0;
    for (; k + R <= cnt; k += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        load_idx(k + u + kPrefetch, ring[(u + kPrefetch) % R]);
        consume_page(ring[u]);
      }
    }
    // fewer than R tiles remain; they are already in ring[0 ..] (no loads here)
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u)
      if (k + u < cnt) consume_page(ring[u]);
  }

  // ---- merge the token groups of the wave (lanes congruent mod LPT)
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float M = max_strided<LPT>(m[hh]);
    const float f = m[hh] == -INFINITY ? 0.0f : exp2f(m[hh] - M);
    l[hh] = sum_strided<LPT>(l[hh] * f);
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[hh][c] = sum_strided<LPT>((acc[hh][c] + zacc[hh]) * f);
    m[hh] = M;
  }

  // ---- merge the block's waves through LDS and write the split's partials
  __shared__ float sm_ml[NW][G][2];
  __shared__ float sm_acc[NW][G][D];
  if (tg == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int c = 0; c < CH; ++c) sm_acc[w][hh][ch0 + c] = acc[hh][c];
      if (lane == 0) {
        sm_ml[w][hh][0] = m[hh];
        sm_ml[w][hh][1] = l[hh];
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += NW * 64) {
    const int hh = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, sm_ml[v][hh][0]);
    float sa = 0.0f, sl = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float mv = sm_ml[v][hh][0];
      const float f = mv == -INFINITY ? 0.0f : exp2f(mv - M);  // 0 for a wave without pages
      sa = __builtin_fmaf(f, sm_acc[v][hh][c], sa);
      sl = __builtin_fmaf(f, sm_ml[v][hh][1], sl);
    }
    const size_t prow = ((size_t)b * a.Hq + g * G + hh) * a.max_splits + s;
    a.part_acc[prow * D + c] = sa;
    if (c == 0) {
      a.part_ml[prow * 2 + 0] = M;
      a.part_ml[prow * 2 + 1] = sl;
    }
  }

}

// Room for dynamic LDS a launch of the SEL kernel has under the device's
// per-block limit (its static LDS taken off), or 0 if that cannot be queried.
// Looked up once per instance (a function-local static).
template <int FMT, int D, int G>
size_t sel_lds_room() {
  static const size_t room = [] {
    hipFuncAttributes fa{};
    int dev = 0, lim = 0;
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(&decode_attn_kernel<FMT, D, G, kAttnWaves, true>)) !=
            hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        (size_t)lim < fa.sharedSizeBytes)
      return (size_t)0;
    return (size_t)lim - fa.sharedSizeBytes;
  }();
  return room;
}

template <int FMT, int D, int G>
hipError_t run(const AttnArgs& a, int B, hipStream_t st) {
  dim3 grid(a.max_splits, a.H, B);
  if (a.scores) {
    const size_t dyn = (size_t)a.pps * sizeof(int);
    if (dyn > sel_lds_room<FMT, D, G>()) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_attn_kernel<FMT, D, G, kAttnWaves, true>), grid, dim3(kAttnWaves * 64), dyn, st, a);
  } else {
    hipLaunchKernelGGL((decode_attn_kernel<FMT, D, G, kAttnWaves, false>), grid, dim3(kAttnWaves * 64), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((combine_kernel<D, G>), dim3(B * a.Hq), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int FMT, int D>
hipError_t run_g(const AttnArgs& a, int B, int G, hipStream_t st) {
  switch (G) {
    case 1: return run<FMT, D, 1>(a, B, st);
    case 2: return run<FMT, D, 2>(a, B, st);
    case 4: return run<FMT, D, 4>(a, B, st);
    default: return run<FMT, D, 8>(a, B, st);
  }
}

template <int FMT>
hipError_t run_d(const AttnArgs& a, int B, int D, int G, hipStream_t st) {
  return D == 64 ? run_g<FMT, 64>(a, B, G, st) : run_g<FMT, 128>(a, B, G, st);
}

}  // namespace

hipError_t launch_decode_attn(const kvq_cache& c, const kvq_seqs& s, const uint16_t* q, int num_q_heads,
                              const int32_t* sel_pages, const int32_t* sel_count, const InKernelSelect* ks,
                              int k_cap, float sm_scale, int pages_per_split, int max_splits, float* out, void* ws,
                              hipStream_t st) {
  const size_t n_part = (size_t)s.batch * num_q_heads * max_splits;
  float* part_ml = (float*)ws;
  float* part_acc = part_ml + n_part * 2;
  AttnArgs a{c.k_pages, c.v_pages, c.kv_params, s.block_table, s.seq_lens, q,
             ks ? nullptr : sel_pages, ks ? nullptr : sel_count,
             ks ? ks->scores : nullptr, ks ? ks->sel_out : nullptr, ks ? ks->cnt_out : nullptr,
             ks ? ks->rnum : 0, ks ? ks->rden : 1, ks ? ks->k_fixed : 0,
             part_acc, part_ml, out, c.num_kv_heads, num_q_heads, s.max_pages, k_cap,
             pages_per_split, max_splits, sm_scale * 1.4426950408889634f};
  const int G = num_q_heads / c.num_kv_heads;
  if (c.format == KVQ_FP16) return run_d<kFp16>(a, s.batch, c.head_dim, G, st);
  if (c.format == KVQ_INT8_TOKEN) return run_d<kInt8Token>(a, s.batch, c.head_dim, G, st);
  return run_d<kInt8Group>(a, s.batch, c.head_dim, G, st);
}

}  // namespace kvq
