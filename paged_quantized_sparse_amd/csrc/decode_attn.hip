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
// INT8 codes are dequantized in registers with the dequant folded into the
// dot product: q.k = s * sum(q_i c_i) + z * sum(q_i); values accumulate
// (p s) * c per channel plus p z once per token.  The G query heads of a KV
// group share every loaded tile.  Each wave keeps an online softmax
// (running max m, sum l, acc[d]) per query head in the exp2 domain; waves merge
// through LDS and the block writes one partial (m, l, acc) per query head and
// split.  combine_kernel then merges a row's splits with log-sum-exp weights.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kAttnWaves = 4;

struct AttnArgs {
  const void* k_pages;
  const void* v_pages;
  const float* params;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint16_t* q;
  const int32_t* sel_pages;  // NULL: all pages
  const int32_t* sel_count;
  float* part_acc;  // [B][Hq][max_splits][D]
  float* part_ml;   // [B][Hq][max_splits][2]
  float* out;       // [B][Hq][D]
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
  static constexpr int LPT = RB / 16;  // lanes per token
  static constexpr int TPL = 64 / LPT;  // tokens per load
  static constexpr int NL = kPage / TPL;  // loads per page
  static constexpr int CH = 16 / ELEM;  // channels per lane
};

__device__ __forceinline__ float byte_to_float(uint32_t w, int i) { return (float)((w >> (8 * i)) & 0xFFu); }

template <int FMT, int D, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_attn_kernel(AttnArgs a) {
  using T = Tile<FMT, D>;
  constexpr int LPT = T::LPT, TPL = T::TPL, NL = T::NL, CH = T::CH;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int row = b * a.H + g;
  const int L = a.seq_lens[b];
  const int P = (L + kPage - 1) / kPage;
  const int K = a.sel_pages ? a.sel_count[row] : P;
  const int first = s * a.pps;
  if (first >= K) return;
  const int n = min(a.pps, K - first);

  const int w = wave_id();
  const int lane = lane_id();
  const int tg = lane / LPT;  // token group
  const int cc = lane % LPT;  // channel chunk
  const int ch0 = cc * CH;

  // ---- query chunk in registers
  float qf[G][CH];
  float qsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint16_t* qp = a.q + ((size_t)b * a.Hq + g * G + hh) * D + ch0;
    const uint4 raw = *(const uint4*)qp;  // CH = 8 halves for fp16 tiles ...
    uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
    float acc = 0.0f;
    if constexpr (CH == 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[hh][i] = half_bits_to_float((wds[i / 2] >> (16 * (i % 2))) & 0xFFFFu);
    } else {  // ... 16 halves for INT8 tiles
      const uint4 raw2 = *(const uint4*)(qp + 8);
      uint32_t wds2[4] = {raw2.x, raw2.y, raw2.z, raw2.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[hh][i] = half_bits_to_float((wds[i / 2] >> (16 * (i % 2))) & 0xFFFFu);
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[hh][8 + i] = half_bits_to_float((wds2[i / 2] >> (16 * (i % 2))) & 0xFFFFu);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) acc += qf[hh][i];
    qsum[hh] = acc;
  }

  // ---- this wave's pages: k-th page is split index w + k*NW
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
  for (int k0 = 0; k0 < nw; k0 += 64) {
    // gather up to 64 page ids with one lane each
    int jlog_v = 0, phys_v = 0;
    if (k0 + lane < nw) {
      const int idx = first + w + (k0 + lane) * NW;
      jlog_v = a.sel_pages ? a.sel_pages[(size_t)row * a.k_cap + idx] : idx;
      phys_v = a.block_table[(size_t)b * a.max_pages + jlog_v];
    }
    const int cnt = min(64, nw - k0);
    for (int k = 0; k < cnt; ++k) {
      const int jl = __builtin_amdgcn_readlane(jlog_v, k);
      const int ph = __builtin_amdgcn_readlane(phys_v, k);
      const int nvalid = min(kPage, L - jl * kPage);
      const size_t tile = ((size_t)ph * a.H + g) * tile_elems;
      uint4 kr[NL], vr[NL];
      float4 pr[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const size_t off = (tile + (size_t)(i * TPL + tg) * D + ch0) * T::ELEM;
        kr[i] = *(const uint4*)((const char*)a.k_pages + off);
        vr[i] = *(const uint4*)((const char*)a.v_pages + off);
        if constexpr (FMT == kInt8Token)
          pr[i] = *(const float4*)(a.params + ((size_t)ph * a.H + g) * (kPage * 4) + (i * TPL + tg) * 4);
      }
      if constexpr (FMT == kInt8Group) {
        const float4 gp = *(const float4*)(a.params + ((size_t)ph * a.H + g) * 4);
#pragma unroll
        for (int i = 0; i < NL; ++i) pr[i] = gp;
      }
      if (nvalid < kPage) {  // partial last page (wave-uniform): padding slots hold no data
#pragma unroll
        for (int i = 0; i < NL; ++i)
          if (i * TPL + tg >= nvalid) {
            vr[i] = make_uint4(0, 0, 0, 0);
            pr[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          }
      }
      // decode this lane's chunk of each token once; reused by the G heads
      float kf[NL][CH], vf[NL][CH];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
        const uint32_t vw[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          if constexpr (FMT == kFp16) {
            kf[i][c] = half_bits_to_float((kw[c / 2] >> (16 * (c % 2))) & 0xFFFFu);
            vf[i][c] = half_bits_to_float((vw[c / 2] >> (16 * (c % 2))) & 0xFFFFu);
          } else {
            kf[i][c] = byte_to_float(kw[c / 4], c % 4);
            vf[i][c] = byte_to_float(vw[c / 4], c % 4);
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float lg[NL];
        float pmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float dot = 0.0f;
#pragma unroll
          for (int c = 0; c < CH; ++c) dot = __builtin_fmaf(qf[hh][c], kf[i][c], dot);
          if constexpr (FMT != kFp16) dot = __builtin_fmaf(pr[i].x, dot, pr[i].y * qsum[hh]);
          dot = sum_contig<LPT>(dot);
          lg[i] = (i * TPL + tg) < nvalid ? dot * a.scale_log2 : -INFINITY;
          pmax = fmaxf(pmax, lg[i]);
        }
        pmax = max_contig<64>(pmax);
        if (pmax > m[hh]) {  // wave-uniform
          const float alpha = exp2f(m[hh] - pmax);
          l[hh] *= alpha;
          zacc[hh] *= alpha;
#pragma unroll
          for (int c = 0; c < CH; ++c) acc[hh][c] *= alpha;
          m[hh] = pmax;
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const float p = exp2f(lg[i] - m[hh]);
          l[hh] += p;
          if constexpr (FMT == kFp16) {
#pragma unroll
            for (int c = 0; c < CH; ++c) acc[hh][c] = __builtin_fmaf(p, vf[i][c], acc[hh][c]);
          } else {
            const float ps = p * pr[i].z;
            zacc[hh] = __builtin_fmaf(p, pr[i].w, zacc[hh]);
#pragma unroll
            for (int c = 0; c < CH; ++c) acc[hh][c] = __builtin_fmaf(ps, vf[i][c], acc[hh][c]);
          }
        }
      }
    }
  }

  // ---- reduce over token groups (lanes congruent mod LPT)
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    l[hh] = sum_strided<LPT>(l[hh]);
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[hh][c] = sum_strided<LPT>(acc[hh][c] + zacc[hh]);
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
      const float f = exp2f(sm_ml[v][hh][0] - M);  // 0 for a wave without pages
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

// grid (B * Hq), D threads: out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
template <int D, int G>
__global__ __launch_bounds__(D) void combine_kernel(AttnArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int row = b * a.H + h / G;
  const int P = (a.seq_lens[b] + kPage - 1) / kPage;
  const int K = a.sel_pages ? a.sel_count[row] : P;
  const int ns = (K + a.pps - 1) / a.pps;
  const int c = threadIdx.x;
  const float* ml = a.part_ml + (size_t)bh * a.max_splits * 2;
  const float* pa = a.part_acc + (size_t)bh * a.max_splits * D;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const float f = exp2f(ml[2 * s] - M);
    num = __builtin_fmaf(f, pa[(size_t)s * D + c], num);
    den = __builtin_fmaf(f, ml[2 * s + 1], den);
  }
  a.out[(size_t)bh * D + c] = ns > 0 ? num / den : 0.0f;
}

template <int FMT, int D, int G>
hipError_t run(const AttnArgs& a, int B, hipStream_t st) {
  dim3 grid(a.max_splits, a.H, B);
  hipLaunchKernelGGL((decode_attn_kernel<FMT, D, G, kAttnWaves>), grid, dim3(kAttnWaves * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((combine_kernel<D, G>), dim3(B * a.Hq), dim3(D), 0, st, a);
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
                              const int32_t* sel_pages, const int32_t* sel_count, int k_cap, float sm_scale,
                              int pages_per_split, int max_splits, float* out, void* ws, hipStream_t st) {
  const size_t n_part = (size_t)s.batch * num_q_heads * max_splits;
  float* part_acc = (float*)ws;
  float* part_ml = part_acc + n_part * c.head_dim;
  AttnArgs a{c.k_pages, c.v_pages, c.kv_params, s.block_table, s.seq_lens, q, sel_pages, sel_count,
             part_acc, part_ml, out, c.num_kv_heads, num_q_heads, s.max_pages, k_cap, pages_per_split,
             max_splits, sm_scale * 1.4426950408889634f};
  const int G = num_q_heads / c.num_kv_heads;
  if (c.format == KVQ_FP16) return run_d<kFp16>(a, s.batch, c.head_dim, G, st);
  if (c.format == KVQ_INT8_TOKEN) return run_d<kInt8Token>(a, s.batch, c.head_dim, G, st);
  return run_d<kInt8Group>(a, s.batch, c.head_dim, G, st);
}

}  // namespace kvq
