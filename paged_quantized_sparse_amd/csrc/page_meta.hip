// page_meta.hip -- per-page key metadata phi(K_j) = (m_j, M_j): the
// per-channel min and max of the page's keys ("TinyServe", lpnh.cn, section
// 2.1 direction-aware bounding box), kept in fp32 (section 5.2).  The keys
// are taken as attention decodes them (fmaf(code, scale, zero) for codes), so
// the page score bounds every stored key exactly.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

struct MetaArgs {
  const void* k_pages;
  const float* params;
  float* meta;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* page_begin;
  int H;
  int max_pages;
  int n16;  // mixed precision: physical pages below n16 are the FP16 pool
};

// The min / max rows of the first nvalid keys of page idx of a pool of format
// FMT, written to m (min row, then max row).  Lane l owns channels
// l*E .. l*E+E-1 and loads all 16 slots at once (padding slots are not read).
template <int FMT, int D>
__device__ __forceinline__ void page_lo_hi(const void* k_pages, const float* params, int idx, int h, int H,
                                           int nvalid, float* m) {
  constexpr int E = D / 64;
  const int lane = lane_id();
  {
    const size_t tile = ((size_t)idx * H + h) * kPage;
    float lo[E], hi[E];
#pragma unroll
    for (int e = 0; e < E; ++e) { lo[e] = INFINITY; hi[e] = -INFINITY; }
    // per-token (scale, zero) of the 16 slots in one load: lane t < 16 takes
    // slot t's pair, each row reads it back with readlane
    float2 prm = make_float2(0.0f, 0.0f);
    if constexpr (FMT != kFp16 && fmt_token(FMT)) prm = *(const float2*)(params + (tile + (lane & 15)) * 4);
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      if (t < nvalid) {
        const size_t row = (tile + t) * D + lane * E;
        float k[E];
        if constexpr (FMT == kFp16) {
          const uint16_t* src = (const uint16_t*)k_pages + row;
#pragma unroll
          for (int e = 0; e < E; ++e) k[e] = half_bits_to_float(src[e]);
        } else {
          float sc, zr;
          if constexpr (fmt_token(FMT)) {
            sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, prm.x), t));
            zr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, prm.y), t));
          } else {
            const float* p = params + ((size_t)idx * H + h) * 4;
            sc = p[0];
            zr = p[1];
          }
          if constexpr (fmt_int4(FMT)) {  // channels 2l, 2l+1: the two nibbles of byte l
            const uint32_t c = ((const uint8_t*)k_pages)[row / 2];
#pragma unroll
            for (int e = 0; e < E; ++e) k[e] = __builtin_fmaf((float)((c >> (4 * e)) & 0xFu), sc, zr);
          } else {
            const uint8_t* src = (const uint8_t*)k_pages + row;
#pragma unroll
            for (int e = 0; e < E; ++e) k[e] = __builtin_fmaf((float)src[e], sc, zr);
          }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) { lo[e] = fminf(lo[e], k[e]); hi[e] = fmaxf(hi[e], k[e]); }
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) { m[lane * E + e] = lo[e]; m[D + lane * E + e] = hi[e]; }
  }
}

// grid (ceil(span * H / 4), B), 4 waves per block.  Each wave takes one
// (logical page, KV head) item: lane l owns channels l*E .. l*E+E-1 (E = d/64)
// and loads all 16 token slots at once (padding slots are not read).
template <int FMT, int D>
__global__ __launch_bounds__(256) void page_meta_kernel(MetaArgs a) {
  const int b = blockIdx.y;
  const int L = a.seq_lens[b];
  const int P = (L + kPage - 1) / kPage;
  const int j0 = a.page_begin ? a.page_begin[b] : 0;
  for (int item = blockIdx.x * 4 + wave_id();; item += gridDim.x * 4) {
    const int j = j0 + item / a.H, h = item % a.H;
    if (j >= P) break;
    const int phys = a.block_table[(size_t)b * a.max_pages + j];
    const int nvalid = min(kPage, L - j * kPage);
    if constexpr (FMT == kMixed) {  // wave-uniform: the page's pool decides its format
      if (phys < a.n16)
        page_lo_hi<kFp16, D>(a.k_pages, nullptr, phys, h, a.H, nvalid, a.meta + ((size_t)phys * a.H + h) * 2 * D);
      else
        page_lo_hi<kInt8Token, D>((const char*)a.k_pages + (size_t)a.n16 * a.H * kPage * D * 2, a.params,
                                  phys - a.n16, h, a.H, nvalid, a.meta + ((size_t)phys * a.H + h) * 2 * D);
    } else {
      page_lo_hi<FMT, D>(a.k_pages, a.params, phys, h, a.H, nvalid, a.meta + ((size_t)phys * a.H + h) * 2 * D);
    }
  }
}

template <int FMT>
hipError_t launch_fmt(const MetaArgs& a, int d, dim3 grid, hipStream_t st) {
  if constexpr (fmt_int4(FMT))
    hipLaunchKernelGGL((page_meta_kernel<FMT, 128>), grid, dim3(256), 0, st, a);
  else if (d == 64)
    hipLaunchKernelGGL((page_meta_kernel<FMT, 64>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((page_meta_kernel<FMT, 128>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_page_meta(const kvq_cache& c, const kvq_seqs& s, const int32_t* page_begin,
                            int max_span, hipStream_t st) {
  MetaArgs a{c.k_pages, c.kv_params, c.page_meta, s.block_table, s.seq_lens, page_begin,
             c.num_kv_heads, s.max_pages, fp16_pool(c)};
  const int span = max_span > 0 ? (max_span < s.max_pages ? max_span : s.max_pages) : s.max_pages;
  const long long items = (long long)span * c.num_kv_heads;
  dim3 grid((unsigned)((items + 3) / 4 < 65536 ? (items + 3) / 4 : 65536), s.batch);
  if (c.format == KVQ_FP16) return launch_fmt<kFp16>(a, c.head_dim, grid, st);
  if (c.format == KVQ_INT8_TOKEN) return launch_fmt<kInt8Token>(a, c.head_dim, grid, st);
  if (c.format == KVQ_INT8_GROUP64) return launch_fmt<kInt8Group>(a, c.head_dim, grid, st);
  if (c.format == KVQ_INT4_TOKEN) return launch_fmt<kInt4Token>(a, c.head_dim, grid, st);
  if (c.format == KVQ_MIXED_FP16_INT8) return launch_fmt<kMixed>(a, c.head_dim, grid, st);
  return launch_fmt<kInt4Group>(a, c.head_dim, grid, st);
}

}  // namespace kvq
