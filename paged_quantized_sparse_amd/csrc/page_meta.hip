// page_meta.hip -- per-page key metadata phi(K_j) = (m_j, M_j): the
// per-channel min and max of the page's keys ("TinyServe", lpnh.cn, section
// 2.1 direction-aware bounding box), kept in fp32 (section 5.2).  The keys
// are taken as attention decodes them (fmaf(code, scale, zero) for INT8), so
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
};

// grid (span blocks, B), 256 threads.  Block x handles logical pages
// page_begin + x, + gridDim.x, ...; each thread one (KV head, channel).
template <int FMT, int D>
__global__ __launch_bounds__(256) void page_meta_kernel(MetaArgs a) {
  const int b = blockIdx.y;
  const int L = a.seq_lens[b];
  const int P = (L + kPage - 1) / kPage;
  const int j0 = a.page_begin ? a.page_begin[b] : 0;
  for (int j = j0 + blockIdx.x; j < P; j += gridDim.x) {
    const int phys = a.block_table[(size_t)b * a.max_pages + j];
    const int nvalid = min(kPage, L - j * kPage);
    for (int e = threadIdx.x; e < a.H * D; e += 256) {
      const int h = e / D, ch = e % D;
      const size_t tile = ((size_t)phys * a.H + h) * kPage;
      float lo = INFINITY, hi = -INFINITY;
      for (int t = 0; t < nvalid; ++t) {
        float k;
        if constexpr (FMT == kFp16) {
          k = half_bits_to_float(((const uint16_t*)a.k_pages)[(tile + t) * D + ch]);
        } else {
          const float c = (float)((const uint8_t*)a.k_pages)[(tile + t) * D + ch];
          const float* p = FMT == kInt8Token ? a.params + (tile + t) * 4 : a.params + ((size_t)phys * a.H + h) * 4;
          k = __builtin_fmaf(c, p[0], p[1]);
        }
        lo = fminf(lo, k);
        hi = fmaxf(hi, k);
      }
      float* m = a.meta + ((size_t)phys * a.H + h) * 2 * D;
      m[ch] = lo;
      m[D + ch] = hi;
    }
  }
}

template <int FMT>
hipError_t launch_fmt(const MetaArgs& a, int d, dim3 grid, hipStream_t st) {
  if (d == 64)
    hipLaunchKernelGGL((page_meta_kernel<FMT, 64>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((page_meta_kernel<FMT, 128>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_page_meta(const kvq_cache& c, const kvq_seqs& s, const int32_t* page_begin,
                            int max_span, hipStream_t st) {
  MetaArgs a{c.k_pages, c.kv_params, c.page_meta, s.block_table, s.seq_lens, page_begin,
             c.num_kv_heads, s.max_pages};
  const int span = max_span > 0 ? (max_span < s.max_pages ? max_span : s.max_pages) : s.max_pages;
  dim3 grid(span, s.batch);
  if (c.format == KVQ_FP16) return launch_fmt<kFp16>(a, c.head_dim, grid, st);
  if (c.format == KVQ_INT8_TOKEN) return launch_fmt<kInt8Token>(a, c.head_dim, grid, st);
  return launch_fmt<kInt8Group>(a, c.head_dim, grid, st);
}

}  // namespace kvq
