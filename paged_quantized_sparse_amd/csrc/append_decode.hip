// append_decode.hip -- the decode-time append in one kernel: write each
// sequence's newest rows into their pages and rebuild the metadata of every
// page those rows touch (append_body.h), one 256-thread block per
// (KV head, sequence).
#include "append_body.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

template <int FMT, int D>
__global__ __launch_bounds__(256) void append_decode_kernel(AppendView a) {
  append_rows_and_meta<FMT, D>(a, blockIdx.y, blockIdx.x, nullptr);
}

template <int FMT>
hipError_t launch_fmt(const AppendView& a, int d, dim3 grid, hipStream_t st) {
  if constexpr (fmt_int4(FMT))
    hipLaunchKernelGGL((append_decode_kernel<FMT, 128>), grid, dim3(256), 0, st, a);
  else if (d == 64)
    hipLaunchKernelGGL((append_decode_kernel<FMT, 64>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((append_decode_kernel<FMT, 128>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_decode(const kvq_cache& c, const kvq_seqs& s, const int32_t* start_pos,
                                const int32_t* new_off, const uint16_t* k_new, const uint16_t* v_new,
                                hipStream_t st) {
  AppendView a{c.k_pages, c.v_pages, c.kv_params, c.page_meta, s.block_table, start_pos, new_off,
               k_new, v_new, c.num_kv_heads, s.max_pages, fp16_pool(c)};
  dim3 grid(c.num_kv_heads, s.batch);
  if (c.format == KVQ_FP16) return launch_fmt<kFp16>(a, c.head_dim, grid, st);
  if (c.format == KVQ_INT8_TOKEN) return launch_fmt<kInt8Token>(a, c.head_dim, grid, st);
  if (c.format == KVQ_INT8_GROUP64) return launch_fmt<kInt8Group>(a, c.head_dim, grid, st);
  if (c.format == KVQ_INT4_TOKEN) return launch_fmt<kInt4Token>(a, c.head_dim, grid, st);
  if (c.format == KVQ_MIXED_FP16_INT8) return launch_fmt<kMixed>(a, c.head_dim, grid, st);
  return launch_fmt<kInt4Group>(a, c.head_dim, grid, st);
}

}  // namespace kvq
