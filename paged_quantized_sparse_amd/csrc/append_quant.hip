// append_quant.hip -- write new tokens into their 16-token pages, quantizing
// to INT8 per token or per 64-token group.
//
// Paged placement: token t of sequence b goes to physical page
// block_table[b][t/16], slot t%16 ("KV-cache layout from the HBM-bandwidth
// viewpoint", pzsr.cn, section 2 layout C and section 3 block tables).
// Per-token INT8 from each token's own min/max (same page, section 2); one
// scale/zero-point per 64 tokens ("Gemini KV cache: FlashAttention-3
// adaptation", uyd888.cn, chapter 1); the same with 4-bit codes (the
// quantization table's 4-bit row, intelliparadigm.com KV-cache page,
// section 3.2).  Quantization arithmetic is IEEE fp32,
// round-to-nearest-even, without contraction, so codes are reproducible
// bit for bit.
#include "append_body.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

struct AppendArgs {
  void* k_pages;
  void* v_pages;
  float* params;
  const int32_t* block_table;
  const int32_t* start_pos;
  const int32_t* new_off;
  const uint16_t* k_new;
  const uint16_t* v_new;
  int H;
  int max_pages;
  int n16;  // mixed precision: physical pages below n16 are the FP16 pool
};

// ---------------------------------------------------------------- fp16 copy
// grid (ceil(max_new / 4), B), 256 threads: 4 tokens per block, 16-byte chunks.
template <int D>
__global__ __launch_bounds__(256) void append_fp16_kernel(AppendArgs a) {
  const int b = blockIdx.y;
  const int r0 = a.new_off[b], n = a.new_off[b + 1] - r0;
  const int start = a.start_pos[b];
  constexpr int CPR = D / 8;  // 16-byte chunks per (token, head) row
  const int chunks = 4 * a.H * CPR;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const int i = blockIdx.x * 4 + c / (a.H * CPR);
    if (i >= n) continue;
    const int rem = c % (a.H * CPR);
    const int h = rem / CPR, part = rem % CPR;
    const int t = start + i;
    const int phys = a.block_table[(size_t)b * a.max_pages + t / kPage];
    const size_t src = ((size_t)(r0 + i) * a.H + h) * D + part * 8;
    const size_t dst = (((size_t)phys * a.H + h) * kPage + t % kPage) * D + part * 8;
    *(uint4*)((uint16_t*)a.k_pages + dst) = *(const uint4*)(a.k_new + src);
    *(uint4*)((uint16_t*)a.v_pages + dst) = *(const uint4*)(a.v_new + src);
  }
}

// ------------------------------- INT8 / INT4 per token or per group, mixed
// grid (ceil(max_new / 64), H, B): block (c, h, b) appends sequence b's new
// rows 64c .. 64c+63 for KV head h (append_body.h without the metadata: one
// wave per touched page, each page's rows loaded four at a time; a per-group
// format's chunk is one 64-token group, whose scale/zero come from all its
// rows).  A mixed-precision cache copies a row into an FP16-pool page and
// quantizes it per token into an INT8-pool page.
template <int FMT, int D>
__global__ __launch_bounds__(256) void append_chunk_kernel(AppendView a, int max_new) {
  const int skip = 64 * (int)blockIdx.x;  // rows past max_new are not written
  append_rows_and_meta<FMT, D, false, false>(a, blockIdx.z, blockIdx.y, nullptr, skip, max_new - skip);
}

template <int D>
hipError_t launch_append_d(const kvq_cache& c, const kvq_seqs& s, const AppendArgs& a, int max_new,
                           hipStream_t st) {
  const int B = s.batch, H = c.num_kv_heads;
  const dim3 chunk_grid((max_new + 63) / 64, H, B);
  const AppendView v{a.k_pages, a.v_pages, a.params, nullptr, a.block_table, a.start_pos, a.new_off, a.k_new,
                     a.v_new, a.H, a.max_pages, a.n16};
  switch (c.format) {
    case KVQ_FP16: hipLaunchKernelGGL(append_fp16_kernel<D>, dim3((max_new + 3) / 4, B), dim3(256), 0, st, a); break;
    case KVQ_INT8_TOKEN: hipLaunchKernelGGL((append_chunk_kernel<kInt8Token, D>), chunk_grid, dim3(256), 0, st, v, max_new); break;
    case KVQ_INT8_GROUP64: hipLaunchKernelGGL((append_chunk_kernel<kInt8Group, D>), chunk_grid, dim3(256), 0, st, v, max_new); break;
    case KVQ_INT4_TOKEN:
      if constexpr (D == 128) hipLaunchKernelGGL((append_chunk_kernel<kInt4Token, D>), chunk_grid, dim3(256), 0, st, v, max_new);
      break;
    case KVQ_MIXED_FP16_INT8: hipLaunchKernelGGL((append_chunk_kernel<kMixed, D>), chunk_grid, dim3(256), 0, st, v, max_new); break;
    default:
      if constexpr (D == 128) hipLaunchKernelGGL((append_chunk_kernel<kInt4Group, D>), chunk_grid, dim3(256), 0, st, v, max_new);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const kvq_cache& c, const kvq_seqs& s, const int32_t* start_pos,
                         const int32_t* new_off, int max_new, const uint16_t* k_new,
                         const uint16_t* v_new, hipStream_t st) {
  if (max_new == 0) return hipSuccess;
  AppendArgs a{c.k_pages, c.v_pages, c.kv_params, s.block_table, start_pos, new_off, k_new, v_new,
               c.num_kv_heads, s.max_pages, fp16_pool(c)};
  return c.head_dim == 64 ? launch_append_d<64>(c, s, a, max_new, st)
                          : launch_append_d<128>(c, s, a, max_new, st);
}

}  // namespace kvq
