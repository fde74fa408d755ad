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
// grid (ceil(max_new / 4), B), 256 threads: 4 tokens per block, 16-byte chunks;
// rows past max_new are not written.
template <int D>
__global__ __launch_bounds__(256) void append_fp16_kernel(AppendArgs a, int max_new) {
  const int b = blockIdx.y;
  const int r0 = a.new_off[b], n = a.new_off[b + 1] - r0;
  const int start = a.start_pos[b];
  constexpr int CPR = D / 8;  // 16-byte chunks per (token, head) row
  const int chunks = 4 * a.H * CPR;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const int i = blockIdx.x * 4 + c / (a.H * CPR);
    if (i >= n || i >= max_new) continue;
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

// The per-token formats in bulk: four rows per wave instruction.  A quarter
// wave (16 lanes, C = D/16 channels each) takes one row, so a row's min/max
// reductions run over 16 lanes and its scale / 1/scale are computed once for
// four rows; the arithmetic is the per-token rule of append_body.h.  Grid and
// chunks as above; one wave per touched page.  A mixed-precision cache copies
// the rows of an FP16-pool page and quantizes those of an INT8-pool page.
template <int FMT, int D>
__global__ __launch_bounds__(256) void append_token_chunk_kernel(AppendView a, int max_new) {
  constexpr int C = D / 16;  // channels per lane
  constexpr int LV = fmt_levels(FMT);
  constexpr int BITS = fmt_int4(FMT) ? 4 : 8;
  static_assert(!fmt_int4(FMT) || D == 128, "4-bit rows are built for head_dim 128");
  const int b = blockIdx.z, h = blockIdx.y, skip = 64 * (int)blockIdx.x;
  const int r0 = a.new_off[b] + skip, n = min(a.new_off[b + 1] - r0, min(max_new - skip, 64));
  if (n <= 0) return;  // block-uniform
  const int start = a.start_pos[b] + skip;
  const int j_lo = start / kPage, npages = (start + n - 1) / kPage - j_lo + 1;
  const int lane = lane_id(), q = lane >> 4, ql = lane & 15;
  for (int pi = wave_id(); pi < npages; pi += 4) {  // wave-uniform
    const int j = j_lo + pi;
    int phys = a.block_table[(size_t)b * a.max_pages + j];
    const int t_begin = max(start, j * kPage), t_end = min(start + n, (j + 1) * kPage);
    bool fp16_page = false;
    char* kpool = (char*)a.k_pages;
    char* vpool = (char*)a.v_pages;
    if constexpr (FMT == kMixed) {  // wave-uniform: the page's pool decides
      fp16_page = phys < a.n16;
      if (!fp16_page) {
        const size_t off = (size_t)a.n16 * a.H * kPage * D * 2;
        kpool += off;
        vpool += off;
        phys -= a.n16;
      }
    }
    const size_t tile = ((size_t)phys * a.H + h) * kPage;  // first token row of the page
    for (int t0 = t_begin; t0 < t_end; t0 += 4) {  // wave-uniform; row t0 + q in quarter q
      const int t = t0 + q;
      const bool live = t < t_end;
      const size_t src = ((size_t)(r0 + min(t, t_end - 1) - start) * a.H + h) * D + ql * C;
      uint16_t kin[C], vin[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        kin[c] = a.k_new[src + c];
        vin[c] = a.v_new[src + c];
      }
      const size_t row = tile + t % kPage;
      if (fp16_page) {  // wave-uniform (mixed only): a copy
        if (live) {
#pragma unroll
          for (int c = 0; c < C; ++c) {
            ((uint16_t*)kpool)[row * D + ql * C + c] = kin[c];
            ((uint16_t*)vpool)[row * D + ql * C + c] = vin[c];
          }
        }
        continue;
      }
      float kx[C], vx[C];
      float klo = INFINITY, khi = -INFINITY, vlo = INFINITY, vhi = -INFINITY;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        kx[c] = half_bits_to_float(kin[c]);
        vx[c] = half_bits_to_float(vin[c]);
        klo = fminf(klo, kx[c]); khi = fmaxf(khi, kx[c]);
        vlo = fminf(vlo, vx[c]); vhi = fmaxf(vhi, vx[c]);
      }
      klo = zero_point(min_contig<16>(klo)); khi = max_contig<16>(khi);
      vlo = zero_point(min_contig<16>(vlo)); vhi = max_contig<16>(vhi);
      float ks, kinv, vs, vinv;
      quant_params<LV>(klo, khi, ks, kinv);
      quant_params<LV>(vlo, vhi, vs, vinv);
      uint32_t kc[C * BITS / 32 > 0 ? C * BITS / 32 : 1] = {}, vc[C * BITS / 32 > 0 ? C * BITS / 32 : 1] = {};
#pragma unroll
      for (int c = 0; c < C; ++c) {
        kc[c * BITS / 32] |= quant_code<LV>(kx[c], klo, kinv) << ((c * BITS) % 32);
        vc[c * BITS / 32] |= quant_code<LV>(vx[c], vlo, vinv) << ((c * BITS) % 32);
      }
      if (live) {
        uint8_t* kd = (uint8_t*)kpool + row * (D * BITS / 8) + ql * (C * BITS / 8);
        uint8_t* vd = (uint8_t*)vpool + row * (D * BITS / 8) + ql * (C * BITS / 8);
        if constexpr (C * BITS == 64) {
          *(uint2*)kd = make_uint2(kc[0], kc[1]);
          *(uint2*)vd = make_uint2(vc[0], vc[1]);
        } else {
          *(uint32_t*)kd = kc[0];
          *(uint32_t*)vd = vc[0];
        }
        if (ql == 0) *(float4*)(a.params + row * 4) = make_float4(ks, klo, vs, vlo);
      }
    }
  }
}

template <int D>
hipError_t launch_append_d(const kvq_cache& c, const kvq_seqs& s, const AppendArgs& a, int max_new,
                           hipStream_t st) {
  const int B = s.batch, H = c.num_kv_heads;
  const dim3 chunk_grid((max_new + 63) / 64, H, B);
  const AppendView v{a.k_pages, a.v_pages, a.params, nullptr, a.block_table, a.start_pos, a.new_off, a.k_new,
                     a.v_new, a.H, a.max_pages, a.n16};
  switch (c.format) {
    case KVQ_FP16:
      hipLaunchKernelGGL(append_fp16_kernel<D>, dim3((max_new + 3) / 4, B), dim3(256), 0, st, a, max_new);
      break;
    case KVQ_INT8_TOKEN:
      hipLaunchKernelGGL((append_token_chunk_kernel<kInt8Token, D>), chunk_grid, dim3(256), 0, st, v, max_new);
      break;
    case KVQ_INT8_GROUP64: hipLaunchKernelGGL((append_chunk_kernel<kInt8Group, D>), chunk_grid, dim3(256), 0, st, v, max_new); break;
    case KVQ_INT4_TOKEN:
      if constexpr (D == 128)
        hipLaunchKernelGGL((append_token_chunk_kernel<kInt4Token, D>), chunk_grid, dim3(256), 0, st, v, max_new);
      break;
    case KVQ_MIXED_FP16_INT8:
      hipLaunchKernelGGL((append_token_chunk_kernel<kMixed, D>), chunk_grid, dim3(256), 0, st, v, max_new);
      break;
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
