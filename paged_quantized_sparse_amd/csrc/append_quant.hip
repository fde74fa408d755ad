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
#include "kvq_device.h"
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

// ----------------------------------------- INT8 / INT4 per token, mixed
// One wave per (token, KV head); 4 waves per block; grid (ceil(max_new*H/4), B).
// A mixed-precision cache copies the row into an FP16-pool page and
// quantizes it per token into an INT8-pool page.
template <int FMT, int D>
__global__ __launch_bounds__(256) void append_token_kernel(AppendArgs a) {
  constexpr int E = D / 64;  // elements per lane
  constexpr int LV = fmt_levels(FMT);
  static_assert(!fmt_int4(FMT) || E == 2, "4-bit rows are built for head_dim 128");
  const int b = blockIdx.y;
  const int r0 = a.new_off[b], n = a.new_off[b + 1] - r0;
  const int pair = blockIdx.x * 4 + wave_id();
  const int i = pair / a.H, h = pair % a.H;
  if (i >= n) return;
  const int lane = lane_id();
  const int t = a.start_pos[b] + i;
  int phys = a.block_table[(size_t)b * a.max_pages + t / kPage];
  const size_t src = ((size_t)(r0 + i) * a.H + h) * D + lane * E;
  if constexpr (FMT == kMixed) {
    if (phys < a.n16) {  // wave-uniform: an fp16 copy
      const size_t dst16 = (((size_t)phys * a.H + h) * kPage + t % kPage) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ((uint16_t*)a.k_pages)[dst16 + e] = a.k_new[src + e];
        ((uint16_t*)a.v_pages)[dst16 + e] = a.v_new[src + e];
      }
      return;
    }
    const size_t off = (size_t)a.n16 * a.H * kPage * D * 2;  // the INT8 pool
    a.k_pages = (char*)a.k_pages + off;
    a.v_pages = (char*)a.v_pages + off;
    phys -= a.n16;
  }
  const size_t dst = (((size_t)phys * a.H + h) * kPage + t % kPage) * D + lane * E;
  float kx[E], vx[E];
  float klo = INFINITY, khi = -INFINITY, vlo = INFINITY, vhi = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kx[e] = half_bits_to_float(a.k_new[src + e]);
    vx[e] = half_bits_to_float(a.v_new[src + e]);
    klo = fminf(klo, kx[e]); khi = fmaxf(khi, kx[e]);
    vlo = fminf(vlo, vx[e]); vhi = fmaxf(vhi, vx[e]);
  }
  klo = zero_point(min_contig<64>(klo)); khi = max_contig<64>(khi);
  vlo = zero_point(min_contig<64>(vlo)); vhi = max_contig<64>(vhi);
  float ks, kinv, vs, vinv;
  quant_params<LV>(klo, khi, ks, kinv);
  quant_params<LV>(vlo, vhi, vs, vinv);
  constexpr int BITS = fmt_int4(FMT) ? 4 : 8;
  uint32_t kc = 0, vc = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kc |= quant_code<LV>(kx[e], klo, kinv) << (BITS * e);
    vc |= quant_code<LV>(vx[e], vlo, vinv) << (BITS * e);
  }
  if constexpr (fmt_int4(FMT)) {  // the lane's two channels are one byte of the d/2-byte row
    const size_t byte = dst / 2;
    ((uint8_t*)a.k_pages)[byte] = (uint8_t)kc;
    ((uint8_t*)a.v_pages)[byte] = (uint8_t)vc;
  } else if constexpr (E == 2) {
    *(uint16_t*)((uint8_t*)a.k_pages + dst) = (uint16_t)kc;
    *(uint16_t*)((uint8_t*)a.v_pages + dst) = (uint16_t)vc;
  } else {
    ((uint8_t*)a.k_pages)[dst] = (uint8_t)kc;
    ((uint8_t*)a.v_pages)[dst] = (uint8_t)vc;
  }
  if (lane == 0) {
    float4* p = (float4*)(a.params + (((size_t)phys * a.H + h) * kPage + t % kPage) * 4);
    *p = make_float4(ks, klo, vs, vlo);
  }
}

// ------------------------------------------------- INT8 / INT4 per group
// One block of 256 threads per (64-token group, KV head, sequence);
// grid (ceil(max_new / 64), H, B).
template <int FMT, int D>
__global__ __launch_bounds__(256) void append_group_kernel(AppendArgs a) {
  constexpr int LV = fmt_levels(FMT);
  const int b = blockIdx.z, h = blockIdx.y, gi = blockIdx.x;
  const int r0 = a.new_off[b], n = a.new_off[b + 1] - r0;
  const int g0 = gi * 64;
  if (g0 >= n) return;
  const int gn = min(64, n - g0);
  const int start = a.start_pos[b];
  const int elems = gn * D;
  float klo = INFINITY, khi = -INFINITY, vlo = INFINITY, vhi = -INFINITY;
  for (int e = threadIdx.x; e < elems; e += 256) {
    const size_t src = ((size_t)(r0 + g0 + e / D) * a.H + h) * D + e % D;
    const float kx = half_bits_to_float(a.k_new[src]), vx = half_bits_to_float(a.v_new[src]);
    klo = fminf(klo, kx); khi = fmaxf(khi, kx);
    vlo = fminf(vlo, vx); vhi = fmaxf(vhi, vx);
  }
  klo = min_contig<64>(klo); khi = max_contig<64>(khi);
  vlo = min_contig<64>(vlo); vhi = max_contig<64>(vhi);
  __shared__ float red[4][4];
  const int w = wave_id();
  if (lane_id() == 0) { red[w][0] = klo; red[w][1] = khi; red[w][2] = vlo; red[w][3] = vhi; }
  __syncthreads();
  klo = zero_point(fminf(fminf(red[0][0], red[1][0]), fminf(red[2][0], red[3][0])));
  khi = fmaxf(fmaxf(red[0][1], red[1][1]), fmaxf(red[2][1], red[3][1]));
  vlo = zero_point(fminf(fminf(red[0][2], red[1][2]), fminf(red[2][2], red[3][2])));
  vhi = fmaxf(fmaxf(red[0][3], red[1][3]), fmaxf(red[2][3], red[3][3]));
  float ks, kinv, vs, vinv;
  quant_params<LV>(klo, khi, ks, kinv);
  quant_params<LV>(vlo, vhi, vs, vinv);
  constexpr int PER = fmt_int4(FMT) ? 2 : 1;  // channels per stored byte
  for (int e = threadIdx.x * PER; e < elems; e += 256 * PER) {
    const int i = g0 + e / D, ch = e % D;
    const size_t src = ((size_t)(r0 + i) * a.H + h) * D + ch;
    const int t = start + i;
    const int phys = a.block_table[(size_t)b * a.max_pages + t / kPage];
    const size_t dst = ((((size_t)phys * a.H + h) * kPage + t % kPage) * D + ch) / PER;
    uint32_t kc = 0, vc = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      kc |= quant_code<LV>(half_bits_to_float(a.k_new[src + u]), klo, kinv) << (4 * u);
      vc |= quant_code<LV>(half_bits_to_float(a.v_new[src + u]), vlo, vinv) << (4 * u);
    }
    ((uint8_t*)a.k_pages)[dst] = (uint8_t)kc;
    ((uint8_t*)a.v_pages)[dst] = (uint8_t)vc;
  }
  // the group's (scale, zero) go to every page holding one of its rows
  if (threadIdx.x < 4 && threadIdx.x * kPage < gn) {
    const int t = start + g0 + threadIdx.x * kPage;
    const int phys = a.block_table[(size_t)b * a.max_pages + t / kPage];
    *(float4*)(a.params + ((size_t)phys * a.H + h) * 4) = make_float4(ks, klo, vs, vlo);
  }
}

template <int D>
hipError_t launch_append_d(const kvq_cache& c, const kvq_seqs& s, const AppendArgs& a, int max_new,
                           hipStream_t st) {
  const int B = s.batch, H = c.num_kv_heads;
  const dim3 token_grid((unsigned)(((long long)max_new * H + 3) / 4), B);
  const dim3 group_grid((max_new + 63) / 64, H, B);
  switch (c.format) {
    case KVQ_FP16: hipLaunchKernelGGL(append_fp16_kernel<D>, dim3((max_new + 3) / 4, B), dim3(256), 0, st, a); break;
    case KVQ_INT8_TOKEN: hipLaunchKernelGGL((append_token_kernel<kInt8Token, D>), token_grid, dim3(256), 0, st, a); break;
    case KVQ_INT8_GROUP64: hipLaunchKernelGGL((append_group_kernel<kInt8Group, D>), group_grid, dim3(256), 0, st, a); break;
    case KVQ_INT4_TOKEN:
      if constexpr (D == 128) hipLaunchKernelGGL((append_token_kernel<kInt4Token, D>), token_grid, dim3(256), 0, st, a);
      break;
    case KVQ_MIXED_FP16_INT8: hipLaunchKernelGGL((append_token_kernel<kMixed, D>), token_grid, dim3(256), 0, st, a); break;
    default:
      if constexpr (D == 128) hipLaunchKernelGGL((append_group_kernel<kInt4Group, D>), group_grid, dim3(256), 0, st, a);
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
