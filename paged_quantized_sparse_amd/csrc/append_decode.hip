// append_decode.hip -- the decode-time append in one kernel: write each
// sequence's newest rows into their pages (fp16 copy, INT8 per token, or INT8
// per 64-token group, as in append_quant.hip) and rebuild the metadata
// phi = (per-channel min, max of the decoded keys) of every page those rows
// touch ("TinyServe", lpnh.cn, section 2.1; metadata kept exact at every step
// rather than refreshed every few steps as its section 5.2 suggests).
//
// One 256-thread block per (KV head, sequence).  The rows end the sequence,
// so a touched page's valid tokens are those before start + rows.  Phase 1
// writes the rows; after the block barrier, phase 2 reads the touched pages
// back (a wave per page) and writes their metadata.  No other block touches
// these pages, so no device-scope synchronization is needed.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

struct DecodeAppendArgs {
  void* k_pages;
  void* v_pages;
  float* params;
  float* meta;
  const int32_t* block_table;
  const int32_t* start_pos;
  const int32_t* new_off;
  const uint16_t* k_new;
  const uint16_t* v_new;
  int H;
  int max_pages;
};

template <int FMT, int D>
__global__ __launch_bounds__(256) void append_decode_kernel(DecodeAppendArgs a) {
  constexpr int E = D / 64;  // channels per lane: lane l owns l*E .. l*E+E-1
  const int h = blockIdx.x, b = blockIdx.y;
  const int r0 = a.new_off[b], n = a.new_off[b + 1] - r0;
  if (n <= 0) return;
  const int start = a.start_pos[b];
  const int L = start + n;
  const int w = wave_id(), lane = lane_id();
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;

  // ---- phase 1: the rows
  float gk[2] = {0.0f, 0.0f}, gv[2] = {0.0f, 0.0f}, ginv[2] = {1.0f, 1.0f};  // group (scale, zero), 1/scale
  if constexpr (FMT == kInt8Group) {
    float klo = INFINITY, khi = -INFINITY, vlo = INFINITY, vhi = -INFINITY;
    for (int e = threadIdx.x; e < n * D; e += 256) {
      const size_t src = ((size_t)(r0 + e / D) * a.H + h) * D + e % D;
      const float kx = half_bits_to_float(a.k_new[src]), vx = half_bits_to_float(a.v_new[src]);
      klo = fminf(klo, kx); khi = fmaxf(khi, kx);
      vlo = fminf(vlo, vx); vhi = fmaxf(vhi, vx);
    }
    klo = min_contig<64>(klo); khi = max_contig<64>(khi);
    vlo = min_contig<64>(vlo); vhi = max_contig<64>(vhi);
    __shared__ float red[4][4];
    if (lane == 0) { red[w][0] = klo; red[w][1] = khi; red[w][2] = vlo; red[w][3] = vhi; }
    __syncthreads();
    klo = fminf(fminf(red[0][0], red[1][0]), fminf(red[2][0], red[3][0]));
    khi = fmaxf(fmaxf(red[0][1], red[1][1]), fmaxf(red[2][1], red[3][1]));
    vlo = fminf(fminf(red[0][2], red[1][2]), fminf(red[2][2], red[3][2]));
    vhi = fmaxf(fmaxf(red[0][3], red[1][3]), fmaxf(red[2][3], red[3][3]));
    quant_params(klo, khi, gk[0], ginv[0]);
    quant_params(vlo, vhi, gv[0], ginv[1]);
    gk[1] = klo;
    gv[1] = vlo;
    if (threadIdx.x < 4 && threadIdx.x * kPage < n) {  // every page holding a row of the group
      const int phys = bt[(start + threadIdx.x * kPage) / kPage];
      *(float4*)(a.params + ((size_t)phys * a.H + h) * 4) = make_float4(gk[0], gk[1], gv[0], gv[1]);
    }
  }
  for (int i = w; i < n; i += 4) {
    const int t = start + i;
    const int phys = bt[t / kPage];
    const size_t src = ((size_t)(r0 + i) * a.H + h) * D + lane * E;
    const size_t dst = (((size_t)phys * a.H + h) * kPage + t % kPage) * D + lane * E;
    if constexpr (FMT == kFp16) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ((uint16_t*)a.k_pages)[dst + e] = a.k_new[src + e];
        ((uint16_t*)a.v_pages)[dst + e] = a.v_new[src + e];
      }
    } else {
      float kx[E], vx[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        kx[e] = half_bits_to_float(a.k_new[src + e]);
        vx[e] = half_bits_to_float(a.v_new[src + e]);
      }
      float ks = gk[0], kz = gk[1], kinv = ginv[0], vs = gv[0], vz = gv[1], vinv = ginv[1];
      if constexpr (FMT == kInt8Token) {
        float klo = INFINITY, khi = -INFINITY, vlo = INFINITY, vhi = -INFINITY;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          klo = fminf(klo, kx[e]); khi = fmaxf(khi, kx[e]);
          vlo = fminf(vlo, vx[e]); vhi = fmaxf(vhi, vx[e]);
        }
        klo = min_contig<64>(klo); khi = max_contig<64>(khi);
        vlo = min_contig<64>(vlo); vhi = max_contig<64>(vhi);
        quant_params(klo, khi, ks, kinv);
        quant_params(vlo, vhi, vs, vinv);
        kz = klo;
        vz = vlo;
        if (lane == 0)
          *(float4*)(a.params + (((size_t)phys * a.H + h) * kPage + t % kPage) * 4) = make_float4(ks, kz, vs, vz);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ((uint8_t*)a.k_pages)[dst + e] = (uint8_t)quant_code(kx[e], kz, kinv);
        ((uint8_t*)a.v_pages)[dst + e] = (uint8_t)quant_code(vx[e], vz, vinv);
      }
    }
  }
  __syncthreads();  // the block's rows are visible to the whole block

  // ---- phase 2: metadata of the touched pages, a wave per page
  for (int j = start / kPage + w; j <= (L - 1) / kPage; j += 4) {
    const int phys = bt[j];
    const int nvalid = min(kPage, L - j * kPage);
    const size_t tile = ((size_t)phys * a.H + h) * kPage;
    float lo[E], hi[E];
#pragma unroll
    for (int e = 0; e < E; ++e) { lo[e] = INFINITY; hi[e] = -INFINITY; }
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      if (t < nvalid) {
        const size_t row = (tile + t) * D + lane * E;
        float k[E];
        if constexpr (FMT == kFp16) {
#pragma unroll
          for (int e = 0; e < E; ++e) k[e] = half_bits_to_float(((const uint16_t*)a.k_pages)[row + e]);
        } else {
          const float* p = FMT == kInt8Token ? a.params + (tile + t) * 4 : a.params + ((size_t)phys * a.H + h) * 4;
          const float sc = p[0], zr = p[1];
#pragma unroll
          for (int e = 0; e < E; ++e) k[e] = __builtin_fmaf((float)((const uint8_t*)a.k_pages)[row + e], sc, zr);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) { lo[e] = fminf(lo[e], k[e]); hi[e] = fmaxf(hi[e], k[e]); }
      }
    }
    float* m = a.meta + ((size_t)phys * a.H + h) * 2 * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) { m[e] = lo[e]; m[D + e] = hi[e]; }
  }
}

template <int FMT>
hipError_t launch_fmt(const DecodeAppendArgs& a, int d, dim3 grid, hipStream_t st) {
  if (d == 64)
    hipLaunchKernelGGL((append_decode_kernel<FMT, 64>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((append_decode_kernel<FMT, 128>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append_decode(const kvq_cache& c, const kvq_seqs& s, const int32_t* start_pos,
                                const int32_t* new_off, const uint16_t* k_new, const uint16_t* v_new,
                                hipStream_t st) {
  DecodeAppendArgs a{c.k_pages, c.v_pages, c.kv_params, c.page_meta, s.block_table, start_pos, new_off,
                     k_new, v_new, c.num_kv_heads, s.max_pages};
  dim3 grid(c.num_kv_heads, s.batch);
  if (c.format == KVQ_FP16) return launch_fmt<kFp16>(a, c.head_dim, grid, st);
  if (c.format == KVQ_INT8_TOKEN) return launch_fmt<kInt8Token>(a, c.head_dim, grid, st);
  return launch_fmt<kInt8Group>(a, c.head_dim, grid, st);
}

}  // namespace kvq
