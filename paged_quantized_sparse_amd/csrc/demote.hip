// demote.hip -- a mixed-precision cache moves pages from its FP16 pool to its
// INT8 pool ("TinyServe", lpnh.cn, section 6: pages of high importance stay
// FP16, the rest are INT8).  Per page: every valid token quantized per token
// from its fp16 rows (each (token, KV head) row with its own min/max, as the
// per-token append does: "KV-cache layout from the HBM-bandwidth viewpoint",
// pzsr.cn, section 2), the page's metadata rebuilt from the decoded keys
// ("TinyServe", section 2.1), and the block-table entry pointed at the new page.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

struct DemoteArgs {
  const uint16_t* k16;  // the FP16 pools
  const uint16_t* v16;
  uint8_t* k8;          // the INT8 pools
  uint8_t* v8;
  float* params;        // the INT8 pool's (scale, zero) per token slot
  float* meta;
  int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* seq;
  const int32_t* page;
  const int32_t* dst;
  int n16, H, max_pages;
};

// One block of 256 threads per item; wave w takes KV heads w, w+4, ...  Lane l
// owns channels l*E .. l*E+E-1 of every row, so it keeps its own channels'
// min / max of the decoded keys and no wave reads what another wrote.  The
// block-table entry is written after a barrier, once every wave has read it.
template <int D>
__global__ __launch_bounds__(256) void demote_kernel(DemoteArgs a) {
  constexpr int E = D / 64;
  const int i = blockIdx.x;
  const int b = a.seq[i], j = a.page[i], dst = a.dst[i];
  int32_t* entry = a.block_table + (size_t)b * a.max_pages + j;
  const int src = *entry;
  const int nvalid = min(kPage, a.seq_lens[b] - j * kPage);
  const int lane = lane_id();
  const int to = dst - a.n16;  // page index inside the INT8 pool
  for (int h = wave_id(); h < a.H; h += 4) {  // wave-uniform
    float lo[E], hi[E];
#pragma unroll
    for (int e = 0; e < E; ++e) { lo[e] = INFINITY; hi[e] = -INFINITY; }
    // tokens four at a time: their fp16 rows are loaded together (a slot
    // past the page's last valid token re-reads the last one, unused)
    for (int t0 = 0; t0 < nvalid; t0 += 4) {
      uint16_t kin[4][E], vin[4][E];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const size_t from = (((size_t)src * a.H + h) * kPage + min(t0 + u, nvalid - 1)) * D + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          kin[u][e] = a.k16[from + e];
          vin[u][e] = a.v16[from + e];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u;
        if (t >= nvalid) break;  // wave-uniform
        const size_t row = (((size_t)to * a.H + h) * kPage + t) * D + lane * E;
        float kx[E], vx[E];
        float klo = INFINITY, khi = -INFINITY, vlo = INFINITY, vhi = -INFINITY;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          kx[e] = half_bits_to_float(kin[u][e]);
          vx[e] = half_bits_to_float(vin[u][e]);
          klo = fminf(klo, kx[e]); khi = fmaxf(khi, kx[e]);
          vlo = fminf(vlo, vx[e]); vhi = fmaxf(vhi, vx[e]);
        }
        klo = zero_point(min_contig<64>(klo)); khi = max_contig<64>(khi);
        vlo = zero_point(min_contig<64>(vlo)); vhi = max_contig<64>(vhi);
        float ks, kinv, vs, vinv;
        quant_params(klo, khi, ks, kinv);
        quant_params(vlo, vhi, vs, vinv);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t kc = quant_code(kx[e], klo, kinv), vc = quant_code(vx[e], vlo, vinv);
          a.k8[row + e] = (uint8_t)kc;
          a.v8[row + e] = (uint8_t)vc;
          const float k = __builtin_fmaf((float)kc, ks, klo);
          lo[e] = fminf(lo[e], k);
          hi[e] = fmaxf(hi[e], k);
        }
        if (lane == 0)
          *(float4*)(a.params + (((size_t)to * a.H + h) * kPage + t) * 4) = make_float4(ks, klo, vs, vlo);
      }
    }
    float* m = a.meta + ((size_t)dst * a.H + h) * 2 * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      m[e] = lo[e];
      m[D + e] = hi[e];
    }
  }
  __syncthreads();  // every wave has read the old entry
  if (threadIdx.x == 0) *entry = dst;
}

}  // namespace

hipError_t launch_demote(const kvq_cache& c, const kvq_seqs& s, int n, const int32_t* seq, const int32_t* page,
                         const int32_t* dst, hipStream_t st) {
  const int n16 = c.num_fp16_pages;
  const size_t pool16 = (size_t)n16 * c.num_kv_heads * kPage * c.head_dim * 2;
  DemoteArgs a{(const uint16_t*)c.k_pages, (const uint16_t*)c.v_pages, (uint8_t*)c.k_pages + pool16,
               (uint8_t*)c.v_pages + pool16, c.kv_params, c.page_meta, const_cast<int32_t*>(s.block_table),
               s.seq_lens, seq, page, dst, n16, c.num_kv_heads, s.max_pages};
  if (c.head_dim == 64)
    hipLaunchKernelGGL(demote_kernel<64>, dim3(n), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(demote_kernel<128>, dim3(n), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvq
