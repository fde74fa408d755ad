// append_body.h -- the append of up to 64 rows of one (sequence, KV head),
// as a block-level device function shared by the decode-time append
// (append_decode.hip), the fused append + scores kernel and, without the
// metadata, the bulk append (append_quant.hip, 64-row chunks).  Called by all
// 256 threads of a block.
//
// Writes sequence b's newest rows for KV head h into their pages (fp16 copy,
// INT8 per token, or INT8 per 64-token group: "KV-cache layout from the
// HBM-bandwidth viewpoint", pzsr.cn, sections 2-3; "Gemini KV cache:
// FlashAttention-3 adaptation", uyd888.cn, chapter 1; the same two with 4-bit
// codes, two per byte: the KV-cache quantization page of intelliparadigm.com,
// section 3.2), and rebuilds the
// metadata phi = (per-channel min, max of the decoded keys) of every page the
// rows touch ("TinyServe", lpnh.cn, section 2.1).  The rows end the sequence,
// so a touched page's valid tokens are those before start + rows.
//
// Nothing written here is read back.  Each touched page belongs to one wave
// (page pi of the touched run to wave pi mod 4), which loads the page's older
// tokens, quantizes the page's new rows, keeps their decoded keys in
// registers (lane l owns channels l*E .. l*E+E-1) and so holds the page's
// whole min/max without any exchange between waves.  The metadata is written
// to HBM and, for a caller that scores the touched pages, to `sm_meta` in LDS.
// Decoded keys are fmaf(code, scale, zero) exactly as every other reader
// computes them.
#pragma once

#include "kvq_device.h"

namespace kvq {

constexpr int kMaxTouched = 5;  // 64 rows starting anywhere in a page touch at most 5 pages
constexpr int kRowBatch = 4;    // new rows (or channel pairs) whose loads are issued together

struct AppendView {
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
  int n16;  // mixed precision: physical pages below n16 are the FP16 pool
};

// One token row's codes, NB bytes per lane (lane l holding bytes NB l ..
// NB l + NB-1 of the row), written as whole dwords with device-scope stores:
// lanes gather their neighbours' bytes over DPP and every (4/NB)-th lane stores.
template <int NB>
__device__ __forceinline__ void store_row_dev(uint8_t* row, uint32_t bits) {
  const int lane = lane_id();
  if constexpr (NB == 4) {
    store_u32<true>((uint32_t*)(row + 4 * lane), bits);
  } else if constexpr (NB == 2) {
    const uint32_t nb = dpp_u32<kDppXor1>(bits);
    if ((lane & 1) == 0) store_u32<true>((uint32_t*)(row + 2 * lane), (bits & 0xFFFFu) | (nb << 16));
  } else {
    const uint32_t b1 = dpp_u32<0x39>(bits), b2 = dpp_u32<kDppXor2>(bits), b3 = dpp_u32<0x93>(bits);  // lanes +1, +2, +3 of the quad
    if ((lane & 3) == 0)
      store_u32<true>((uint32_t*)(row + lane), (bits & 0xFFu) | ((b1 & 0xFFu) << 8) | ((b2 & 0xFFu) << 16) | (b3 << 24));
  }
}

// One touched page j of sequence b, KV head h, stored in format PF at index
// idx of the arrays kpool / vpool / params: its older tokens decoded and its
// new rows written (rows r0 .. r0+n-1 hold tokens start .. start+n-1), each
// decoded key folded into lo / hi (lane l: channels l*E .. l*E+E-1).  gk, gv,
// ginv: the group's (scale, zero) and 1/scale for the per-group formats.
template <int PF, int D, bool WT, bool META = true>
__device__ __forceinline__ void append_page(const AppendView& a, void* kpool, void* vpool, float* params, int idx,
                                            int j, int h, int start, int n, int r0, const float* gk,
                                            const float* gv, const float* ginv, float* lo, float* hi) {
  constexpr int E = D / 64;
  constexpr int BITS = fmt_int4(PF) ? 4 : 8;
  constexpr int LV = fmt_levels(PF);
  constexpr int CROW = D * BITS / 8;  // bytes of one token's codes
  const int lane = lane_id();
  {
    const size_t tile = ((size_t)idx * a.H + h) * kPage;  // first token row of the page
    const int t_begin = max(start, j * kPage), t_end = min(start + n, (j + 1) * kPage);

    // older tokens of the page (only the first touched page has any): all 16
    // slots are loaded at once and the slots at or past `start` masked out,
    // so no load waits on another
    const int nold = META ? t_begin - j * kPage : 0;
    if (nold > 0) {  // wave-uniform
      float kold[kPage][E];
#pragma unroll
      for (int t = 0; t < kPage; ++t) {
        const size_t row = (tile + t) * D + lane * E;
        if constexpr (PF == kFp16) {
#pragma unroll
          for (int e = 0; e < E; ++e) kold[t][e] = half_bits_to_float(((const uint16_t*)kpool)[row + e]);
        } else {
          const float* p = fmt_token(PF) ? params + (tile + t) * 4 : params + ((size_t)idx * a.H + h) * 4;
          const float s = p[0], z = p[1];
          const uint8_t* cp = (const uint8_t*)kpool + (tile + t) * CROW + lane * E * BITS / 8;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const uint32_t c = fmt_int4(PF) ? (cp[0] >> (4 * e)) & 0xFu : cp[e];
            kold[t][e] = __builtin_fmaf((float)c, s, z);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < kPage; ++t)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          lo[e] = fminf(lo[e], t < nold ? kold[t][e] : INFINITY);
          hi[e] = fmaxf(hi[e], t < nold ? kold[t][e] : -INFINITY);
        }
    }

    // the page's new rows, four at a time: their fp16 bits are loaded
    // together (a row past the page's last re-reads the last), so a page's
    // rows cost a few dependent loads, not one each
    for (int t0 = t_begin; t0 < t_end; t0 += kRowBatch) {  // wave-uniform
      uint16_t kin[kRowBatch][E], vin[kRowBatch][E];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const size_t src = ((size_t)(r0 + min(t0 + u, t_end - 1) - start) * a.H + h) * D + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          kin[u][e] = a.k_new[src + e];
          vin[u][e] = a.v_new[src + e];
        }
      }
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const int t = t0 + u;
        if (t >= t_end) break;  // wave-uniform
        const size_t dst = (tile + t % kPage) * D + lane * E;
        float kdec[E];
        if constexpr (PF == kFp16) {
          uint32_t kw = 0, vw = 0;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const uint16_t kb = kin[u][e];
            const uint16_t vb = vin[u][e];
            if constexpr (WT) {
              kw |= (uint32_t)kb << (16 * e);
              vw |= (uint32_t)vb << (16 * e);
            } else {
              ((uint16_t*)kpool)[dst + e] = kb;
              ((uint16_t*)vpool)[dst + e] = vb;
            }
            kdec[e] = half_bits_to_float(kb);
          }
          if constexpr (WT) {
            const size_t row = (tile + t % kPage) * D * 2;
            store_row_dev<2 * E>((uint8_t*)kpool + row, kw);
            store_row_dev<2 * E>((uint8_t*)vpool + row, vw);
          }
        } else {
          float kx[E], vx[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            kx[e] = half_bits_to_float(kin[u][e]);
            vx[e] = half_bits_to_float(vin[u][e]);
          }
          float ks = gk[0], kz = gk[1], kinv = ginv[0], vs = gv[0], vz = gv[1], vinv = ginv[1];
          if constexpr (fmt_token(PF)) {
            float klo = INFINITY, khi = -INFINITY, vlo = INFINITY, vhi = -INFINITY;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              klo = fminf(klo, kx[e]); khi = fmaxf(khi, kx[e]);
              vlo = fminf(vlo, vx[e]); vhi = fmaxf(vhi, vx[e]);
            }
            klo = zero_point(min_contig<64>(klo)); khi = max_contig<64>(khi);
            vlo = zero_point(min_contig<64>(vlo)); vhi = max_contig<64>(vhi);
            quant_params<LV>(klo, khi, ks, kinv);
            quant_params<LV>(vlo, vhi, vs, vinv);
            kz = klo;
            vz = vlo;
            if (lane == 0) {
              float* tp = params + (tile + t % kPage) * 4;
              if constexpr (WT) {
                store_f<true>(tp, ks);
                store_f<true>(tp + 1, kz);
                store_f<true>(tp + 2, vs);
                store_f<true>(tp + 3, vz);
              } else {
                *(float4*)tp = make_float4(ks, kz, vs, vz);
              }
            }
          }
          uint32_t kw = 0, vw = 0;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const uint32_t kc = quant_code<LV>(kx[e], kz, kinv);
            const uint32_t vc = quant_code<LV>(vx[e], vz, vinv);
            kw |= kc << (BITS * e);
            vw |= vc << (BITS * e);
            kdec[e] = __builtin_fmaf((float)kc, ks, kz);
          }
          const size_t row = (tile + t % kPage) * CROW;
          if constexpr (WT) {
            store_row_dev<E * BITS / 8>((uint8_t*)kpool + row, kw);
            store_row_dev<E * BITS / 8>((uint8_t*)vpool + row, vw);
          } else {
            uint8_t* kp = (uint8_t*)kpool + row + lane * (E * BITS / 8);
            uint8_t* vp = (uint8_t*)vpool + row + lane * (E * BITS / 8);
            if constexpr (E * BITS / 8 == 2) {
              *(uint16_t*)kp = (uint16_t)kw;
              *(uint16_t*)vp = (uint16_t)vw;
            } else {
              *kp = (uint8_t)kw;
              *vp = (uint8_t)vw;
            }
          }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          lo[e] = fminf(lo[e], kdec[e]);
          hi[e] = fmaxf(hi[e], kdec[e]);
        }
      }
    }

  }
}

// WT: every store is a device-scope (written-through) store, for readers in
// other blocks of the same launch (the fused decode step); otherwise the
// stores are ordinary.  META: the touched pages' metadata is rebuilt (from
// their older tokens too); without it only codes and scale/zero are written
// (the bulk append, whose metadata kvq_build_page_meta builds).  `skip`: the
// block takes sequence b's new rows skip .. skip+limit-1, limit <= 64 (the
// bulk append's 64-row chunks; a per-group format's chunks start on its
// groups).
template <int FMT, int D, bool WT = false, bool META = true>
__device__ __forceinline__ void append_rows_and_meta(const AppendView& a, int b, int h,
                                                     float (*sm_meta)[2][D], int skip = 0, int limit = 64) {
  constexpr int E = D / 64;
  constexpr int LV = fmt_levels(FMT);
  static_assert(!fmt_int4(FMT) || E == 2, "4-bit rows are built for head_dim 128");
  // at most 64 rows (the documented limit; clamping keeps every index in range)
  const int r0 = a.new_off[b] + skip, n = min(a.new_off[b + 1] - r0, min(limit, 64));
  if (n <= 0) return;  // block-uniform
  const int start = a.start_pos[b] + skip;
  const int j_lo = start / kPage;
  const int npages = (start + n - 1) / kPage - j_lo + 1;
  const int w = wave_id(), lane = lane_id();
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;

  // ---- group (scale, zero): one per (64-token group, KV head), K and V apart
  float gk[2] = {0.0f, 0.0f}, gv[2] = {0.0f, 0.0f}, ginv[2] = {1.0f, 1.0f};
  if constexpr (fmt_group(FMT)) {
    // thread t takes channel pairs t, t + 256, ..., kRowBatch of them in
    // flight (a pair past the group's last re-reads the last: min and max
    // do not change)
    float klo = INFINITY, khi = -INFINITY, vlo = INFINITY, vhi = -INFINITY;
    const int npairs = n * D / 2;
    for (int p0 = threadIdx.x; p0 < npairs; p0 += 256 * kRowBatch) {
      uint16_t kin[kRowBatch][2], vin[kRowBatch][2];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const int e = 2 * min(p0 + 256 * u, npairs - 1);
        const size_t src = ((size_t)(r0 + e / D) * a.H + h) * D + e % D;
        kin[u][0] = a.k_new[src];
        kin[u][1] = a.k_new[src + 1];
        vin[u][0] = a.v_new[src];
        vin[u][1] = a.v_new[src + 1];
      }
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const float k0 = half_bits_to_float(kin[u][0]), k1 = half_bits_to_float(kin[u][1]);
        const float v0 = half_bits_to_float(vin[u][0]), v1 = half_bits_to_float(vin[u][1]);
        klo = fminf(klo, fminf(k0, k1)); khi = fmaxf(khi, fmaxf(k0, k1));
        vlo = fminf(vlo, fminf(v0, v1)); vhi = fmaxf(vhi, fmaxf(v0, v1));
      }
    }
    klo = min_contig<64>(klo); khi = max_contig<64>(khi);
    vlo = min_contig<64>(vlo); vhi = max_contig<64>(vhi);
    __shared__ float red[4][4];
    if (lane == 0) { red[w][0] = klo; red[w][1] = khi; red[w][2] = vlo; red[w][3] = vhi; }
    __syncthreads();
    klo = zero_point(fminf(fminf(red[0][0], red[1][0]), fminf(red[2][0], red[3][0])));
    khi = fmaxf(fmaxf(red[0][1], red[1][1]), fmaxf(red[2][1], red[3][1]));
    vlo = zero_point(fminf(fminf(red[0][2], red[1][2]), fminf(red[2][2], red[3][2])));
    vhi = fmaxf(fmaxf(red[0][3], red[1][3]), fmaxf(red[2][3], red[3][3]));
    quant_params<LV>(klo, khi, gk[0], ginv[0]);
    quant_params<LV>(vlo, vhi, gv[0], ginv[1]);
    gk[1] = klo;
    gv[1] = vlo;
    if (threadIdx.x < 4 && threadIdx.x * kPage < n) {  // every page holding a row of the group
      const int phys = bt[(start + threadIdx.x * kPage) / kPage];
      float* gp = a.params + ((size_t)phys * a.H + h) * 4;
      if constexpr (WT) {
        store_f<true>(gp, gk[0]);
        store_f<true>(gp + 1, gk[1]);
        store_f<true>(gp + 2, gv[0]);
        store_f<true>(gp + 3, gv[1]);
      } else {
        *(float4*)gp = make_float4(gk[0], gk[1], gv[0], gv[1]);
      }
    }
  }

  for (int pi = w; pi < npages; pi += 4) {  // wave-uniform
    const int j = j_lo + pi;
    const int phys = bt[j];
    float lo[E], hi[E];
#pragma unroll
    for (int e = 0; e < E; ++e) { lo[e] = INFINITY; hi[e] = -INFINITY; }
    if constexpr (FMT == kMixed) {  // the page's pool decides its format
      if (phys < a.n16) {
        append_page<kFp16, D, WT, META>(a, a.k_pages, a.v_pages, a.params, phys, j, h, start, n, r0, gk, gv, ginv,
                                        lo, hi);
      } else {
        const size_t off = (size_t)a.n16 * a.H * kPage * D * 2;
        append_page<kInt8Token, D, WT, META>(a, (char*)a.k_pages + off, (char*)a.v_pages + off, a.params,
                                             phys - a.n16, j, h, start, n, r0, gk, gv, ginv, lo, hi);
      }
    } else {
      append_page<FMT, D, WT, META>(a, a.k_pages, a.v_pages, a.params, phys, j, h, start, n, r0, gk, gv, ginv, lo,
                                    hi);
    }
    if constexpr (META) {  // the page's metadata: min row then max row
      float* m = a.meta + ((size_t)phys * a.H + h) * 2 * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        store_f<WT>(m + e, lo[e]);
        store_f<WT>(m + D + e, hi[e]);
        if (sm_meta) {
          sm_meta[pi][0][lane * E + e] = lo[e];
          sm_meta[pi][1][lane * E + e] = hi[e];
        }
      }
    }
  }
  if (sm_meta) __syncthreads();  // block-uniform: the LDS copy is complete
}

}  // namespace kvq
