// attn_body.h -- the split-K decode attention of one split and the split
// combine, as block-level device functions shared by decode_attn.hip (one
// launch each) and decode_step.hip (the fused, persistent decode step).
//
// paged, optionally INT8, KV cache ("TinyServe", lpnh.cn, section 3.1 phases
// 3-4: load only the selected pages' KV, then reduce; attention itself is
// softmax(q k^T / sqrt(d)) v, intelliparadigm.com KV-cache page, section 2.1).
//
// Split-K: block (split s, KV head g, sequence b) takes selected pages
// [s*PPS, (s+1)*PPS) of row (b, g); its waves take every NW-th page.  A wave
// holds a whole (page, KV head) tile in flight as LB-byte loads (16; 8 for
// 4-bit codes, so a lane holds the same 16 channels as with INT8): for a
// token row of RB bytes, LPT = RB/LB lanes share a token, so one load
// instruction covers TPL = 64/LPT tokens, and NL = 16/TPL loads cover the page.
// The next tile's loads are issued before the current tile is consumed.
//
// Keys: q.k runs on v_dot2_f32_f16 with the fp16 query.  A code c (8 or 4
// bits) becomes the fp16 value 1024 + c with one byte permute (0x64 is the
// high byte of 1024.0h; 4-bit codes are first split into their low and high
// nibbles), and one packed fp16 subtraction makes it c exactly, so for
// per-token or per-group (scale s, zero z)
//   q.k = s * sum q_i c_i + z * sum q_i.
// (Keeping the 1024 and folding -1024 s sum q_i into the zero term saves the
// subtraction but cancels a term ~1024 s |sum q_i| in fp32: ten times the
// output error on the 32K INT8 layer at the same speed.)
// Values: acc += (p s) * c per channel (byte or nibble converts + fma), plus
// p z once per token.  The G query heads of a KV group share every loaded tile.
//
// Online softmax per lane (exp2 domain): each lane keeps the running max m of
// the tokens it saw and rescales only when a logit exceeds m by more than
// kLazy (weights stay below 2^kLazy), so the inner loop needs no cross-lane
// max.  Lanes, then waves, merge with log-sum-exp weights; each block writes a
// partial (m, l, acc) per query head and split, and combine_kernel merges a
// row's splits.  (Merging in the last-arriving split block instead needs a
// device-scope release per block, which on gfx950 writes back the XCD's L2
// each time and costs far more than a second launch.)
//
// The SEL instances select the block's pages themselves (select_body.h) from
// the row's scores instead of reading a selection: every block of the row
// repeats the row's top-K and keeps the pages of its split's ranks.
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"
#include "select_body.h"

namespace kvq {

constexpr int kAttnWaves = 4;
// tiles in flight ahead of the one being consumed (1, 3, 4 and 6 measured the
// same or slower at 32K context)
constexpr int kPrefetch = 2;

constexpr float kLazy = 8.0f;

struct AttnArgs {
  const void* k_pages;
  const void* v_pages;
  const float* params;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint16_t* q;
  const int32_t* sel_pages;  // NULL: all pages (or selection in the kernel, below)
  const int32_t* sel_count;
  const float* scores;       // [B][H][max_pages]: select in the kernel (the SEL instances)
  int32_t* sel_out;          // optional copies of that selection, as kvq_topk_pages writes it
  int32_t* cnt_out;
  int rnum, rden, k_fixed;   // its selection rule
  float* part_acc;    // [B][Hq][max_splits][D]
  float* part_ml;     // [B][Hq][max_splits][2]
  float* out;         // [B][Hq][D]
  int H;
  int Hq;
  int max_pages;
  int k_cap;
  int pps;  // pages per split
  int max_splits;
  float scale_log2;  // sm_scale * log2(e)
  int n16;           // mixed precision: physical pages below n16 are the FP16 pool
  int direct;        // every row has at most one split: its block writes out, no combine follows
};

// The per-wave partials a block merges: NWS slots of (m, l) and acc per head.
template <int G, int D, int NWS>
struct WaveParts {
  float ml[NWS][G][2];
  float acc[NWS][G][D];
};

template <int G, int D, int NWS>
__device__ __forceinline__ WaveParts<G, D, NWS>* wave_parts() {
  __shared__ WaveParts<G, D, NWS> parts;
  return &parts;
}

// Mixed-precision pages, one phase per pool: of the first `valid` lanes (one
// page each), keep those whose physical page lies in phase PH's pool (1: the
// FP16 pool, pages below n16; 2: the INT8 pool), packed in order into the low
// lanes, with the INT8 pool's pages renumbered from 0.  Returns their count.
template <int PH>
__device__ __forceinline__ int pool_filter(int& jlog, int& phys, int valid, int n16) {
  const bool keep = lane_id() < valid && ((phys < n16) == (PH == 1));
  const uint64_t mask = __ballot(keep);
  const int cnt = __popcll(mask);
  // a dropped lane sends to lane 63, which is unused unless every lane is kept
  const int to = keep ? lanes_below(mask) : kWave - 1;
  jlog = __builtin_amdgcn_ds_permute(4 * to, jlog);
  phys = __builtin_amdgcn_ds_permute(4 * to, phys) - (PH == 2 ? n16 : 0);
  return cnt;
}

template <int FMT, int D>
struct Tile {
  static constexpr int BITS = FMT == kFp16 ? 16 : fmt_int4(FMT) ? 4 : 8;  // per channel
  static constexpr int RB = D * BITS / 8;                 // bytes of a token row
  static constexpr int LB = fmt_int4(FMT) ? 8 : 16;       // bytes per lane and load
  static constexpr int NWD = LB / 4;                      // words per lane and load
  static constexpr int LPT = RB / LB;     // lanes per token
  static constexpr int TPL = 64 / LPT;    // tokens per load
  static constexpr int NL = kPage / TPL;  // loads per page
  static constexpr int CH = LB * 8 / BITS;  // channels per lane
  static_assert(!fmt_int4(FMT) || D == 128, "4-bit tiles are built for head_dim 128");
};

// One lane's part of one load: NWD words.
template <int NWD>
struct Raw {
  uint32_t w[NWD];
};

template <int NWD>
__device__ __forceinline__ Raw<NWD> load_raw(const void* p) {
  if constexpr (NWD == 4) {
    const uint4 v = load_stream_u4(p);
    return Raw<4>{{v.x, v.y, v.z, v.w}};
  } else {
    const uint2 v = load_stream_u2(p);
    return Raw<2>{{v.x, v.y}};
  }
}

__device__ __forceinline__ Raw<4> load_raw_cached(const void* p) {
  const uint4 v = *(const uint4*)p;
  return Raw<4>{{v.x, v.y, v.z, v.w}};
}

__device__ __forceinline__ float byte_to_float(uint32_t w, int i) { return (float)((w >> (8 * i)) & 0xFFu); }

__device__ __forceinline__ half2v as_half2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));  // four bf16 bit patterns
typedef float float4v __attribute__((ext_vector_type(4)));

// Matrix-core form for a GQA group (G >= 2 query heads per KV head) over
// INT8 or 4-bit codes (and over the fp16 pages of a mixed cache, see the
// fp16 value product below), where q.k and p.v are small GEMMs per 16-token
// page.  A
// 16x16xKB MFMA takes A[i][k] from lane i + 16(k/KL), element k%KL, B[k][j]
// from lane j + 16(k/KL), element k%KL (KL = KB/4 elements per lane), and
// leaves D[i][j] in lane j + 16(i/4), register i%4.
//   Logits: C[t][h] = sum_k K[t][k] Q[h][k] on v_mfma_f32_16x16x32_f16 (the
//   full-rate shape on gfx950) with the page's 16 tokens as rows and the
//   heads (padded to 16) as columns.  Lane l holds token l%16's channels
//   (D/4)(l/16) .. +D/4 (one contiguous run of its row), MFMA m taking the
//   eight at offset 8m; the query is laid out to match, once.  C
//   then sits in lane h + 16g as tokens 4g .. 4g+3 of head h, which is
//   exactly the A layout of the second product.
//   Output: O[h][c] += sum_t W[h][t] V[t][c] on v_mfma_f32_16x16x16_bf16
//   (same layouts), W = p * v_scale split by truncation into three bf16
//   parts (three MFMAs, ~2^-21 relative; bf16 keeps fp32's exponent range,
//   so small weights keep their relative precision, which an fp16 split
//   loses below 2^-14), V as exact bf16 codes.  B needs four tokens of one
//   channel per lane, so each lane loads a run of its row (token
//   4g + l%4) and a 4x4 byte transpose inside each lane quad (two DPP
//   exchanges and byte permutes) hands lane (g, q, r) channel
//   (D/4)q + 4j + r of tokens 4g .. 4g+3 for MFMA j.
// The key codes become exact fp16 values as in the vector path.  fp16 tiles
// take the same two products with the fp16 keys and values as they are,
// the weights for the values being 2^7 p split into two fp16 parts.
template <int FMT, int D, int G>
struct MfmaPath {
  static constexpr bool on = G >= 2 && G <= 16;
  // value MFMAs per page (16 output channels each); also the query's groups
  // of 4 channels per lane (two per logits MFMA)
  static constexpr int NM = D / 16;
  // 16-byte loads per lane per tile, K and V each (a lane's run of D/4
  // channels: D/2 bytes of fp16, D/4 of INT8 codes, D/8 of 4-bit codes)
  static constexpr int NU = FMT == kFp16 ? D / 32 : fmt_int4(FMT) ? D / 128 : D / 64;
};

// fp16 tiles in the matrix-core form: the 4x4 transpose, inside each lane
// quad, of 16-bit values.  Lane r of a quad holds (lo, hi) = channels
// (c, c+1), (c+2, c+3) of token r; afterwards it holds channel c+r of tokens
// 0..3, as an MFMA B operand.  sel1 is the lane's permute of the first
// exchange (its pair-partner's half next to its own).
__device__ __forceinline__ half4v quad_transpose_halves(uint32_t lo, uint32_t hi, uint32_t sel1) {
  const int lane = lane_id();
  // lanes 2k, 2k+1: channels (c, c+2) or (c+1, c+3) of tokens 2k, 2k+1
  const uint32_t plo = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, kDppXor1, 0xF, 0xF, false);
  const uint32_t phi = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, kDppXor1, 0xF, 0xF, false);
  const uint32_t a = __builtin_amdgcn_perm(plo, lo, sel1);  // channel c (even lane) or c+1, tokens 2k, 2k+1
  const uint32_t b = __builtin_amdgcn_perm(phi, hi, sel1);  // channel c+2 or c+3
  // lanes 0, 1 keep a and take lane 2, 3's a; lanes 2, 3 take lane 0, 1's b and keep b
  const bool upper = lane & 2;
  const uint32_t send = upper ? a : b;
  const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, kDppXor2, 0xF, 0xF, false);
  const uint32_t t01 = upper ? recv : a, t23 = upper ? b : recv;
  return __builtin_bit_cast(half4v, ((uint64_t)t23 << 32) | t01);
}

// The fp16 pair (1024 + c0, 1024 + c1) less 1024: (c0, c1), exact.
__device__ __forceinline__ half2v minus_1024(uint32_t x) { return as_half2(x) - half2v{1024.0f16, 1024.0f16}; }

// 4-bit codes in the matrix-core form: a dword holds channels 0..7 of its run
// as nibbles (2i low, 2i+1 high).  Its codes as exact fp16 values in the
// order 0, 2, 4, 6, 1, 3, 5, 7 (the query is laid out in the same order, so
// the products pair up); the values take the even and the odd channels as
// two dwords of byte codes.
__device__ __forceinline__ half8v nibbles_f16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const half2v a = minus_1024(__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u));
  const half2v b = minus_1024(__builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u));
  const half2v c = minus_1024(__builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u));
  const half2v d = minus_1024(__builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u));
  return half8v{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Lane-quad byte transpose: lane r of each quad holds word W_r with bytes
// (token r, channels c..c+3); afterwards it holds (tokens 0..3, channel c+r).
__device__ __forceinline__ uint32_t quad_transpose_bytes(uint32_t x, uint32_t sel1, uint32_t sel2) {
  const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppXor1, 0xF, 0xF, false);
  const uint32_t t = __builtin_amdgcn_perm(x, p1, sel1);
  const uint32_t p2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)t, kDppXor2, 0xF, 0xF, false);
  return __builtin_amdgcn_perm(t, p2, sel2);
}

// Pairs of fp32 values' upper halves (their bf16 truncations) packed as the
// four elements of an MFMA operand.
__device__ __forceinline__ short4v pack_bf16(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  const uint32_t lo = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
  const uint32_t hi = __builtin_amdgcn_perm(x3, x2, 0x07060302u);
  return __builtin_bit_cast(short4v, ((uint64_t)hi << 32) | lo);
}

// Four INT8 codes (bytes of w) as exact bf16 values.
__device__ __forceinline__ short4v codes_bf16(uint32_t w) {
  return pack_bf16(__builtin_bit_cast(uint32_t, (float)(w & 0xFFu)),
                   __builtin_bit_cast(uint32_t, (float)((w >> 8) & 0xFFu)),
                   __builtin_bit_cast(uint32_t, (float)((w >> 16) & 0xFFu)),
                   __builtin_bit_cast(uint32_t, (float)(w >> 24)));
}

// Four INT8 codes (bytes of w) as exact fp16 values.
__device__ __forceinline__ half4v codes_f16(uint32_t w) {
  const half2v lo = minus_1024(__builtin_amdgcn_perm(0x64646464u, w, 0x04010400u));
  const half2v hi = minus_1024(__builtin_amdgcn_perm(0x64646464u, w, 0x04030402u));
  return half4v{lo[0], lo[1], hi[0], hi[1]};
}

// grid (B * Hq), 256 threads: out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
// with M = max_s m_s.  Thread (part, c) takes channel c of splits part,
// part + PARTS, ...: it loads eight splits' (m, l, acc) at once (indices past
// the row's splits re-read its last split and are masked), together with the
// split count, and merges them online; the PARTS partial merges then meet in
// LDS.  So the block waits on one round of loads, not two.
template <int D, int G, bool COH>
__device__ __forceinline__ void combine_one(const AttnArgs& a, int bh) {
  constexpr int PARTS = 256 / D;
  constexpr int U = 8;  // splits in flight per thread
  __shared__ float sm_m[PARTS][D], sm_num[PARTS][D], sm_den[PARTS][D];
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int row = b * a.H + h / G;
  const int tid = threadIdx.x;
  const int c = tid % D, part = tid / D;
  const float* ml = a.part_ml + (size_t)bh * a.max_splits * 2;
  const float* pa = a.part_acc + (size_t)bh * a.max_splits * D;
  const int32_t* cnt_p = a.sel_pages ? a.sel_count + row : a.seq_lens + b;  // a select, not a branch
  const int cnt_v = vload_i32(cnt_p, 0);
  float2 mlv[U];
  float av[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {  // speculative: the first U splits of this part
    const int sp = min(part + u * PARTS, a.max_splits - 1);
    mlv[u] = load_f2<COH>(ml + 2 * sp);
    av[u] = load_f<COH>(pa + (size_t)sp * D + c);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the count is waited for
  // with every page selected cnt_p points at the length, so K = P either way
  // (using the value on both paths keeps the load where it is issued)
  const int cnt = __builtin_amdgcn_readfirstlane(cnt_v);
  const int Pc = (cnt + kPage - 1) / kPage;
  const int K = a.sel_pages ? cnt : (a.scores ? num_selected(Pc, a.rnum, a.rden, a.k_fixed) : Pc);
  const int ns = (K + a.pps - 1) / a.pps;
  float M = -INFINITY, num = 0.0f, den = 0.0f;
  for (int s0 = 0;; s0 += U * PARTS) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a slot past the row's splits holds whatever the workspace held (any
      // bits, NaN included), so it is never read; the part is wave-uniform,
      // so this exit is too (a dead slot merged as (-inf, 0, 0) would leave
      // every value as it is, bit for bit, at the cost of two exp2f)
      if (s0 + part + u * PARTS >= ns) break;
      const float ms = mlv[u].x;
      const float as = av[u];
      const float ls = mlv[u].y;
      const float Mn = fmaxf(M, ms);
      const float fo = M == -INFINITY ? 0.0f : exp2f(M - Mn);
      const float fs = ms == -INFINITY ? 0.0f : exp2f(ms - Mn);
      num = __builtin_fmaf(fs, as, num * fo);
      den = __builtin_fmaf(fs, ls, den * fo);
      M = Mn;
    }
    if (s0 + U * PARTS >= ns) break;  // block-uniform
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = min(s0 + U * PARTS + part + u * PARTS, a.max_splits - 1);
      mlv[u] = load_f2<COH>(ml + 2 * sp);
      av[u] = load_f<COH>(pa + (size_t)sp * D + c);
    }
  }
  sm_m[part][c] = M;
  sm_num[part][c] = num;
  sm_den[part][c] = den;
  __syncthreads();
  if (part == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int p = 0; p < PARTS; ++p) Mt = fmaxf(Mt, sm_m[p][c]);
    float n = 0.0f, dd = 0.0f;
#pragma unroll
    for (int p = 0; p < PARTS; ++p) {
      const float f = sm_m[p][c] == -INFINITY ? 0.0f : exp2f(sm_m[p][c] - Mt);
      n = __builtin_fmaf(f, sm_num[p][c], n);
      dd = __builtin_fmaf(f, sm_den[p][c], dd);
    }
    a.out[(size_t)bh * D + c] = dd > 0.0f ? n / dd : 0.0f;
  }
  if constexpr (COH) __syncthreads();  // the LDS above is reused by the caller's next item
}

// One split of one (sequence b, KV head g) row: the attention of the G query
// heads over the row's selected pages of ranks [s*pps, (s+1)*pps), written as
// one partial (m, l, acc) per head.  Called by all NW * 64 threads of a block.
// SEL: the block selects its pages itself (select_body.h) from a.scores into
// `list` (LDS, pps entries).  COH: the row's scores are read, and the partials
// written, at device scope (the fused step kernel, where other blocks of the
// same launch wrote the scores and merge the partials).
// PH: 0 for a single-format cache.  A mixed-precision cache runs two phases
// over the same split: PH 1 (FMT = fp16) attends to the split's FP16-pool
// pages and leaves its waves' partials in LDS; PH 2 (FMT = INT8 per token)
// reuses the selection, attends to the INT8-pool pages, and merges all 2 NW
// wave partials into the split's partial.
template <int FMT, int D, int G, int NW, bool SEL, bool COH, int PH = 0>
__device__ __forceinline__ void attend_split(const AttnArgs& a, int g, int b, int s, int* list) {
  static_assert(NW == 4, "the split merge and the combine assume 4 waves");
  using T = Tile<FMT, D>;
  constexpr int LPT = T::LPT, TPL = T::TPL, NL = T::NL, CH = T::CH;
  using MP = MfmaPath<FMT, D, G>;
  // fp16 tiles take the matrix cores only in the FP16 pass of a mixed cache,
  // whose short page lists leave the vector form's per-tile work exposed
  // (GQA batch of 64 ragged sequences, mixed: 192 against 231 us per attention
  // call); a whole fp16 cache is bandwidth-bound and the vector form is faster
  // there (about 270 against 284 us on the same batch stored as fp16)
  constexpr bool MF = MP::on && (FMT != kFp16 || PH == 1);
  static_assert(!MF || NL * T::LB == 16 * MP::NU, "a lane's tile row is the same bytes in both forms");
  constexpr int NWD = T::NWD;
  const int row = b * a.H + g;
  const int first = s * a.pps;
  const int w = wave_id();
  const int lane = lane_id();
  // Prologue, three levels of dependent loads.  Level 1, issued together and
  // unconditionally: this lane's selection slot (first + w + lane * NW, the
  // wave's first 64 pages), the sequence length, the selected count and the
  // query.  Level 2: the block-table entry of the slot's page.  Level 3: the
  // first tiles.  Indices are clamped into their arrays, so a slot past the
  // row's count reads some entry of the row and is never used; with no
  // selection (all pages) the slot load reads the block table and is replaced
  // by the slot index itself.
  // With in-kernel selection, level 1 carries the row's first scores
  // instead of the selection slot, and the slot comes from LDS after the
  // selection.
  const bool sparse = !SEL && a.sel_pages != nullptr;
  const int idx0 = first + w + lane * NW;
  SelPrefetch<NW * 64> pre;
  if constexpr (SEL && PH != 2) pre.template load<COH>(a.scores + (size_t)row * a.max_pages, a.max_pages);
  // the tiles of a mixed cache's INT8 pool start after its FP16 pool
  const size_t pool_off = PH == 2 ? (size_t)a.n16 * a.H * kPage * D * 2 : 0;
  const char* const k_base = (const char*)a.k_pages + pool_off;
  const char* const v_base = (const char*)a.v_pages + pool_off;
  const int slot_raw = SEL      ? 0
                       : sparse ? vload_i32(a.sel_pages, (size_t)row * a.k_cap + min(idx0, a.k_cap - 1))
                                : vload_i32(a.block_table, (size_t)b * a.max_pages + min(idx0, a.max_pages - 1));
  const int len_v = vload_i32(a.seq_lens, b);
  const int32_t* cnt_p = sparse ? a.sel_count + row : a.seq_lens + b;  // a select, not a branch
  const int cnt_v = vload_i32(cnt_p, 0);
  const int tg = lane / LPT;  // token group
  const int cc = lane % LPT;  // channel chunk
  const int ch0 = cc * CH;

  // ---- query chunk in registers: fp16 pairs for v_dot2, and its fp32 sum.
  // With 4-bit codes each group of 8 channels is held as the pairs (0, 2),
  // (4, 6), (1, 3), (5, 7), the order in which a key word's nibbles come out.
  half2v qh[G][CH / 2];
  float qsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint32_t* qp = (const uint32_t*)(a.q + ((size_t)b * a.Hq + g * G + hh) * D + ch0);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CH / 8; ++i) {
      const uint4 raw = *(const uint4*)(qp + 4 * i);
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qh[hh][4 * i + j] = as_half2(wd[j]);
        acc += half_bits_to_float(wd[j] & 0xFFFFu) + half_bits_to_float(wd[j] >> 16);
      }
      if constexpr (fmt_int4(FMT)) {
        qh[hh][4 * i + 0] = as_half2(__builtin_amdgcn_perm(wd[1], wd[0], 0x05040100u));
        qh[hh][4 * i + 1] = as_half2(__builtin_amdgcn_perm(wd[3], wd[2], 0x05040100u));
        qh[hh][4 * i + 2] = as_half2(__builtin_amdgcn_perm(wd[1], wd[0], 0x07060302u));
        qh[hh][4 * i + 3] = as_half2(__builtin_amdgcn_perm(wd[3], wd[2], 0x07060302u));
      }
    }
    qsum[hh] = acc;
  }
  // matrix-core form: lane l holds head l%16's channels (D/4)(l/16) .. +D/4
  // (zeros for the padding heads), as groups of 4 (two per MFMA, which
  // takes the eight at offset 8m)
  half4v qB[MP::NM];
  float qs_mf = 0.0f;
  if constexpr (MF) {
    const int hn = lane & 15, gq = lane >> 4;
    const uint32_t* qp = (const uint32_t*)(a.q + ((size_t)b * a.Hq + g * G + min(hn, G - 1)) * D + (D / 4) * gq);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const uint4 raw = *(const uint4*)(qp + 4 * i);
      const uint32_t wd[4] = {hn < G ? raw.x : 0u, hn < G ? raw.y : 0u, hn < G ? raw.z : 0u, hn < G ? raw.w : 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += half_bits_to_float(wd[j] & 0xFFFFu) + half_bits_to_float(wd[j] >> 16);
      if constexpr (fmt_int4(FMT)) {  // channels 0, 2, 4, 6 then 1, 3, 5, 7 (as nibbles_f16)
        qB[2 * i] = __builtin_bit_cast(half4v, ((uint64_t)__builtin_amdgcn_perm(wd[3], wd[2], 0x05040100u) << 32) |
                                                   __builtin_amdgcn_perm(wd[1], wd[0], 0x05040100u));
        qB[2 * i + 1] = __builtin_bit_cast(half4v,
                                           ((uint64_t)__builtin_amdgcn_perm(wd[3], wd[2], 0x07060302u) << 32) |
                                               __builtin_amdgcn_perm(wd[1], wd[0], 0x07060302u));
      } else {
        qB[2 * i] = __builtin_bit_cast(half4v, ((uint64_t)wd[1] << 32) | wd[0]);
        qB[2 * i + 1] = __builtin_bit_cast(half4v, ((uint64_t)wd[3] << 32) | wd[2]);
      }
    }
    qs_mf = acc;
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every level-1 load ahead of the first use below
  if constexpr (MF) {  // the head's whole sum over its four lanes
    qs_mf += __shfl_xor(qs_mf, 16, kWave);
    qs_mf += __shfl_xor(qs_mf, 32, kWave);
  }

  const int L = __builtin_amdgcn_readfirstlane(len_v);
  const int P = (L + kPage - 1) / kPage;
  // with every page selected cnt_p points at the length, so K = P either way
  // (using the value on both paths keeps the load where it is issued)
  const int cnt = __builtin_amdgcn_readfirstlane(cnt_v);
  const int Pc = (cnt + kPage - 1) / kPage;
  const int K = SEL ? num_selected(Pc, a.rnum, a.rden, a.k_fixed) : (sparse ? cnt : Pc);
  if constexpr (SEL && PH != 2) {  // the selection's count and padding, once per row
    if (s == 0 && a.sel_out) {
      if (threadIdx.x == 0) a.cnt_out[row] = K;
      for (int i = K + threadIdx.x; i < a.k_cap; i += NW * 64) a.sel_out[(size_t)row * a.k_cap + i] = -1;
    }
  }
  if (first >= K) {
    // with one split per row and no combine, split 0 writes an empty row's zeros
    if (!COH && PH != 1 && a.direct && s == 0)
      for (int e = threadIdx.x; e < G * D; e += NW * 64) a.out[((size_t)b * a.Hq + g * G + e / D) * D + e % D] = 0.0f;
    return;
  }
  const int n = min(a.pps, K - first);
  int jlog0;
  if constexpr (SEL) {  // list: this block's pages, ascending
    __shared__ int sm_hist[2 * kSelBins];
    __shared__ int sm_wtot[2 * NW];
    __shared__ uint32_t sm_wrange[2 * NW];
    if constexpr (PH != 2) {  // (the second phase of a mixed cache reuses the first one's list)
      if (K < P) {
        select_chunk<NW>(pre, P, K, first, n, SelShared{sm_hist, sm_wtot, sm_wrange}, list);
      } else {
        for (int i = threadIdx.x; i < n; i += NW * 64) list[i] = first + i;
        __syncthreads();
      }
      if (a.sel_out)
        for (int i = threadIdx.x; i < n; i += NW * 64) a.sel_out[(size_t)row * a.k_cap + first + i] = list[i];
    }
    jlog0 = list[min(w + lane * NW, n - 1)];
  } else {
    jlog0 = sparse ? min(max(slot_raw, 0), a.max_pages - 1) : min(idx0, a.max_pages - 1);
  }
  // level 2 for the wave's first 64 pages
  const int phys0 = vload_i32(a.block_table, (size_t)b * a.max_pages + jlog0);

  // ---- per-lane online softmax state
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
  // matrix-core form: (m, l, z) of head lane%16 over this lane's tokens (m the
  // same in the head's four lanes), and O[h][c] accumulators in MFMA layout
  float mf_m = -INFINITY, mf_l = 0.0f, mf_z = 0.0f;
  float4v mf_acc[MP::NM];
#pragma unroll
  for (int j = 0; j < MP::NM; ++j) mf_acc[j] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  const size_t tile_elems = (size_t)kPage * D;
  // scale/zero registers per tile: the matrix-core form wants tokens
  // 4(l/16) .. +3 per lane (per token) or the tile's one group pair
  constexpr int NP = MF ? (fmt_token(FMT) ? 4 : 1) : NL;
  struct PageRegs {
    Raw<NWD> kr[NL], vr[NL];
    float4 pr[NP];
    int nvalid;
  };
  // issue every load of one (page, KV head) tile
  auto load_page = [&](int jl, int ph, PageRegs& r) {
    r.nvalid = min(kPage, L - jl * kPage);
    const size_t tile = ((size_t)ph * a.H + g) * tile_elems;
    if constexpr (MF && fmt_int4(FMT)) {
      // as below, at half a byte per channel: one 16-byte load per lane, K and V each
      const char* kp = k_base + tile / 2 + (lane & 15) * (D / 2) + (D / 8) * (lane >> 4);
      const char* vp = v_base + tile / 2 + (4 * (lane >> 4) + (lane & 3)) * (D / 2) + (D / 8) * ((lane >> 2) & 3);
      const Raw<4> kk = load_raw_cached(kp), vv = load_raw_cached(vp);
#pragma unroll
      for (int u = 0; u < NL; ++u) {
#pragma unroll
        for (int x = 0; x < NWD; ++x) {
          r.kr[u].w[x] = kk.w[NWD * u + x];
          r.vr[u].w[x] = vv.w[NWD * u + x];
        }
      }
    }
    if constexpr (MF && FMT == kFp16) {
      // as below, at two bytes per channel: NU 16-byte loads per lane, K and V each
      const char* kp = k_base + 2 * tile + (lane & 15) * (2 * D) + (D / 2) * (lane >> 4);
      const char* vp = v_base + 2 * tile + (4 * (lane >> 4) + (lane & 3)) * (2 * D) + (D / 2) * ((lane >> 2) & 3);
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        r.kr[u] = load_raw_cached(kp + 16 * u);
        r.vr[u] = load_raw_cached(vp + 16 * u);
      }
      return;
    }
    if constexpr (MF && FMT != kFp16 && !fmt_int4(FMT)) {
      // K: token l%16, run (D/4)(l/16); V: token 4(l/16) + l%4, run (D/4)((l/4)%4)
      const char* kp = k_base + tile + (lane & 15) * D + (D / 4) * (lane >> 4);
      const char* vp = v_base + tile + (4 * (lane >> 4) + (lane & 3)) * D + (D / 4) * ((lane >> 2) & 3);
      // Each of these loads covers half of every 128-byte row of the tile (the
      // other half comes with the next), so they are ordinary loads, which keep
      // the line in L2 for its second half (64 ragged sequences, 8 KV heads in
      // groups of 4: 166 against 178 us per attention call with the streaming
      // hint).
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        r.kr[u] = load_raw_cached(kp + 16 * u);
        r.vr[u] = load_raw_cached(vp + 16 * u);
      }
    }
    if constexpr (MF) {
      if constexpr (fmt_token(FMT)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          r.pr[i] = load_stream_f4(a.params + (((size_t)ph * a.H + g) * kPage + 4 * (lane >> 4) + i) * 4);
      } else {
        r.pr[0] = load_stream_f4(a.params + ((size_t)ph * a.H + g) * 4);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const size_t off = (tile + (size_t)(i * TPL + tg) * D + ch0) * T::BITS / 8;
      r.kr[i] = load_raw<NWD>(k_base + off);
      r.vr[i] = load_raw<NWD>(v_base + off);
      if constexpr (fmt_token(FMT))
        r.pr[i] = load_stream_f4(a.params + ((size_t)ph * a.H + g) * (kPage * 4) + (i * TPL + tg) * 4);
    }
    if constexpr (fmt_group(FMT)) {
      const float4 gp = load_stream_f4(a.params + ((size_t)ph * a.H + g) * 4);
#pragma unroll
      for (int i = 0; i < NL; ++i) r.pr[i] = gp;
    }
  };
  // fold one loaded tile into the online softmax of the G heads
  auto consume_page = [&](PageRegs& r) {
    const int nvalid = r.nvalid;
    if constexpr (MF) {
      const int hn = lane & 15, g4 = lane >> 4;
      // logits of tokens 4 g4 + i for head hn: C = K Q^T on the matrix cores
      float4v cq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < (fmt_int4(FMT) || FMT == kFp16 ? 0 : NL); ++u) {
        const uint32_t* kw = r.kr[u].w;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const half4v k0 = codes_f16(kw[2 * h2]), k1 = codes_f16(kw[2 * h2 + 1]);
          const half4v q0 = qB[4 * u + 2 * h2], q1 = qB[4 * u + 2 * h2 + 1];
          const half8v ka = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
          const half8v qa = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
          cq = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qa, cq, 0, 0, 0);
        }
      }
      if constexpr (FMT == kFp16) {  // MFMA m: load m of the lane's run, channels 8m .. 8m+7
#pragma unroll
        for (int m = 0; m < NL; ++m) {
          const half4v q0 = qB[2 * m], q1 = qB[2 * m + 1];
          const half8v qa = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
          const uint32_t* kw = r.kr[m].w;
          const half4v k0 = __builtin_bit_cast(half4v, ((uint64_t)kw[1] << 32) | kw[0]);
          const half4v k1 = __builtin_bit_cast(half4v, ((uint64_t)kw[3] << 32) | kw[2]);
          const half8v ka = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
          cq = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qa, cq, 0, 0, 0);
        }
      }
      if constexpr (fmt_int4(FMT)) {  // MFMA m: dword m of the lane's run, channels 8m .. 8m+7
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const half4v q0 = qB[2 * m], q1 = qB[2 * m + 1];
          const half8v qa = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
          cq = __builtin_amdgcn_mfma_f32_16x16x32_f16(nibbles_f16(r.kr[m / NWD].w[m % NWD]), qa, cq, 0, 0, 0);
        }
      }
      float lg[4];
      bool valid[4];
      float lm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        valid[i] = 4 * g4 + i < nvalid && hn < G;
        float part = cq[i];
        if constexpr (FMT != kFp16) {
          const float4 pp = r.pr[NP == 4 ? i : 0];
          part = __builtin_fmaf(pp.x, cq[i], pp.y * qs_mf);
        }
        lg[i] = valid[i] ? part * a.scale_log2 : -INFINITY;
        lm = fmaxf(lm, lg[i]);
      }
      if (__ballot(lm > mf_m + kLazy)) {  // wave-uniform; rare once the max settles
        // every lane of a head decides on the head's max over its four lanes
        float hm = fmaxf(lm, __shfl_xor(lm, 16, kWave));
        hm = fmaxf(hm, __shfl_xor(hm, 32, kWave));
        const float mn = hm > mf_m + kLazy ? hm : mf_m;
        const float alpha = mn == mf_m ? 1.0f : __builtin_amdgcn_exp2f(mf_m - mn);
        mf_l *= alpha;
        mf_z *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // O row 4 g4 + i takes that head's factor (from its lane)
          const float ai = __shfl(alpha, 4 * g4 + i, kWave);
#pragma unroll
          for (int j = 0; j < MP::NM; ++j) mf_acc[j][i] *= ai;
        }
        mf_m = mn;
      }
      if constexpr (FMT == kFp16) {
        // values: O += (W_hi + W_lo) V on v_mfma_f32_16x16x16_f16, V exact fp16,
        // W = 2^7 p split into two fp16 parts (~2^-22 relative; the scale keeps
        // weights down to 2^-21 normal in fp16, and p <= 2^kLazy keeps 2^7 p
        // below fp16's maximum), O scaled back by 2^-7 when the partial is written
        half4v whi, wlo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = lg[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(lg[i] - mf_m);
          mf_l += p;
          const float w = 128.0f * p;
          whi[i] = (_Float16)w;
          wlo[i] = (_Float16)(w - (float)whi[i]);
        }
        // a padding token's row may hold any bits (NaN included): zeroed
        const bool vpad = 4 * g4 + (lane & 3) >= nvalid;
        const uint32_t sel1 = (lane & 1) ? 0x03020706u : 0x05040100u;
#pragma unroll
        for (int j = 0; j < MP::NM; ++j) {  // channels 4j .. 4j+3 of the lane's run: dwords 2j, 2j+1
          const uint32_t lo = vpad ? 0u : r.vr[j / 2].w[2 * (j % 2)];
          const uint32_t hi = vpad ? 0u : r.vr[j / 2].w[2 * (j % 2) + 1];
          const half4v vb = quad_transpose_halves(lo, hi, sel1);
          mf_acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(wlo, vb, mf_acc[j], 0, 0, 0);
          mf_acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(whi, vb, mf_acc[j], 0, 0, 0);
        }
        return;
      }
      uint32_t wb0[4], wb1[4], wb2[4];  // w = b0 + b1 + b2, each a bf16 (low 16 bits zero)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = lg[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(lg[i] - mf_m);
        mf_l += p;
        // padding slots may hold any bits: their scale/zero never reach the sums
        const float4 pp = r.pr[NP == 4 ? i : 0];
        const float w = valid[i] ? p * pp.z : 0.0f;
        mf_z = valid[i] ? __builtin_fmaf(p, pp.w, mf_z) : mf_z;
        wb0[i] = __builtin_bit_cast(uint32_t, w) & 0xFFFF0000u;
        const float r1 = w - __builtin_bit_cast(float, wb0[i]);  // exact
        wb1[i] = __builtin_bit_cast(uint32_t, r1) & 0xFFFF0000u;
        const float r2 = r1 - __builtin_bit_cast(float, wb1[i]);  // exact
        wb2[i] = __builtin_bit_cast(uint32_t, r2) & 0xFFFF0000u;
      }
      const short4v wa0 = pack_bf16(wb0[0], wb0[1], wb0[2], wb0[3]);
      const short4v wa1 = pack_bf16(wb1[0], wb1[1], wb1[2], wb1[3]);
      const short4v wa2 = pack_bf16(wb2[0], wb2[1], wb2[2], wb2[3]);
      // values: quad byte transpose to four tokens of one channel, exact bf16
      // codes, then O += (W_0 + W_1 + W_2) V
      const uint32_t sel1 = (lane & 1) ? 0x07030501u : 0x02060004u;
      const uint32_t sel2 = (lane & 2) ? 0x07060302u : 0x01000504u;
#pragma unroll
      for (int j = 0; j < MP::NM; ++j) {
        // INT8: dword j of the lane's run, channels 4j .. 4j+3; 4-bit: the
        // even (j even) or odd channels of dword j/2, as bytes
        uint32_t x;
        if constexpr (fmt_int4(FMT)) {
          const uint32_t wv = r.vr[(j / 2) / NWD].w[(j / 2) % NWD];
          x = (j % 2 ? wv >> 4 : wv) & 0x0F0F0F0Fu;
        } else {
          x = r.vr[j / 4].w[j % 4];
        }
        const short4v vb = codes_bf16(quad_transpose_bytes(x, sel1, sel2));
        mf_acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(wa2, vb, mf_acc[j], 0, 0, 0);
        mf_acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(wa1, vb, mf_acc[j], 0, 0, 0);
        mf_acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(wa0, vb, mf_acc[j], 0, 0, 0);
      }
      return;
    }
    // Padding slots of a partial last page hold no data (possibly NaN bits):
    // zero their values and scale/zero with per-lane selects.  A branch that
    // rewrote the loaded registers would make the compiler wait for every
    // outstanding load, including the prefetched tiles, at its join.
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const bool pad = i * TPL + tg >= nvalid;
#pragma unroll
      for (int k = 0; k < NWD; ++k) r.vr[i].w[k] = pad ? 0u : r.vr[i].w[k];
      if constexpr (FMT != kFp16) {
        r.pr[i].z = pad ? 0.0f : r.pr[i].z;
        r.pr[i].w = pad ? 0.0f : r.pr[i].w;
      }
    }
    // logits
    float lg[G][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t* kw = r.kr[i].w;
      float dot[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) dot[hh] = 0.0f;
#pragma unroll
      for (int d4 = 0; d4 < NWD; ++d4) {
        if constexpr (fmt_int4(FMT)) {  // word d4: channels 8 d4 .. 8 d4 + 7 of the lane's run
          const uint32_t lo = kw[d4] & 0x0F0F0F0Fu, hi = (kw[d4] >> 4) & 0x0F0F0F0Fu;
          const half2v k02 = minus_1024(__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u));
          const half2v k46 = minus_1024(__builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u));
          const half2v k13 = minus_1024(__builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u));
          const half2v k57 = minus_1024(__builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u));
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            dot[hh] = __builtin_amdgcn_fdot2(k02, qh[hh][4 * d4 + 0], dot[hh], false);
            dot[hh] = __builtin_amdgcn_fdot2(k46, qh[hh][4 * d4 + 1], dot[hh], false);
            dot[hh] = __builtin_amdgcn_fdot2(k13, qh[hh][4 * d4 + 2], dot[hh], false);
            dot[hh] = __builtin_amdgcn_fdot2(k57, qh[hh][4 * d4 + 3], dot[hh], false);
          }
        } else if constexpr (FMT == kFp16) {
#pragma unroll
          for (int hh = 0; hh < G; ++hh) dot[hh] = __builtin_amdgcn_fdot2(as_half2(kw[d4]), qh[hh][d4], dot[hh], false);
        } else {
          const half2v lo = minus_1024(__builtin_amdgcn_perm(0x64646464u, kw[d4], 0x04010400u));
          const half2v hi = minus_1024(__builtin_amdgcn_perm(0x64646464u, kw[d4], 0x04030402u));
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            dot[hh] = __builtin_amdgcn_fdot2(lo, qh[hh][2 * d4], dot[hh], false);
            dot[hh] = __builtin_amdgcn_fdot2(hi, qh[hh][2 * d4 + 1], dot[hh], false);
          }
        }
      }
      const bool valid = i * TPL + tg < nvalid;
      float zz = 0.0f;
      if constexpr (FMT != kFp16) zz = r.pr[i].y;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float part = dot[hh];
        if constexpr (FMT != kFp16) part = __builtin_fmaf(r.pr[i].x, dot[hh], zz * qsum[hh]);
        part = sum_contig<LPT>(part);
        lg[hh][i] = valid ? part * a.scale_log2 : -INFINITY;
      }
    }
    // values, decoded once for the G heads
    float vf[NL][CH];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t* vw = r.vr[i].w;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if constexpr (fmt_int4(FMT))
          vf[i][c] = (float)((vw[c / 8] >> (4 * (c % 8))) & 0xFu);
        else if constexpr (FMT == kFp16)
          vf[i][c] = half_bits_to_float((vw[c / 2] >> (16 * (c % 2))) & 0xFFFFu);
        else
          vf[i][c] = byte_to_float(vw[c / 4], c % 4);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float mx = lg[hh][0];
#pragma unroll
      for (int i = 1; i < NL; ++i) mx = fmaxf(mx, lg[hh][i]);
      const bool need = mx > m[hh] + kLazy;
      if (__ballot(need)) {  // wave-uniform branch; rare once the max settles
        const float mn = need ? mx : m[hh];
        const float alpha = mn == m[hh] ? 1.0f : __builtin_amdgcn_exp2f(m[hh] - mn);
        l[hh] *= alpha;
        zacc[hh] *= alpha;
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[hh][c] *= alpha;
        m[hh] = mn;
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float p = lg[hh][i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(lg[hh][i] - m[hh]);
        l[hh] += p;
        if constexpr (FMT == kFp16) {
#pragma unroll
          for (int c = 0; c < CH; ++c) acc[hh][c] = __builtin_fmaf(p, vf[i][c], acc[hh][c]);
        } else {
          const float ps = p * r.pr[i].z;
          zacc[hh] = __builtin_fmaf(p, r.pr[i].w, zacc[hh]);
#pragma unroll
          for (int c = 0; c < CH; ++c) acc[hh][c] = __builtin_fmaf(ps, vf[i][c], acc[hh][c]);
        }
      }
    }
  };

  for (int k0 = 0; k0 < nw; k0 += 64) {
    // page ids with one lane each (the first 64 come from the prologue)
    int jlog_v = jlog0, phys_v = phys0;
    if (k0 > 0) {  // wave-uniform; only when a split gives a wave more than 64 pages
      // clamped to the split's last page: a slot past the wave's count reads
      // some page of this split (its load is never used), and the in-kernel
      // list holds only the split's n entries
      const int idx = min(first + w + (k0 + lane) * NW, first + n - 1);
      if constexpr (SEL)
        jlog_v = list[idx - first];
      else
        jlog_v = sparse ? min(max(a.sel_pages[(size_t)row * a.k_cap + idx], 0), a.max_pages - 1) : idx;
      phys_v = a.block_table[(size_t)b * a.max_pages + jlog_v];
    }
    int cnt = min(64, nw - k0);
    if constexpr (PH != 0) {  // this phase's pool only
      cnt = pool_filter<PH>(jlog_v, phys_v, cnt, a.n16);
      if (cnt == 0) continue;  // wave-uniform
    }
    // Software pipeline over a ring of R = PF + 1 register tiles: the loads of
    // tiles k+1 .. k+PF are in flight while tile k is consumed.
    // Every load is unconditional (an index past the chunk re-reads its last
    // tile, which is cached), so the compiler's wait counts stay exact; a
    // conditional load would make it wait for all outstanding loads.  The main
    // loop is unrolled by R so ring indices are compile-time constants.
    constexpr int PF = kPrefetch;
    constexpr int R = PF + 1;
    PageRegs ring[R];
    auto load_idx = [&](int k, PageRegs& r) {
      const int kk = min(k, cnt - 1);
      load_page(__builtin_amdgcn_readlane(jlog_v, kk), __builtin_amdgcn_readlane(phys_v, kk), r);
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) load_idx(u, ring[u]);
    int k = 0;
    for (; k + R <= cnt; k += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        load_idx(k + u + PF, ring[(u + PF) % R]);
        consume_page(ring[u]);
      }
    }
    // fewer than R tiles remain; they are already in ring[0 ..] (no loads here)
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (k + u < cnt) consume_page(ring[u]);
  }

  // ---- merge the token groups of the wave (lanes congruent mod LPT)
#pragma unroll
  for (int hh = 0; hh < (MF ? 0 : G); ++hh) {
    const float M = max_strided<LPT>(m[hh]);
    const float f = m[hh] == -INFINITY ? 0.0f : exp2f(m[hh] - M);
    l[hh] = sum_strided<LPT>(l[hh] * f);
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[hh][c] = sum_strided<LPT>((acc[hh][c] + zacc[hh]) * f);
    m[hh] = M;
  }

  // ---- merge the block's waves through LDS and write the split's partials
  // (a mixed cache's phases fill slots [0, NW) and [NW, 2 NW))
  constexpr int NWS = PH == 0 ? NW : 2 * NW;
  WaveParts<G, D, NWS>* const parts = wave_parts<G, D, NWS>();
  float(*const sm_ml)[G][2] = parts->ml + (PH == 2 ? NW : 0);
  float(*const sm_acc)[G][D] = parts->acc + (PH == 2 ? NW : 0);
  if constexpr (MF) {
    // (l, z) of head lane%16 summed over its four lanes; O[h][c] = acc + z,
    // lane l register i holding head 4(l/16) + i at channel
    // (D/4)(n/4) + 4j + n%4 of MFMA j, n = l%16
    mf_l += __shfl_xor(mf_l, 16, kWave);
    mf_l += __shfl_xor(mf_l, 32, kWave);
    mf_z += __shfl_xor(mf_z, 16, kWave);
    mf_z += __shfl_xor(mf_z, 32, kWave);
    const int hn = lane & 15, g4 = lane >> 4;
    if (lane < G) {
      sm_ml[w][lane][0] = mf_m;
      sm_ml[w][lane][1] = mf_l;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * g4 + i;
      const float zh = __shfl(mf_z, hh, kWave);
      if (hh < G) {
#pragma unroll
        for (int j = 0; j < MP::NM; ++j) {
          // column n = hn of MFMA j: channel (D/4)(n/4) + 4j + n%4 (INT8), or
          // (D/4)(n/4) + 8(j/2) + 2(n%4) + j%2 (4-bit, even then odd channels)
          const int ch = fmt_int4(FMT) ? (D / 4) * (hn >> 2) + 8 * (j >> 1) + 2 * (hn & 3) + (j & 1)
                                       : (D / 4) * (hn >> 2) + 4 * j + (hn & 3);
          sm_acc[w][hh][ch] = FMT == kFp16 ? mf_acc[j][i] * 0.0078125f : mf_acc[j][i] + zh;  // fp16: 2^-7
        }
      }
    }
  } else if (tg == 0) {
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
  if constexpr (PH == 1) return;  // the second phase merges
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += NW * 64) {
    const int hh = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NWS; ++v) M = fmaxf(M, parts->ml[v][hh][0]);
    float sa = 0.0f, sl = 0.0f;
#pragma unroll
    for (int v = 0; v < NWS; ++v) {
      const float mv = parts->ml[v][hh][0];
      const float f = mv == -INFINITY ? 0.0f : exp2f(mv - M);  // 0 for a wave without pages
      sa = __builtin_fmaf(f, parts->acc[v][hh][c], sa);
      sl = __builtin_fmaf(f, parts->ml[v][hh][1], sl);
    }
    if (!COH && a.direct) {  // the row's only split: out = acc / l, as the combine would write it
      a.out[((size_t)b * a.Hq + g * G + hh) * D + c] = sl > 0.0f ? sa / sl : 0.0f;
      continue;
    }
    const size_t prow = ((size_t)b * a.Hq + g * G + hh) * a.max_splits + s;
    store_f<COH>(a.part_acc + prow * D + c, sa);
    if (c == 0) {
      store_f<COH>(a.part_ml + prow * 2 + 0, M);
      store_f<COH>(a.part_ml + prow * 2 + 1, sl);
    }
  }
  if constexpr (COH) {  // the partials are in memory, and the LDS above free for the caller's next item
    stores_done();
    __syncthreads();
  }
}

}  // namespace kvq
