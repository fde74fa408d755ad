// kvq_device.h -- device helpers shared by the gfx950 kernels of libkvq.
//
// Wave64 reductions use DPP row operations inside a row of 16 lanes and
// ds_bpermute (__shfl_xor) across rows; the sums and extrema are all-reduce
// (every participating lane ends with the result).  Scans and min/max over a
// whole wave stay in DPP and readlane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kPage = 16;
constexpr int kWave = 64;

// kMixed: an FP16 pool of pages and an INT8-per-token pool in one cache.
enum Format : int { kFp16 = 0, kInt8Token = 1, kInt8Group = 2, kInt4Token = 3, kInt4Group = 4, kMixed = 5 };

// One (scale, zero) per token slot, or per 64-token group; 4-bit codes (two
// per byte, channel 2i in the low nibble of byte i); the largest code.
constexpr bool fmt_token(int f) { return f == kInt8Token || f == kInt4Token; }
constexpr bool fmt_group(int f) { return f == kInt8Group || f == kInt4Group; }
constexpr bool fmt_int4(int f) { return f == kInt4Token || f == kInt4Group; }
constexpr int fmt_levels(int f) { return fmt_int4(f) ? 15 : 255; }

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Lanes' DPP controls (row = 16 lanes).
enum : int {
  kDppXor1 = 0xB1,         // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,         // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141,  // lane i <-> 7-i within each 8 lanes
  kDppMirror = 0x140,      // lane i <-> 15-i within each 16 lanes
  kDppRor4 = 0x124,        // row rotate right by 4
  kDppRor8 = 0x128,        // row rotate right by 8
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, kWave); }

// Sum over aligned blocks of W consecutive lanes (W = 1, 2, 4, 8, 16, 32, 64).
template <int W>
__device__ __forceinline__ float sum_contig(float x) {
  if constexpr (W >= 2) x += dpp<kDppXor1>(x);
  if constexpr (W >= 4) x += dpp<kDppXor2>(x);
  if constexpr (W >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (W >= 16) x += dpp<kDppMirror>(x);
  if constexpr (W >= 32) x += shfl_xor(x, 16);
  if constexpr (W >= 64) x += shfl_xor(x, 32);
  return x;
}

template <int W>
__device__ __forceinline__ float max_contig(float x) {
  if constexpr (W >= 2) x = fmaxf(x, dpp<kDppXor1>(x));
  if constexpr (W >= 4) x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (W >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (W >= 16) x = fmaxf(x, dpp<kDppMirror>(x));
  if constexpr (W >= 32) x = fmaxf(x, shfl_xor(x, 16));
  if constexpr (W >= 64) x = fmaxf(x, shfl_xor(x, 32));
  return x;
}

template <int W>
__device__ __forceinline__ float min_contig(float x) {
  if constexpr (W >= 2) x = fminf(x, dpp<kDppXor1>(x));
  if constexpr (W >= 4) x = fminf(x, dpp<kDppXor2>(x));
  if constexpr (W >= 8) x = fminf(x, dpp<kDppHalfMirror>(x));
  if constexpr (W >= 16) x = fminf(x, dpp<kDppMirror>(x));
  if constexpr (W >= 32) x = fminf(x, shfl_xor(x, 16));
  if constexpr (W >= 64) x = fminf(x, shfl_xor(x, 32));
  return x;
}

// Sum over the lanes congruent modulo S (S = 4, 8, 16, 32, 64): the 64/S
// lanes l, l+S, l+2S, ... all end with their total.
template <int S>
__device__ __forceinline__ float sum_strided(float x) {
  static_assert(S >= 4 && S <= 64, "strides 4..64");
  if constexpr (S <= 4) x += dpp<kDppRor4>(x);
  if constexpr (S <= 8) x += dpp<kDppRor8>(x);
  if constexpr (S <= 16) x += shfl_xor(x, 16);
  if constexpr (S <= 32) x += shfl_xor(x, 32);
  return x;
}

template <int S>
__device__ __forceinline__ float max_strided(float x) {
  static_assert(S >= 4 && S <= 64, "strides 4..64");
  if constexpr (S <= 4) x = fmaxf(x, dpp<kDppRor4>(x));
  if constexpr (S <= 8) x = fmaxf(x, dpp<kDppRor8>(x));
  if constexpr (S <= 16) x = fmaxf(x, shfl_xor(x, 16));
  if constexpr (S <= 32) x = fmaxf(x, shfl_xor(x, 32));
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave, DPP only: Hillis-Steele
// inside each row of 16 (row_shr 1, 2, 4, 8), then row_bcast:15 adds row 0's
// total to row 1 and row 2's to row 3, and row_bcast:31 adds lane 31's
// running total to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan_add(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}

// Min / max over the wave: DPP inside each row of 16, then the four row
// results through readlane (wave-uniform result).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u32<kDppXor1>(x));
  x = min(x, dpp_u32<kDppXor2>(x));
  x = min(x, dpp_u32<kDppHalfMirror>(x));
  x = min(x, dpp_u32<kDppMirror>(x));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return min(min(a, b), min(c, d));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<kDppXor1>(x));
  x = max(x, dpp_u32<kDppXor2>(x));
  x = max(x, dpp_u32<kDppHalfMirror>(x));
  x = max(x, dpp_u32<kDppMirror>(x));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return max(max(a, b), max(c, d));
}

// Inclusive prefix sum inside each row of 16 lanes (DPP row_shr 1, 2, 4, 8).
__device__ __forceinline__ int row16_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
  return x;
}

// Lanes below this one whose bit is set in a 64-bit lane mask.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Order-preserving map fp32 -> uint32 (larger float, larger key); -0 == +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A per-sequence (uniform) value read with a vector load, to be made uniform
// with readfirstlane where it is first needed.  A scalar load would do, but
// scalar loads return out of order, so the compiler waits for all of them
// (kernel arguments included) before using any; as a vector load it stays in
// flight beside the other vector loads issued with it.
__device__ __forceinline__ int vload_i32(const int32_t* p, size_t i) {
  int zero;  // a zero the compiler cannot see as uniform, so the load stays a vector load
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  return p[i + zero];
}

// Streaming loads for data a launch reads exactly once (KV tiles,
// their scale/zero, page metadata): the nontemporal hint marks the lines for
// early eviction instead of normal allocation, which on this part raises the
// rate of a plain streaming read from ~5.5 to ~6.3 TB/s (grid-stride) and to
// ~7.1 TB/s when each block reads contiguous runs.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream_u4(const void* p) {
  const u32x4v v = __builtin_nontemporal_load((const u32x4v*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint2 load_stream_u2(const void* p) {
  const u32x2v v = __builtin_nontemporal_load((const u32x2v*)p);
  return make_uint2(v.x, v.y);
}

typedef float f32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float2 load_stream_f2(const float* p) {
  const f32x2v v = __builtin_nontemporal_load((const f32x2v*)p);
  return make_float2(v.x, v.y);
}

__device__ __forceinline__ float4 load_stream_f4(const float* p) {
  const f32x4v v = __builtin_nontemporal_load((const f32x4v*)p);
  return make_float4(v.x, v.y, v.z, v.w);
}

// Loads and stores of data other blocks of the same launch write or read
// (COH = true): device-scope relaxed accesses, which on gfx950 are the sc1
// forms -- a store written through to memory, a load served from memory --
// so no L2 write-back or invalidate is needed for that data.  COH = false:
// ordinary accesses.
template <bool COH>
__device__ __forceinline__ float load_f(const float* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}

template <bool COH>
__device__ __forceinline__ float2 load_f2(const float* p) {
  if constexpr (COH) return make_float2(load_f<true>(p), load_f<true>(p + 1));
  return *(const float2*)p;
}

template <bool COH>
__device__ __forceinline__ void store_f(float* p, float v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

template <bool COH>
__device__ __forceinline__ void store_u32(uint32_t* p, uint32_t v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// Every store this thread issued has completed (reached the level its cache
// policy writes to): the ordering point before a device-scope counter update
// that publishes data written with store_f<true> / store_u32<true>.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Asymmetric min/max quantization of a row with minimum lo and maximum hi to
// codes 0..LEVELS (255: INT8, 15: 4-bit): zero = lo, scale = (hi - lo) /
// LEVELS, code = clamp(rint((x - zero) / scale)) with 1/scale precomputed;
// IEEE fp32, round to nearest even, no contraction, so codes are
// reproducible bit for bit.  A constant row gets scale 1.
template <int LEVELS = 255>
__device__ __forceinline__ void quant_params(float lo, float hi, float& scale, float& inv) {
#pragma clang fp contract(off)
  if (hi > lo) {
    float range = hi - lo;
    scale = range / (float)LEVELS;
    inv = 1.0f / scale;
  } else {
    scale = 1.0f;
    inv = 1.0f;
  }
}

// The zero-point of a row is its minimum, with a minimum of -0 stored as +0
// (x + 0 is +0 for either zero and x otherwise), so the stored bits do not
// depend on which of two equal zeros a min reduction happens to return.
__device__ __forceinline__ float zero_point(float lo) {
#pragma clang fp contract(off)
  return lo + 0.0f;
}

template <int LEVELS = 255>
__device__ __forceinline__ uint32_t quant_code(float x, float zero, float inv) {
#pragma clang fp contract(off)
  float t = (x - zero) * inv;
  float r = __builtin_rintf(t);
  r = fminf(fmaxf(r, 0.0f), (float)LEVELS);
  return (uint32_t)r;
}

// Number of pages selected from P by the ratio / fixed count (integers only).
__host__ __device__ __forceinline__ int num_selected(int P, int rnum, int rden, int k_fixed) {
  if (P <= 0) return 0;
  long long k = k_fixed > 0 ? (long long)k_fixed : ((long long)rnum * P + rden - 1) / rden;
  if (k < 1) k = 1;
  if (k > P) k = P;
  return (int)k;
}

}  // namespace kvq
