// decode_attn.hip -- single-token attention over the selected pages of a
// paged, optionally INT8, KV cache ("TinyServe", lpnh.cn, section 3.1 phases
// 3-4; intelliparadigm.com KV-cache page, section 2.1): the split kernel and
// the split combine as launches of their own, and the launchers.  The
// arithmetic is attn_body.h.
#include <mutex>

#include "attn_body.h"

namespace kvq {
namespace {

// grid (B * Hq), 256 threads: the splits of query head bh = b * Hq + h.
template <int D, int G>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  combine_one<D, G, false>(a, blockIdx.x);
}

// grid (KV head, sequence, split): blocks are dispatched split-major, so a
// ragged batch's full first splits go out first and its shorter last splits
// last, and all splits of a head share the XCD of block id mod 8.  The SEL
// instance's dynamic LDS holds the block's pages (pps entries).
// A mixed-precision cache attends to each split's FP16-pool pages, then its
// INT8-pool pages, and merges the two (attend_split phases 1 and 2).
template <int FMT, int D, int G, int NW, bool SEL>
__global__ __launch_bounds__(NW * 64) void decode_attn_kernel(AttnArgs a) {
  extern __shared__ int sm_dyn[];
  if constexpr (FMT == kMixed) {
    attend_split<kFp16, D, G, NW, SEL, false, 1>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm_dyn);
    attend_split<kInt8Token, D, G, NW, SEL, false, 2>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm_dyn);
  } else {
    attend_split<FMT, D, G, NW, SEL, false>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm_dyn);
  }
}

// Room for dynamic LDS a launch of the SEL kernel has under the device's
// per-block limit (its static LDS taken off), or 0 if that cannot be queried.
// Looked up once per instance and device.
template <int FMT, int D, int G>
size_t sel_lds_room() {
  static std::atomic<long long> memo[kMaxDevices];
  return (size_t)per_device(memo, [] {
    hipFuncAttributes fa{};
    int dev = 0, lim = 0;
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(&decode_attn_kernel<FMT, D, G, kAttnWaves, true>)) !=
            hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        (size_t)lim < fa.sharedSizeBytes)
      return 0LL;
    return (long long)((size_t)lim - fa.sharedSizeBytes);
  });
}

template <int FMT, int D, int G>
hipError_t run(const AttnArgs& a, int B, hipStream_t st) {
  if (a.max_splits > 65535 || B > 65535) return hipErrorInvalidConfiguration;
  dim3 grid(a.H, B, a.max_splits);
  if (a.scores) {
    const size_t dyn = (size_t)a.pps * sizeof(int);
    if (dyn > sel_lds_room<FMT, D, G>()) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_attn_kernel<FMT, D, G, kAttnWaves, true>), grid, dim3(kAttnWaves * 64), dyn, st, a);
  } else {
    hipLaunchKernelGGL((decode_attn_kernel<FMT, D, G, kAttnWaves, false>), grid, dim3(kAttnWaves * 64), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.direct) return e;  // (one split per row: the split kernel wrote out)
  hipLaunchKernelGGL((combine_kernel<D, G>), dim3(B * a.Hq), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int FMT, int D>
hipError_t run_g(const AttnArgs& a, int B, int G, hipStream_t st) {
  switch (G) {
    case 1: return run<FMT, D, 1>(a, B, st);
    case 2: return run<FMT, D, 2>(a, B, st);
    case 4: return run<FMT, D, 4>(a, B, st);
    default: return run<FMT, D, 8>(a, B, st);
  }
}

template <int FMT>
hipError_t run_d(const AttnArgs& a, int B, int D, int G, hipStream_t st) {
  if constexpr (fmt_int4(FMT))
    return run_g<FMT, 128>(a, B, G, st);
  else
    return D == 64 ? run_g<FMT, 64>(a, B, G, st) : run_g<FMT, 128>(a, B, G, st);
}

// Scratch for callers that cannot allocate (kvq_select_decode_attn_noalloc):
// the per-split partials live in this file-scope device array instead of a
// caller's workspace.  Its name is a host-side stand-in, never a device
// address: the address comes from hipGetSymbolAddress, once per device, with
// that device current, and only that address reaches a kernel.
__device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    void* p = nullptr;
    slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    slot.ptr = slot.err == hipSuccess ? p : nullptr;
  });
  *ptr = slot.ptr;
  return slot.err;
}

hipError_t launch_decode_attn(const kvq_cache& c, const kvq_seqs& s, const uint16_t* q, int num_q_heads,
                              const int32_t* sel_pages, const int32_t* sel_count, const InKernelSelect* ks,
                              int k_cap, float sm_scale, int pages_per_split, int max_splits, float* out, void* ws,
                              hipStream_t st) {
  const size_t n_part = (size_t)s.batch * num_q_heads * max_splits;
  float* part_ml = (float*)ws;
  float* part_acc = part_ml + n_part * 2;
  AttnArgs a{c.k_pages, c.v_pages, c.kv_params, s.block_table, s.seq_lens, q,
             ks ? nullptr : sel_pages, ks ? nullptr : sel_count,
             ks ? ks->scores : nullptr, ks ? ks->sel_out : nullptr, ks ? ks->cnt_out : nullptr,
             ks ? ks->rnum : 0, ks ? ks->rden : 1, ks ? ks->k_fixed : 0,
             part_acc, part_ml, out, c.num_kv_heads, num_q_heads, s.max_pages, k_cap,
             pages_per_split, max_splits, sm_scale * 1.4426950408889634f, fp16_pool(c), max_splits == 1};
  const int G = num_q_heads / c.num_kv_heads;
  if (c.format == KVQ_FP16) return run_d<kFp16>(a, s.batch, c.head_dim, G, st);
  if (c.format == KVQ_INT8_TOKEN) return run_d<kInt8Token>(a, s.batch, c.head_dim, G, st);
  if (c.format == KVQ_INT8_GROUP64) return run_d<kInt8Group>(a, s.batch, c.head_dim, G, st);
  if (c.format == KVQ_INT4_TOKEN) return run_d<kInt4Token>(a, s.batch, c.head_dim, G, st);
  if (c.format == KVQ_MIXED_FP16_INT8) return run_d<kMixed>(a, s.batch, c.head_dim, G, st);
  return run_d<kInt4Group>(a, s.batch, c.head_dim, G, st);
}

}  // namespace kvq
