// read_probe.hip -- a plain streaming read of a device buffer: the bandwidth
// an HBM-bound kernel can reach on this GPU, measured beside the decode step's
// kernels.  Not a step of the method.
//
// Each block reads one contiguous 64 KiB run with nontemporal 16-byte loads,
// four in flight per thread, and folds them into one word that is stored only
// if it equals a constant (so the loads stay live but nothing is written in
// practice).  Contiguous runs and the nontemporal hint together are the
// fastest plain read found on this part (grid-stride loops without the hint
// stay near 5.5 TB/s).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kProbeThreads = 256;
constexpr size_t kProbeRun = 4096;  // 16-byte words per block: 64 KiB
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ p, size_t n16,
                                                                   uint32_t* sink) {
  const size_t base = (size_t)blockIdx.x * kProbeRun;
  const size_t end = base + kProbeRun < n16 ? base + kProbeRun : n16;
  size_t i = base + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < end; i += kProbeUnroll * kProbeThreads) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = load_stream_u4(p + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += kProbeThreads) {
    const uint4 a = load_stream_u4(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const size_t blocks = (n16 + kProbeRun - 1) / kProbeRun;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, st, (const uint4*)buf, n16,
                     sink);
  return hipGetLastError();
}

}  // namespace kvq
