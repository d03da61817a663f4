// Achievable streaming-read bandwidth of the device: the yardstick the decode
// attention kernel is compared with besides the nominal HBM peak.  The decode
// step is bound by re-reading the retained key and value rows (Chapter 37,
// "From causal attention to managed LLM inference state", on the
// memory-bandwidth bottleneck of incremental decoding); this kernel does only
// that read, with the same access shape: 256-thread workgroups, each reading
// contiguous 32 KiB units with eight 16-byte non-temporal loads in flight per
// thread.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 8;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4_t* __restrict__ p, int64_t units,
                                                                    unsigned* __restrict__ sink) {
  unsigned acc = 0;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const u32x4_t* q = p + u * (kProbeThreads * kProbeLoads) + threadIdx.x;
    u32x4_t v[kProbeLoads];
#pragma unroll
    for (int k = 0; k < kProbeLoads; ++k) v[k] = __builtin_nontemporal_load(q + k * kProbeThreads);
#pragma unroll
    for (int k = 0; k < kProbeLoads; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  // data-dependent store keeps every load live; taken only for one xor value
  if (acc == 0x9E3779B9u) sink[threadIdx.x & 3] = acc;
}

}  // namespace

int dev_stream_read(const void* buf, int64_t bytes, void* sink, void* stream) {
  const int64_t units = bytes / kProbeUnitBytes;
  const int grid = int(units < 4096 ? units : 4096);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(buf), units, static_cast<unsigned*>(sink));
  return int(hipGetLastError());
}

}  // namespace kvc
