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

#include "kvc_dev_util.h"
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

// Achievable bf16 matrix-core rate, the yardstick of the chunk projection and
// chunk attention besides the nominal peak: every wave issues rounds of
// kMfmaChains independent 32x32x16 bf16 MFMAs on register operands, with no
// memory traffic inside the loop, so the time is the matrix cores' own.
constexpr int kMfmaChains = 8;
constexpr int kMfmaWavesPerBlock = 4;

__global__ __launch_bounds__(64 * kMfmaWavesPerBlock) void mfma_rate_kernel(int64_t iters, float* __restrict__ sink) {
  using namespace dev;
  Frag8 a, b;
  // small finite operands (bf16 1/64 and 1/32): sums stay far from overflow
  a.u = make_uint4(0x3C803C80u, 0x3C803C80u, 0x3C803C80u, 0x3C803C80u);
  b.u = make_uint4(0x3D003D00u, 0x3D003D00u, 0x3D003D00u, 0x3D003D00u);
  f32x16_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = float(c);
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = mfma32(a.v, b.v, acc[c]);
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[c][r];
  // a value-dependent store keeps every product live; taken only for one sum
  if (sum == -1.0f) sink[threadIdx.x & 3] = sum;
}

}  // namespace

int dev_mfma_rate(int64_t iterations, void* sink, void* stream, double* flops) {
  int units = 0;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&units, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return int(e);
  // two waves per SIMD on every compute unit
  const int blocks = units * 8 / kMfmaWavesPerBlock;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(64 * kMfmaWavesPerBlock), 0,
                     static_cast<hipStream_t>(stream), iterations, static_cast<float*>(sink));
  *flops = double(blocks) * kMfmaWavesPerBlock * double(iterations) * kMfmaChains * (2.0 * 32 * 32 * 16);
  return int(hipGetLastError());
}

int dev_stream_read(const void* buf, int64_t bytes, void* sink, void* stream) {
  const int64_t units = bytes / kProbeUnitBytes;
  const int grid = int(units < 4096 ? units : 4096);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(buf), units, static_cast<unsigned*>(sink));
  return int(hipGetLastError());
}

}  // namespace kvc
