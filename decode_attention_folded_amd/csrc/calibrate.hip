// Streaming-read calibration: the HBM read rate a plain kernel reaches on this
// part, the practical ceiling next to the nominal 8 TB/s for the attention and
// score kernels, which stream K/V or page metadata the same way (coalesced
// 16-byte non-temporal loads, several in flight per lane).
//
// Each workgroup step reads one contiguous block of 256 x 8 chunks of 16 bytes
// (32 KiB), lane t taking chunks t, t + 256, ..., eight loads in flight;
// workgroups take consecutive blocks, grid-strided.  The loads are folded with
// XOR, and the fold is written only if it equals a fixed constant, so the
// loads cannot be dropped and the kernel writes (almost) nothing.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace da {
namespace {

constexpr int kCalThreads = 256;
constexpr int kCalInFlight = 8;
constexpr uint32_t kCalMagic = 0x9E3779B9u;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kCalThreads)
    read_calibration_kernel(const u32x4* __restrict__ src, uint64_t n16, uint32_t* sink) {
  constexpr uint64_t kBlock = (uint64_t)kCalThreads * kCalInFlight;  // chunks per block
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  uint32_t acc = 0;
  uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
  for (; i + (kCalInFlight - 1) * kCalThreads < n16; i += stride) {
    u32x4 v[kCalInFlight];
#pragma unroll
    for (int u = 0; u < kCalInFlight; ++u)
      v[u] = __builtin_nontemporal_load(src + i + u * kCalThreads);
#pragma unroll
    for (int u = 0; u < kCalInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // the partial last block, one chunk at a time
  for (; i < n16; i += kCalThreads) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kCalMagic) sink[0] = acc;
}

}  // namespace

int launch_read_calibration(const void* src, uint64_t bytes, uint32_t* sink, void* stream) {
  // 8 workgroups per CU of 256 CUs: every CU streams, with loads in flight
  // from many waves.
  const uint32_t blocks = 2048;
  hipLaunchKernelGGL(read_calibration_kernel, dim3(blocks), dim3(kCalThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4*>(src),
                     bytes / 16, sink);
  return (int)hipGetLastError();
}

}  // namespace da
