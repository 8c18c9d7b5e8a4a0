// Device-side precondition check (a debugging aid, not part of the method):
// the attention and Quest kernels clamp valid lengths to [0, capacity] and
// mask page-table entries outside the pool, silently.  This kernel counts
// such inputs so that a caller can find them.
//
// One workgroup walks every sequence: its length, and on a paged cache the
// page-table entries of the pages that hold a valid token.  Counts are summed
// with block reductions (no atomics), so the report is deterministic.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "check.h"

namespace da {
namespace {

constexpr int kCheckThreads = 1024;

__device__ __forceinline__ int block_sum(int v, int* red) {
  const int lane = lane_in_wave();
  const int wave = threadIdx.x / kWave;
  v = (int)wave_reduce((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int s = 0;
  for (int w = 0; w < kCheckThreads / kWave; ++w) s += red[w];
  __syncthreads();
  return s;
}

__device__ __forceinline__ int block_min(int v, int* red) {
  const int lane = lane_in_wave();
  const int wave = threadIdx.x / kWave;
  v = (int)wave_reduce((uint32_t)v, [](uint32_t a, uint32_t b) {
    return (int)a < (int)b ? a : b;
  });
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int s = red[0];
  for (int w = 1; w < kCheckThreads / kWave; ++w) s = min(s, red[w]);
  __syncthreads();
  return s;
}

__global__ void __launch_bounds__(kCheckThreads) check_kernel(CheckLaunch a) {
  __shared__ int red[kCheckThreads / kWave];
  int bad_len = 0, bad_page = 0, first = INT32_MAX;
  // lengths: thread t checks sequences t, t + 1024, ...
  for (int b = threadIdx.x; b < a.batch; b += kCheckThreads) {
    const int L = a.seqlens[b];
    if (L < 0 || L > a.capacity) {
      ++bad_len;
      first = min(first, b);
    }
  }
  // page-table entries of the pages that hold a valid token
  if (a.page_table != nullptr) {
    for (int b = 0; b < a.batch; ++b) {
      int L = a.seqlens[b];
      L = L < 0 ? 0 : (L > a.capacity ? a.capacity : L);
      const int pages = (L + (1 << a.page_shift) - 1) >> a.page_shift;
      int bad = 0;
      for (int p = threadIdx.x; p < pages; p += kCheckThreads) {
        const int e = a.page_table[(int64_t)b * a.max_pages + p];
        bad += (e < 0 || (int64_t)e >= a.num_pages) ? 1 : 0;
      }
      if (bad > 0) first = min(first, b);
      bad_page += bad;
    }
  }
  bad_len = block_sum(bad_len, red);
  bad_page = block_sum(bad_page, red);
  first = block_min(first, red);
  if (threadIdx.x == 0) {
    a.report[0] = bad_len;
    a.report[1] = bad_page;
    a.report[2] = first == INT32_MAX ? -1 : first;
    a.report[3] = 0;
  }
}

}  // namespace

int launch_check(const CheckLaunch& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(check_kernel, dim3(1), dim3(kCheckThreads), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace da
