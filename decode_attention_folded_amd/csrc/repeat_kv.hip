// Materialised repeat_kv for gfx950: the copy the folded kernel removes.
//
// [CoreML-GQA] section 2, "Why Does GQA Replicate KV?" (with "expand Is a View,
// but reshape Introduces a Copy"): the GQA reference path turns the
// [B, Hkv, L, D] cache into [B, Hq, L, D] so that query head h reads a copy of
// KV head h / G.  This kernel builds that tensor (valid rows only) so the same
// attention kernel can run on it at G = 1 -- the comparison of the page's
// section 4 (the fold against the materialised copy), run on MI355X.
//
// One workgroup copies a chunk of rows of one (b, kv) unit and writes each
// 16-byte piece to the G heads of the group, so every source byte is read
// from HBM once and written G times (the byte model of the copy: read 1x,
// write Gx).  Sources and destinations are streamed with non-temporal loads
// and stores.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace da {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyRows = 64;  // rows of one unit per workgroup

template <int D>
__global__ void __launch_bounds__(kCopyThreads) repeat_kv_kernel(RepeatLaunch a) {
  constexpr int kChunks = D / 8;                      // 16-byte pieces per row
  constexpr int kRowsPerPass = kCopyThreads / kChunks;
  const int hkv = a.num_kv_heads;
  const uint32_t n_units = (uint32_t)a.batch * (uint32_t)hkv;
  const uint32_t chunk = blockIdx.x / n_units;
  const uint32_t unit = blockIdx.x - chunk * n_units;
  const int b = (int)(unit / (uint32_t)hkv);
  const int kv = (int)(unit - (uint32_t)b * (uint32_t)hkv);
  const int shift = a.page_shift;

  int L = a.seqlens[b];
  L = L < 0 ? 0 : (L > a.capacity ? a.capacity : L);
  const int row0 = (int)chunk * kCopyRows;
  if (row0 >= L) return;
  const int row_end = min(row0 + kCopyRows, L);

  const int piece = threadIdx.x % kChunks;
  const int sub = threadIdx.x / kChunks;
  const int hq = hkv * a.group;
  for (int t = row0 + sub; t < row_end; t += kRowsPerPass) {
    int64_t src;
    if (a.page_table != nullptr) {
      const int phys = a.page_table[(int64_t)b * a.max_pages + (t >> shift)];
      if (phys < 0 || phys >= a.num_pages) continue;  // not a pool page: row left unwritten
      src = (((int64_t)phys * hkv + kv) << shift) * D + (int64_t)(t & ((1 << shift) - 1)) * D;
    } else {
      src = ((int64_t)unit * a.cache_stride + t) * D;
    }
    src += 8 * piece;
    const f16x8 kx = stream_load(reinterpret_cast<const f16*>(a.k) + src);
    const f16x8 vx = stream_load(reinterpret_cast<const f16*>(a.v) + src);
    for (int g = 0; g < a.group; ++g) {
      const int64_t dst = (((int64_t)b * hq + (int64_t)kv * a.group + g) * a.out_capacity + t) * D +
                          8 * piece;
      __builtin_nontemporal_store(kx, reinterpret_cast<f16x8*>(reinterpret_cast<f16*>(a.k_out) + dst));
      __builtin_nontemporal_store(vx, reinterpret_cast<f16x8*>(reinterpret_cast<f16*>(a.v_out) + dst));
    }
  }
}

}  // namespace

int launch_repeat_kv(const RepeatLaunch& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint32_t chunks = (uint32_t)((a.out_capacity + kCopyRows - 1) / kCopyRows);
  const dim3 grid(chunks * (uint32_t)a.batch * (uint32_t)a.num_kv_heads);
  if (a.head_dim == 64) {
    hipLaunchKernelGGL((repeat_kv_kernel<64>), grid, dim3(kCopyThreads), 0, s, a);
  } else if (a.head_dim == 128) {
    hipLaunchKernelGGL((repeat_kv_kernel<128>), grid, dim3(kCopyThreads), 0, s, a);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int repeat_kv_rows_per_workgroup() { return kCopyRows; }

}  // namespace da
