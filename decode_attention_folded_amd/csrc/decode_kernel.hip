// Split-context folded-GQA decode attention for gfx950 (MI355X).
//
// What it computes -- [CoreML-GQA] section 3, "Fold Q Instead of Expanding KV"
// and "Implementation": for every (batch b, KV head kv) the G query heads
// h = G*kv + g are treated as G rows of one small matrix, so each K and V row
// is read from HBM once for all G rows (no repeat_kv copy).  Per row:
// s_t = scale * q.k_t for t < L_b, softmax over t, o = sum_t p_t v_t.
// The Quest variant ([Quest-review], paper sections 3.3-3.5) runs the same
// loop over the tokens of the chosen pages only.
//
// Work decomposition (flash-decode): grid = (splits, Hkv, B).  A workgroup of
// 4 waves owns a contiguous chunk of `tiles_per_split` key tiles of one
// (b, kv) unit; its waves take the chunk's tiles round robin.
//
// Lane layout inside a wave (W lanes per key, KT = 64 / W keys per tile):
//   lane = c * KT + r; r = key slot in the tile, c = channel group.
//   Lane (r, c) loads 16-byte chunks W*jj + c (jj < D / (8W)) of key r's K and
//   V rows, so one load instruction covers W*16 contiguous bytes of each of
//   KT keys.  The partial q.k over the lane's channels (v_dot2_f32_f16) is
//   summed over the W lanes of the key with cross-row exchanges; after that
//   all W lanes hold the same score.
//   Each lane keeps its own online-softmax state (running max m, sum l and
//   the fp32 output accumulator for its channels) over the keys that pass
//   through its slot r; the KT slot states are merged once at the end of the
//   chunk (log-sum-exp), then the 4 waves are merged through LDS.
//   Rescaling is lazy: the running max only moves when a score exceeds it by
//   more than 2^8 (in exp2 units), so steady-state tiles do no rescale work.
//
// Split combine: each workgroup writes its (m, l, o) partial; the last
// workgroup of a unit to finish (atomic counter, reset by that workgroup)
// merges all partials in split order and writes the fp16 output.  No
// floating-point atomics: results are bitwise reproducible.
//
// Keys at or past the valid length are never loaded from their slots: their
// loads are redirected to a valid row of the same unit and their scores forced
// to -inf, so whatever the cache holds there (even NaN) cannot leak in.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace da {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kMaxTilesPerSplit = 128;
constexpr int kMinKeysPerTile = 8;
constexpr int kMinPageSize = 8;
// pages (or chosen-page entries) one chunk can touch
constexpr int kMaxChunkPages = kMaxTilesPerSplit * 16 / kMinPageSize + 2;
constexpr float kRescaleThreshold = 8.0f;
constexpr float kNegBig = -1.0e30f;

template <int D, int G>
struct Lanes {
  static constexpr int W = (D == 128 && G == 8) ? 8 : 4;  // lanes per key
  static constexpr int KT = kWave / W;                     // keys per tile
  static constexpr int NC = D / (8 * W);                   // 16-byte chunks per lane
  static constexpr int NV = NC * 8;                        // channels per lane
};

template <int NC>
struct TileRegs {
  f16x8 k[NC];
  f16x8 v[NC];
  bool valid;
};

template <int D, int G, bool PAGED, bool SPARSE>
__global__ void __launch_bounds__(kThreads) decode_kernel(AttnLaunch a) {
  using LN = Lanes<D, G>;
  constexpr int W = LN::W;
  constexpr int KT = LN::KT;
  constexpr int NC = LN::NC;
  constexpr int NV = LN::NV;

  __shared__ float s_o[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ int32_t s_page[(PAGED || SPARSE) ? kMaxChunkPages : 1];
  __shared__ int32_t s_phys[(PAGED && SPARSE) ? kMaxChunkPages : 1];
  __shared__ int s_last;

  const int lane = lane_in_wave();
  const int wave = threadIdx.x / kWave;
  const int r = lane % KT;
  const int c = lane / KT;
  const int split = blockIdx.x;
  const int kv = blockIdx.y;
  const int b = blockIdx.z;
  const int hkv = a.num_kv_heads;
  const int64_t unit = (int64_t)b * hkv + kv;
  const int shift = a.page_shift;
  const int page_mask = (1 << shift) - 1;

  int L = a.seqlens[b];
  L = L < 0 ? 0 : (L > a.capacity ? a.capacity : L);
  int n_keys = L;
  const int n_pages_L = (L + page_mask) >> shift;
  if constexpr (SPARSE) {
    const int nsel = n_pages_L < a.num_sel ? n_pages_L : a.num_sel;
    n_keys = nsel << shift;
  }
  const int n_tiles = (n_keys + KT - 1) / KT;
  const int nsplit = (n_tiles + a.tiles_per_split - 1) / a.tiles_per_split;
  f16* out = reinterpret_cast<f16*>(a.out) + unit * G * D;  // rows h = G*kv + g of batch b

  if (split >= nsplit) {
    if (split == 0) {  // no valid key at all: defined as a zero output
      for (int i = threadIdx.x; i < G * D; i += kThreads) out[i] = (f16)0.0f;
    }
    return;
  }

  const int tile_begin = split * a.tiles_per_split;
  const int tile_end = min(tile_begin + a.tiles_per_split, n_tiles);
  const int key_begin = tile_begin * KT;
  const int key_last = min(tile_end * KT, n_keys) - 1;
  const int page0 = key_begin >> shift;

  // Page lists of this chunk into LDS: the physical page of each logical page
  // (paged cache) and/or the chosen logical pages (selected-page stream).
  if constexpr (PAGED || SPARSE) {
    const int npg = (key_last >> shift) - page0 + 1;
    for (int i = threadIdx.x; i < npg; i += kThreads) {
      int logical = page0 + i;
      if constexpr (SPARSE) logical = a.page_idx[unit * a.num_sel + page0 + i];
      if constexpr (SPARSE) {
        // a chosen page must exist: 0 <= page < ceil(L / S); anything else
        // is masked (-1) so that no address is formed from it
        if (logical < 0 || logical >= n_pages_L) logical = -1;
      }
      int entry = logical;
      if constexpr (PAGED) {
        int phys = -1;
        if (logical >= 0 && logical < a.max_pages) {
          phys = a.page_table[(int64_t)b * a.max_pages + logical];
          if (phys < 0 || phys >= a.num_pages) phys = -1;
        }
        if constexpr (SPARSE) {
          s_phys[i] = phys;
        } else {
          entry = phys;
        }
      }
      s_page[i] = entry;
    }
    __syncthreads();
  }

  // Masked keys load a row that holds this sequence's data (token 0, valid
  // because L >= 1 here) instead of their own slot, so the value multiplied by
  // their zero weight is finite.  A page-table entry outside the pool falls
  // back to pool page 0, which always exists.
  int64_t safe_off;
  if constexpr (PAGED) {
    int phys0 = a.page_table[(int64_t)b * a.max_pages];
    if (phys0 < 0 || phys0 >= a.num_pages) phys0 = 0;
    safe_off = (((int64_t)phys0 * hkv + kv) << shift) * D;
  } else {
    safe_off = unit * a.cache_stride * D;
  }

  const f16* kc = reinterpret_cast<const f16*>(a.k);
  const f16* vc = reinterpret_cast<const f16*>(a.v);
  const bool has_new = a.k_new != nullptr;
  const f16* knew_row = has_new ? reinterpret_cast<const f16*>(a.k_new) + unit * D : nullptr;
  const f16* vnew_row = has_new ? reinterpret_cast<const f16*>(a.v_new) + unit * D : nullptr;

  // Folded queries: G rows of this KV head, the lane's channels only.
  const f16* qb = reinterpret_cast<const f16*>(a.q) + unit * G * D;
  f16x8 qr[G][NC];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int jj = 0; jj < NC; ++jj)
      qr[g][jj] = *reinterpret_cast<const f16x8*>(qb + g * D + 8 * (W * jj + c));

  float m[G], l[G], acc[G][NV];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegBig;
    l[g] = 0.0f;
#pragma unroll
    for (int x = 0; x < NV; ++x) acc[g][x] = 0.0f;
  }

  auto load_tile = [&](int tile, TileRegs<NC>& T) {
    const int j = tile * KT + r;  // position in this unit's key stream
    int t = j;                    // token position in the sequence
    bool valid = j < n_keys;
    int64_t off;
    if constexpr (SPARSE) {
      const int li = (j >> shift) - page0;
      const int logical = valid ? s_page[li] : 0;
      t = (logical << shift) + (j & page_mask);
      valid = valid && logical >= 0 && t < L;
      if constexpr (PAGED) {
        const int phys = valid ? s_phys[li] : -1;
        valid = valid && phys >= 0;
        off = (((int64_t)phys * hkv + kv) << shift) * D + (int64_t)(t & page_mask) * D;
      } else {
        off = (unit * a.cache_stride + t) * D;
      }
    } else if constexpr (PAGED) {
      const int phys = valid ? s_page[(j >> shift) - page0] : -1;
      valid = valid && phys >= 0;
      off = (((int64_t)phys * hkv + kv) << shift) * D + (int64_t)(t & page_mask) * D;
    } else {
      off = (unit * a.cache_stride + t) * D;
    }
    if (!valid) off = safe_off;
    T.valid = valid;
    const bool is_new = has_new && valid && t == L - 1;
    const f16* kp = kc + off;
    const f16* vp = vc + off;
    if (is_new) {
      kp = knew_row;
      vp = vnew_row;
    }
#pragma unroll
    for (int jj = 0; jj < NC; ++jj) {
      T.k[jj] = *reinterpret_cast<const f16x8*>(kp + 8 * (W * jj + c));
      T.v[jj] = *reinterpret_cast<const f16x8*>(vp + 8 * (W * jj + c));
    }
    if (is_new) {  // append: the new row goes to slot L - 1 of the cache
      f16* kd = reinterpret_cast<f16*>(a.k) + off;
      f16* vd = reinterpret_cast<f16*>(a.v) + off;
#pragma unroll
      for (int jj = 0; jj < NC; ++jj) {
        *reinterpret_cast<f16x8*>(kd + 8 * (W * jj + c)) = T.k[jj];
        *reinterpret_cast<f16x8*>(vd + 8 * (W * jj + c)) = T.v[jj];
      }
    }
  };

  auto compute_tile = [&](const TileRegs<NC>& T) {
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x = 0.0f;
#pragma unroll
      for (int jj = 0; jj < NC; ++jj) x = dot8(qr[g][jj], T.k[jj], x);
      // sum over the W lanes of this key
      if constexpr (W == 8) x += lane_xor<8>(x);
      x += lane_xor<16>(x);
      x += lane_xor<32>(x);
      s[g] = T.valid ? x * a.scale_log2 : -INFINITY;
    }
    bool need = false;
#pragma unroll
    for (int g = 0; g < G; ++g) need |= s[g] > m[g] + kRescaleThreshold;
    if (need) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(m[g], s[g]);
        const float f = fast_exp2(m[g] - mn);
        l[g] *= f;
#pragma unroll
        for (int x = 0; x < NV; ++x) acc[g][x] *= f;
        m[g] = mn;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = fast_exp2(s[g] - m[g]);
      l[g] += p;
#pragma unroll
      for (int jj = 0; jj < NC; ++jj)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[g][jj * 8 + e] = fmaf(p, (float)T.v[jj][e], acc[g][jj * 8 + e]);
    }
  };

  // Two register buffers: the next tile's loads are in flight while the
  // current tile is computed.
  {
    TileRegs<NC> A, B;
    int tile = tile_begin + wave;
    if (tile < tile_end) {
      load_tile(tile, A);
      while (true) {
        const int t1 = tile + kWaves;
        if (t1 < tile_end) load_tile(t1, B);
        compute_tile(A);
        if (t1 >= tile_end) break;
        const int t2 = t1 + kWaves;
        if (t2 < tile_end) load_tile(t2, A);
        compute_tile(B);
        if (t2 >= tile_end) break;
        tile = t2;
      }
    }
  }

  // Merge the KT key slots of each channel group (log-sum-exp).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = group_max<KT>(m[g]);
    const float f = fast_exp2(m[g] - M);
    l[g] = group_sum<KT>(l[g] * f);
#pragma unroll
    for (int x = 0; x < NV; ++x) acc[g][x] = group_sum<KT>(acc[g][x] * f);
    m[g] = M;
  }
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int jj = 0; jj < NC; ++jj) {
        float* dst = &s_o[wave][g][8 * (W * jj + c)];
        *reinterpret_cast<f32x4*>(dst) =
            f32x4{acc[g][jj * 8 + 0], acc[g][jj * 8 + 1], acc[g][jj * 8 + 2], acc[g][jj * 8 + 3]};
        *reinterpret_cast<f32x4*>(dst + 4) =
            f32x4{acc[g][jj * 8 + 4], acc[g][jj * 8 + 5], acc[g][jj * 8 + 6], acc[g][jj * 8 + 7]};
      }
      if (c == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();

  // Merge the waves of this workgroup.
  float* part_o = a.part_o + (unit * a.max_splits + split) * G * D;
  float* part_ml = a.part_ml + (unit * a.max_splits + split) * G * 2;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int g = i / D;
    const int d = i % D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float o = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][g] - M);
      o += f * s_o[w][g][d];
      lsum += f * s_l[w][g];
    }
    if (nsplit == 1) {
      out[i] = (f16)(lsum > 0.0f ? o / lsum : 0.0f);
    } else {
      part_o[i] = o;
      if (d == 0) {
        part_ml[2 * g] = M;
        part_ml[2 * g + 1] = lsum;
      }
    }
  }
  if (nsplit == 1) return;

  // Publish this split; the last one of the unit combines all of them.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(&a.counters[unit], 1u);
    s_last = prev == (unsigned)(nsplit - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const float* all_o = a.part_o + unit * a.max_splits * G * D;
  const float* all_ml = a.part_ml + unit * a.max_splits * G * 2;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int g = i / D;
    float M = kNegBig;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, all_ml[(sp * G + g) * 2]);
    float o = 0.0f, lsum = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float f = fast_exp2(all_ml[(sp * G + g) * 2] - M);
      o += f * all_o[sp * G * D + i];
      lsum += f * all_ml[(sp * G + g) * 2 + 1];
    }
    out[i] = (f16)(lsum > 0.0f ? o / lsum : 0.0f);
  }
  if (threadIdx.x == 0) a.counters[unit] = 0u;
}

template <int D, int G, bool PAGED, bool SPARSE>
int launch_one(const AttnLaunch& a, hipStream_t stream) {
  dim3 grid(a.max_splits, a.num_kv_heads, a.batch);
  hipLaunchKernelGGL((decode_kernel<D, G, PAGED, SPARSE>), grid, dim3(kThreads), 0, stream, a);
  return (int)hipGetLastError();
}

template <int D, int G>
int launch_dg(const AttnLaunch& a, hipStream_t s) {
  const bool paged = a.page_table != nullptr;
  const bool sparse = a.page_idx != nullptr;
  if (paged) return sparse ? launch_one<D, G, true, true>(a, s) : launch_one<D, G, true, false>(a, s);
  return sparse ? launch_one<D, G, false, true>(a, s) : launch_one<D, G, false, false>(a, s);
}

template <int D>
int launch_d(const AttnLaunch& a, hipStream_t s) {
  switch (a.group) {
    case 1: return launch_dg<D, 1>(a, s);
    case 2: return launch_dg<D, 2>(a, s);
    case 4: return launch_dg<D, 4>(a, s);
    case 8: return launch_dg<D, 8>(a, s);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

int keys_per_tile(int head_dim, int group) {
  return (head_dim == 128 && group == 8) ? kWave / 8 : kWave / 4;
}

int max_tiles_per_split() { return kMaxTilesPerSplit; }

int launch_decode(const AttnLaunch& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.head_dim == 64) return launch_d<64>(a, s);
  if (a.head_dim == 128) return launch_d<128>(a, s);
  return (int)hipErrorInvalidValue;
}

static_assert(kMinKeysPerTile == 8, "tile sizes are 8 or 16 keys");

}  // namespace da
