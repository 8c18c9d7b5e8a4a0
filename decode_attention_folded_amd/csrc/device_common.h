// Device helpers shared by the gfx950 kernels: fp16 vector types, lane
// exchanges (DPP, ds_swizzle, ds_bpermute) and small wave/block reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace da {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_in_wave() { return threadIdx.x & (kWave - 1); }

// DPP move of a 32-bit value; CTRL is the dpp_ctrl encoding.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// DPP controls used below.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within each 8-lane half row
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within each 16-lane row
constexpr int kDppRor8 = 0x128;        // lane i <- lane (i+8) mod 16 within each row

// Sum / max over aligned groups of N contiguous lanes (N = 8 or 16).  Every
// lane of a group ends with the same, bitwise identical value.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp_f32<kDppXor1>(x);
  x += dpp_f32<kDppXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  if constexpr (N == 16) x += dpp_f32<kDppMirror>(x);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x = fmaxf(x, dpp_f32<kDppXor1>(x));
  x = fmaxf(x, dpp_f32<kDppXor2>(x));
  x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
  if constexpr (N == 16) x = fmaxf(x, dpp_f32<kDppMirror>(x));
  return x;
}

// Value of lane `l` (a wave-uniform index) as a scalar.
__device__ __forceinline__ float read_lane(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Maximum over the 64 lanes of a wave (wave-uniform result): the 16-lane
// row maxima, then the four rows through readlane.
__device__ __forceinline__ float wave_max_f32(float x) {
  x = group_max<16>(x);
  return fmaxf(fmaxf(read_lane(x, 0), read_lane(x, 16)), fmaxf(read_lane(x, 32), read_lane(x, 48)));
}

// Value of lane (lane ^ MASK) for MASK in {8, 16, 32}.
template <int MASK>
__device__ __forceinline__ float lane_xor(float x) {
  int v = __builtin_bit_cast(int, x);
  if constexpr (MASK == 8) {
    v = __builtin_amdgcn_update_dpp(0, v, kDppRor8, 0xF, 0xF, true);
  } else if constexpr (MASK == 16) {
    // ds_swizzle bitmask mode: and 0x1f, or 0, xor 0x10 (within 32 lanes)
    v = __builtin_amdgcn_ds_swizzle(v, (0x10 << 10) | 0x1F);
  } else {
    static_assert(MASK == 32, "xor distance 8, 16 or 32");
    v = __builtin_amdgcn_ds_bpermute((lane_in_wave() ^ 32) << 2, v);
  }
  return __builtin_bit_cast(float, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A load that stays where it is written: a relaxed workgroup-scope atomic
// compiles to an ordinary global load, but keeps its program order with the
// other such loads and is not sunk past a branch into the only path that uses
// it.  For the first loads of a kernel, so that they are in flight before
// anything waits for the rest of the kernel arguments.
template <typename T>
__device__ __forceinline__ T early_load(const T* p) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  using U = typename std::conditional<sizeof(T) == 4, uint32_t, uint64_t>::type;
  const U u = __hip_atomic_load(reinterpret_cast<const U*>(p), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_bit_cast(T, u);
}

// 16-byte load with the non-temporal hint, for data read exactly once.
__device__ __forceinline__ f16x8 stream_load(const f16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(p));
}

template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  // lanes outside the masks, or whose source lane does not exist, read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, BANK_MASK, true);
}

constexpr int kDppRowShr1 = 0x111;     // lane i <- lane i-1 within each 16-lane row
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr3 = 0x113;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row -> every lane of the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> every lane of rows 2 and 3

// Inclusive prefix sum over the 64 lanes of a wave, in DPP steps (no LDS
// round trips): prefix over 4 lanes from three row shifts of the input, then
// 8 and 16 lanes with bank-masked row shifts, then the row totals carried by
// the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  uint32_t x = v + dpp_u32<kDppRowShr1, 0xF, 0xF>(v) + dpp_u32<kDppRowShr2, 0xF, 0xF>(v) +
               dpp_u32<kDppRowShr3, 0xF, 0xF>(v);
  x += dpp_u32<kDppRowShr4, 0xF, 0xE>(x);     // lanes 4..15 of each row
  x += dpp_u32<kDppRowShr8, 0xF, 0xC>(x);     // lanes 8..15 of each row
  x += dpp_u32<kDppRowBcast15, 0xA, 0xF>(x);  // rows 1 and 3
  x += dpp_u32<kDppRowBcast31, 0xC, 0xF>(x);  // rows 2 and 3
  return x;
}

// Reduction over the 64 lanes of a wave with an associative, commutative op;
// the result is wave-uniform.  DPP within each 16-lane row, then the four row
// results through readlane.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
  uint32_t x = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppXor1, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppXor2, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppHalfMirror, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppMirror, 0xF, 0xF, false));
  return op(op((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16)),
            op((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48)));
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

// Exclusive prefix sum over a block of NWAVES waves; *total gets the block
// sum.  Must be reached by every thread of the block.  Without the trailing
// barrier (TRAILING = false) the caller must pass another barrier before
// `scratch` is written again.
template <int NWAVES, bool TRAILING = true>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch,
                                                         uint32_t* total) {
  const int lane = lane_in_wave();
  const int wave = threadIdx.x / kWave;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  uint32_t base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    const uint32_t s = scratch[w];
    if (w < wave) base += s;
    sum += s;
  }
  if constexpr (TRAILING) __syncthreads();
  *total = sum;
  return base + inc - v;
}

}  // namespace da
