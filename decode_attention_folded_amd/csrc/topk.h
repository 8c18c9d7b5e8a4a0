// Top-K page selection of one (b, kv) unit by one 256-thread workgroup, shared
// by the top-K kernel and the attention kernel that selects its own pages
// ([Quest-review] paper section 3.4: keep the K pages with the largest page
// score; ties to the lower page index; ascending page order).  Device code
// only.

#ifndef DA_TOPK_H
#define DA_TOPK_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"

namespace da {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kRadixBits = 11;
constexpr int kMaxRankCand = 64;  // boundary candidates resolved by exact ranking

__device__ __forceinline__ uint32_t order_key(float f) {
  // Larger float -> larger key; -0 is folded into +0 first.
  const uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-K of one (b, kv) unit's page scores by one workgroup of 256 threads.
// Thread t holds items i = k * 256 + t (k < R), raw[k] = score of item i
// (anything past the valid pages, which are masked); the selected set is kept
// as an LDS bitmap (item i in word i / 32).
//   1. keys = order-preserving u32 of the scores; skip the bits shared by the
//      smallest and largest key;
//   2. radix passes on 11-bit digits: LDS histogram of the remaining
//      candidates, boundary digit by a digit-descending block scan; items
//      above it are taken, below it dropped;
//   3. once at most 64 candidates tie on the boundary, each is ranked exactly
//      by (key descending, index ascending); if all 32 key bits are used up
//      with more candidates, the lowest indices win;
//   4. the bitmap is compacted in index order: emit(pos, page) for the K
//      output positions, ascending pages, then -1 for pad positions.
// Requires n_pages > K (otherwise every page is chosen: see choose_all).
// Integer-only decisions, so every workgroup that runs it on the same scores
// makes the same choice.
template <int R, typename Emit>
__device__ __forceinline__ void select_top_k(const float (&raw)[R], int n_pages, int K, Emit emit) {
  static_assert(R >= 8 && R <= 64 && R % 8 == 0, "items per thread");
  constexpr int NW = R * kTopkThreads / 32;                      // bitmap words
  constexpr int WPT = (NW + kTopkThreads - 1) / kTopkThreads;    // words per thread
  __shared__ uint32_t hist[1 << kRadixBits];
  __shared__ uint32_t info[3];
  __shared__ uint32_t scratch[kTopkWaves];
  __shared__ uint32_t red_min[kTopkWaves], red_max[kTopkWaves];
  __shared__ uint32_t selbits[NW];
  __shared__ uint32_t candbits[NW];
  __shared__ uint32_t ckey[kMaxRankCand];
  __shared__ int32_t cidx[kMaxRankCand];

  // one bit per item of the thread: 32-bit masks while they suffice
  using Mask = typename std::conditional<(R <= 32), uint32_t, uint64_t>::type;
  const int tid = threadIdx.x;
  const int lane = lane_in_wave();
  const int wave = tid / kWave;
  uint32_t key[R];
  Mask cand = 0;   // bit k: item k is still a candidate
  Mask take = 0;   // bit k: item k is chosen
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const bool valid = k * kTopkThreads + tid < n_pages;
    const uint32_t kk = order_key(raw[k]);
    key[k] = valid ? kk : 0u;
    cand |= (Mask)valid << k;
    kmin = min(kmin, valid ? kk : 0xFFFFFFFFu);
    kmax = max(kmax, valid ? kk : 0u);
  }
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  if (lane == 0) {
    red_min[wave] = kmin;
    red_max[wave] = kmax;
  }
  // the first pass's histogram and the bitmap are cleared under the same
  // barrier
  for (int i = tid; i < (1 << kRadixBits); i += kTopkThreads) hist[i] = 0u;
  for (int w = tid; w < NW; w += kTopkThreads) selbits[w] = 0u;
  __syncthreads();
  kmin = red_min[0];
  kmax = red_max[0];
#pragma unroll
  for (int w = 1; w < kTopkWaves; ++w) {
    kmin = min(kmin, red_min[w]);
    kmax = max(kmax, red_max[w]);
  }
  const uint32_t diff = kmin ^ kmax;
  int shift = diff ? 32 - __builtin_clz(diff) : 0;  // bits below the common prefix
  uint32_t need = (uint32_t)K;
  uint32_t ncand = (uint32_t)n_pages;

  bool first = true;
  while (need > 0 && need < ncand && shift > 0 && ncand > (uint32_t)kMaxRankCand) {
    const int nb = shift < kRadixBits ? shift : kRadixBits;
    shift -= nb;
    const uint32_t nbins = 1u << nb;
    if (first) {  // every valid item is a candidate: no per-slot test
#pragma unroll
      for (int k = 0; k < R; ++k)
        atomicAdd(&hist[(key[k] >> shift) & (nbins - 1)], ((cand >> k) & 1) ? 1u : 0u);
    } else {
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const bool c = (cand >> k) & 1;
        if (__ballot(c) != 0)  // wave-uniform: skip slots with no candidate
          atomicAdd(&hist[(key[k] >> shift) & (nbins - 1)], c ? 1u : 0u);
      }
    }
    first = false;
    __syncthreads();
    // thread t sums a run of `per` digits taken from the top digit down,
    // keeping the counts in registers for the boundary search
    constexpr int kPerMax = (1 << kRadixBits) / kTopkThreads;
    const int per = (int)((nbins + kTopkThreads - 1) / kTopkThreads);
    uint32_t cnt[kPerMax];
    uint32_t run = 0;
#pragma unroll
    for (int q = 0; q < kPerMax; ++q) {
      const int dgt = (int)nbins - 1 - (tid * per + q);
      cnt[q] = (q < per && dgt >= 0) ? hist[dgt] : 0u;
      run += cnt[q];
    }
    uint32_t total;
    // (the barrier after the boundary search also guards `scratch`)
    const uint32_t before = block_exclusive_scan<kTopkWaves, false>(run, scratch, &total);
    if (before < need && need <= before + run) {
      uint32_t acc = before;
      bool found = false;
#pragma unroll
      for (int q = 0; q < kPerMax; ++q) {
        if (!found && acc + cnt[q] >= need) {
          info[0] = (uint32_t)((int)nbins - 1 - (tid * per + q));  // boundary digit
          info[1] = acc;                                           // candidates above it
          info[2] = cnt[q];                                        // candidates on it
          found = true;
        }
        acc += cnt[q];
      }
    }
    __syncthreads();
    const uint32_t dstar = info[0];
    const uint32_t above = info[1];
    const uint32_t on = info[2];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const uint32_t dg = (key[k] >> shift) & (nbins - 1);
      const Mask bit = (Mask)1 << k;
      if (dg > dstar) take |= cand & bit;
      if (dg != dstar) cand &= ~bit;
    }
    need -= above;
    ncand = on;
    if (need > 0 && need < ncand && shift > 0 && ncand > (uint32_t)kMaxRankCand) {
      // another pass: its histogram (nobody reads this one any more)
      for (int i = tid; i < (int)nbins; i += kTopkThreads) hist[i] = 0u;
      __syncthreads();  // hist and info are reused by the next pass
    }
  }
  if (need >= ncand) {  // the remaining candidates all fit
    take |= cand;
    cand = 0;
  }

  // chosen items -> bitmap: each thread sets the bits of its own chosen
  // items (K of all items, so about K / 256 per thread)
  for (Mask t = take; t != 0; t &= t - 1) {
    const int i = __builtin_ctzll((uint64_t)t) * kTopkThreads + tid;
    atomicOr(&selbits[i >> 5], 1u << (i & 31));
  }
  __syncthreads();

  if (need > 0 && need < ncand) {
    if (ncand <= (uint32_t)kMaxRankCand) {
      // exact ranking of the boundary candidates by (key desc, index asc):
      // list them in LDS, each thread at the block prefix of its candidate
      // count (plain stores; an LDS atomic per slot costs a round trip each),
      // then rank each one
      uint32_t listed_total;
      uint32_t pos = block_exclusive_scan<kTopkWaves, false>(
          (uint32_t)__builtin_popcountll(cand), scratch, &listed_total);
#pragma unroll
      for (int k = 0; k < R; ++k) {
        if ((cand >> k) & 1) {  // ncand <= 64 candidates exist: pos < 64
          ckey[pos] = key[k];
          cidx[pos] = k * kTopkThreads + tid;
          ++pos;
        }
      }
      __syncthreads();
      // four threads per candidate (a quad), each comparing it with a
      // quarter of the list; the quad's counts add up through DPP
      constexpr int kPerPart = kMaxRankCand / 4;
      const int c = tid >> 2;
      const int part = tid & 3;
      const bool has = c < (int)ncand;
      const uint32_t kc = has ? ckey[c] : 0u;
      const int ic = has ? cidx[c] : 0x7FFFFFFF;
      uint32_t rank = 0;
#pragma unroll
      for (int u = 0; u < kPerPart; ++u) {
        const int j = part + 4 * u;
        const uint32_t kj = ckey[j];
        const int ij = cidx[j];
        rank += (j < (int)ncand) && ((kj > kc) || (kj == kc && ij < ic));
      }
      rank += dpp_u32<kDppXor1, 0xF, 0xF>(rank);
      rank += dpp_u32<kDppXor2, 0xF, 0xF>(rank);
      if (has && part == 0 && rank < need) atomicOr(&selbits[ic >> 5], 1u << (ic & 31));
    } else {
      // all key bits used and more equal keys than places: lowest indices win
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint64_t cb = __ballot((cand >> k) & 1);
        if (lane == 0) {
          candbits[k * 8 + 2 * wave] = (uint32_t)cb;
          candbits[k * 8 + 2 * wave + 1] = (uint32_t)(cb >> 32);
        }
      }
      __syncthreads();
      uint32_t mine = 0;
#pragma unroll
      for (int q = 0; q < WPT; ++q) {
        const int w = tid * WPT + q;
        if (w < NW) mine += __builtin_popcount(candbits[w]);
      }
      uint32_t total;
      uint32_t rank = block_exclusive_scan<kTopkWaves, false>(mine, scratch, &total);
#pragma unroll
      for (int q = 0; q < WPT; ++q) {
        const int w = tid * WPT + q;
        if (w >= NW) break;
        uint32_t bits = candbits[w];
        uint32_t keep = 0;
        while (bits != 0 && rank < need) {
          const uint32_t low = bits & (~bits + 1u);
          keep |= low;
          bits ^= low;
          ++rank;
        }
        if (keep) atomicOr(&selbits[w], keep);
      }
    }
    __syncthreads();
  }

  // ascending compaction of the bitmap
  uint32_t mine = 0;
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    const int w = tid * WPT + q;
    if (w < NW) mine += __builtin_popcount(selbits[w]);
  }
  uint32_t total;
  // (the selection's last use of `scratch`)
  uint32_t pos = block_exclusive_scan<kTopkWaves, false>(mine, scratch, &total);
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    const int w = tid * WPT + q;
    if (w >= NW) break;
    uint32_t bits = selbits[w];
    while (bits != 0) {
      const int bit = __builtin_ctz(bits);
      bits &= bits - 1;
      if (pos < (uint32_t)K) emit((int)pos, w * 32 + bit);
      ++pos;
    }
  }
  for (uint32_t i = total + tid; i < (uint32_t)K; i += kTopkThreads) emit((int)i, -1);
}

// The choice when n_pages <= K: every page, then -1 pads.
template <typename Emit>
__device__ __forceinline__ void choose_all(int n_pages, int K, Emit emit) {
  for (int i = (int)threadIdx.x; i < K; i += kTopkThreads) emit(i, i < n_pages ? i : -1);
}

}  // namespace da

#endif  // DA_TOPK_H
