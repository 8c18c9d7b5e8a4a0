// Quest page metadata, page scores and top-K page selection for gfx950.
//
// [Quest-review] "the page score is not an exact attention probability"
// (paper section 3.4, Algorithm 1):
//   metadata  m_{p,i} / M_{p,i} = per-channel min / max of the Keys in page p,
//             updated as each new Key arrives;
//   score     U(p, q) = sum_i max(q_i m_{p,i}, q_i M_{p,i}), summed here over
//             the G query heads that share the KV head;
//   select    the K pages with the largest U (ties to the lower page index),
//             reported in ascending page order.
//
// Kernels:
//   meta_append_kernel  one wave per (page touched, kv, b); lanes own channel
//                       pairs; exact fp16 min/max.
//   page_score_kernel   HBM-bound scan of the metadata: D/8 lanes per page, each
//                       lane one 16-byte chunk of the min row and of the max
//                       row.  Because M >= m, max(q m, q M) = q M when q >= 0
//                       and q m otherwise, so the G heads fold into two fp32
//                       weight vectors per channel (sum of the non-negative
//                       and of the negative q_gi) and a page costs 2 FMAs per
//                       channel instead of 2G.
//   topk_kernel         one workgroup per (b, kv): scores held in registers as
//                       order-preserving u32 keys; radix select on 11-bit
//                       digits below the common prefix of the min and max key,
//                       exact ranking of the last candidates in registers, an
//                       index-order scan for exact ties and the ascending
//                       compaction.  Integer-only decisions, so the chosen set
//                       is deterministic.  (Bit-serial passes without atomics
//                       measured slower: 7-8 barrier-bound passes cost more
//                       than 2-3 histogram passes.)
//   topk_stream_kernel  the same choice for units with more than 16,384 pages:
//                       1,024 threads, radix passes that re-read the score row
//                       instead of holding it, and output positions from a
//                       block scan over contiguous runs of pages.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"
#include "topk.h"

namespace da {
namespace {

// ------------------------------------------------------------ metadata

template <int D>
__global__ void __launch_bounds__(kWave) meta_append_kernel(MetaLaunch a) {
  const int lane = threadIdx.x;
  const int kv = blockIdx.y;
  const int b = blockIdx.z;
  const int hkv = a.num_kv_heads;
  const int64_t unit = (int64_t)b * hkv + kv;
  const int shift = a.page_shift;
  const int S = 1 << shift;

  int L = a.seqlens[b];
  L = L < 0 ? 0 : (L > a.capacity ? a.capacity : L);
  const int n = a.n_new < L ? a.n_new : L;
  if (n <= 0) return;
  const int t_lo = L - n;
  const int p = (t_lo >> shift) + blockIdx.x;
  if (p >= a.meta_max_pages || (p << shift) >= L) return;
  const int page_start = p << shift;
  const int lo = page_start > t_lo ? page_start : t_lo;
  const int hi = (page_start + S) < L ? (page_start + S) : L;
  const bool fresh = lo == page_start;
  if (lane >= D / 2) return;

  f16x2* mp = reinterpret_cast<f16x2*>(reinterpret_cast<f16*>(a.meta) +
                                       ((unit * a.meta_max_pages + p) * 2) * D);
  const f16 inf = (f16)__builtin_huge_valf();
  f16x2 mn = {inf, inf};
  f16x2 mx = {-inf, -inf};
  if (!fresh) {
    mn = mp[lane];
    mx = mp[D / 2 + lane];
  }
  const bool has_new = a.k_new != nullptr;
  for (int t = lo; t < hi; ++t) {
    int64_t off;
    if (a.page_table != nullptr) {
      const int phys = a.page_table[(int64_t)b * a.max_pages + (t >> shift)];
      if (phys < 0 || phys >= a.num_pages) continue;  // not a pool page: skip the key
      off = (((int64_t)phys * hkv + kv) << shift) * D + (int64_t)(t & (S - 1)) * D;
    } else {
      off = (unit * a.cache_stride + t) * D;
    }
    f16x2 key;
    if (has_new && t == L - 1) {
      key = reinterpret_cast<const f16x2*>(reinterpret_cast<const f16*>(a.k_new) + unit * D)[lane];
      const f16x2 val =
          reinterpret_cast<const f16x2*>(reinterpret_cast<const f16*>(a.v_new) + unit * D)[lane];
      reinterpret_cast<f16x2*>(reinterpret_cast<f16*>(a.k) + off)[lane] = key;
      reinterpret_cast<f16x2*>(reinterpret_cast<f16*>(a.v) + off)[lane] = val;
    } else {
      key = reinterpret_cast<const f16x2*>(reinterpret_cast<const f16*>(a.k) + off)[lane];
    }
    mn = __builtin_elementwise_min(mn, key);
    mx = __builtin_elementwise_max(mx, key);
  }
  mp[lane] = mn;
  mp[D / 2 + lane] = mx;
}

// ------------------------------------------------------------ page score

constexpr int kScoreWaves = 4;
// Page slots per lane per pass (loads in flight): 8, or 4 for a scan that
// would give fewer than about 1,024 workgroups at 8, so that it spreads over
// twice as many (measured at 32K pages x 32 heads: 10.2 us instead of 10.8).
constexpr int kScoreDepth = 8;
constexpr int kScoreDepthShallow = 4;
constexpr int kScoreTargetWorkgroups = 1024;

template <int D, int DEPTH>
struct ScoreShape {
  static constexpr int LPP = D / 8;                 // lanes per page (16-byte chunks)
  static constexpr int PPI = kWave / LPP;           // pages per wave per slot
  static constexpr int PAGES_PER_PASS = kScoreWaves * PPI * DEPTH;
};

// One workgroup scores `score_passes` passes of PAGES_PER_PASS consecutive
// pages of one (b, kv) unit.  Lane (page slot, chunk) loads 16 bytes of the
// page's min row and 16 of its max row (non-temporal: read once), weighs
// them with the group's per-channel sums of non-negative / negative queries,
// and the D/8 lanes of a page add up their partial sums (DPP).
template <int D, int G, int DEPTH>
// The leading scalar arguments repeat the fields of `a` that the first
// instructions need (see `launch_score_topk`); the rest of `a` is read from
// the kernel-argument segment while the valid-length load is in flight.
__global__ void __launch_bounds__(kWave * kScoreWaves)
    page_score_kernel(const int32_t* __restrict__ seqlens, const void* __restrict__ q,
                      void* meta, const void* __restrict__ k_new, int hkv, ScoreLaunch a) {
  using SS = ScoreShape<D, DEPTH>;
  constexpr int LPP = SS::LPP;
  constexpr int PPI = SS::PPI;
  const int lane = lane_in_wave();
  const int wave = threadIdx.x / kWave;
  const int slot = lane / LPP;  // page within a wave step
  const int ch = lane % LPP;    // 16-byte chunk of the D channels
  const int kv = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t unit = (int64_t)b * hkv + kv;
  const int shift = a.page_shift;

  int L = seqlens[b];
  L = L < 0 ? 0 : L;
  int n_pages = (L + (1 << shift) - 1) >> shift;
  if (n_pages > a.meta_max_pages) n_pages = a.meta_max_pages;
  const int wg_begin = blockIdx.x * SS::PAGES_PER_PASS * a.score_passes;
  if (wg_begin >= n_pages) return;

  // Metadata of one pass: DEPTH pages per lane slot; slots past the valid
  // pages read page p0 (which exists) and store no score.  The first pass is
  // requested here, before the query and append loads, so that all of them
  // are in flight together; each later pass is requested after the previous
  // one is scored.
  f16* mbase = reinterpret_cast<f16*>(meta) + unit * a.meta_max_pages * 2 * D;
  f16x8 mins[DEPTH], maxs[DEPTH];
  int pg[DEPTH];
  auto load_pass = [&](int p0) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int p = p0 + (u * kScoreWaves + wave) * PPI + slot;
      pg[u] = p;
      const int64_t pp = p < n_pages ? p : p0;
      mins[u] = stream_load(mbase + pp * 2 * D + 8 * ch);
      maxs[u] = stream_load(mbase + pp * 2 * D + D + 8 * ch);
    }
  };
  load_pass(wg_begin);

  // Per-channel weights: sum of the group's non-negative q_gi (pairs with the
  // max) and of its negative q_gi (pairs with the min).
  float wpos[8], wneg[8];
  const f16* qb = reinterpret_cast<const f16*>(q) + unit * G * D + 8 * ch;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    wpos[e] = 0.0f;
    wneg[e] = 0.0f;
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const f16x8 qv = *reinterpret_cast<const f16x8*>(qb + g * D);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (float)qv[e];
      if (x >= 0.0f) wpos[e] += x; else wneg[e] += x;
    }
  }

  // Fused append: the page holding the step's new key, its new min/max chunk.
  int p_app = -1;  // no lane matches when there is no append
  bool fresh = false;
  f16x8 knew = {};
  int t_app = 0;
  if (k_new != nullptr) {
    int La = seqlens[b];
    La = La < 0 ? 0 : (La > a.capacity ? a.capacity : La);
    if (La >= 1) {
      t_app = La - 1;
      p_app = t_app >> shift;
      fresh = (t_app & ((1 << shift) - 1)) == 0;
      knew = *reinterpret_cast<const f16x8*>(reinterpret_cast<const f16*>(k_new) + unit * D + 8 * ch);
    }
  }

  float* scores = a.scores + unit * a.meta_max_pages;
  for (int pass = 0, p0 = wg_begin;;) {
    // the appended key enters its page's min/max before the page is scored
    // (selects, no branch: the wait counts of the loads stay exact)
    int app_u = -1;
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const bool hit = pg[u] == p_app;
      app_u = hit ? u : app_u;
      const f16x8 mn = fresh ? knew : __builtin_elementwise_min(mins[u], knew);
      const f16x8 mx = fresh ? knew : __builtin_elementwise_max(maxs[u], knew);
      mins[u] = hit ? mn : mins[u];
      maxs[u] = hit ? mx : maxs[u];
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s = fmaf(wpos[e], (float)maxs[u][e], s);
        s = fmaf(wneg[e], (float)mins[u][e], s);
      }
      s = group_sum<LPP>(s);
      if (ch == 0 && pg[u] < n_pages) scores[pg[u]] = s;
    }
    if (app_u >= 0) {  // the D/8 lanes of the appended page write its row back
      f16x8 mn = mins[0], mx = maxs[0];
#pragma unroll
      for (int u = 1; u < DEPTH; ++u) {
        mn = app_u == u ? mins[u] : mn;
        mx = app_u == u ? maxs[u] : mx;
      }
      f16* mrow = mbase + (int64_t)p_app * 2 * D + 8 * ch;
      *reinterpret_cast<f16x8*>(mrow) = mn;
      *reinterpret_cast<f16x8*>(mrow + D) = mx;
      int64_t off = -1;
      if (a.page_table != nullptr) {
        const int phys = p_app < a.max_pages ? a.page_table[(int64_t)b * a.max_pages + p_app] : -1;
        if (phys >= 0 && phys < a.num_pages)
          off = (((int64_t)phys * hkv + kv) << shift) * D +
                (int64_t)(t_app & ((1 << shift) - 1)) * D;
      } else {
        off = (unit * a.cache_stride + t_app) * D;
      }
      if (off >= 0) {  // v_new is read only here, off the scoring path
        const f16x8 vnew =
            *reinterpret_cast<const f16x8*>(reinterpret_cast<const f16*>(a.v_new) + unit * D + 8 * ch);
        *reinterpret_cast<f16x8*>(reinterpret_cast<f16*>(a.k) + off + 8 * ch) = knew;
        *reinterpret_cast<f16x8*>(reinterpret_cast<f16*>(a.v) + off + 8 * ch) = vnew;
      }
    }
    ++pass;
    p0 += SS::PAGES_PER_PASS;
    if (pass >= a.score_passes || p0 >= n_pages) break;
    load_pass(p0);
  }
}

// ------------------------------------------------------------ top-K

// One workgroup per (b, kv): select_top_k over the unit's score row.
// Leading scalar arguments as in the score kernel: the score row and its
// width, so the score loads issue together with the valid-length load.
template <int R>
__global__ void __launch_bounds__(kTopkThreads)
    topk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ seqlens, int hkv,
                int row_pages, ScoreLaunch a) {
  const int tid = threadIdx.x;
  const int kv = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t unit = (int64_t)b * hkv + kv;
  const float* sc = scores + unit * row_pages;
  // The length and all score loads first, unconditionally, the scores at
  // indices clamped to the row (not to the valid pages, which wait for the
  // length), so they are in flight together; entries past the valid pages are
  // masked in the selection.  Early loads are not moved past the exit below.
  int L = early_load(seqlens + b);
  float raw[R];
#pragma unroll
  for (int k = 0; k < R; ++k) raw[k] = early_load(sc + min(k * kTopkThreads + tid, row_pages - 1));

  const int K = a.num_sel;
  int32_t* dst = a.page_idx + unit * K;
  L = L < 0 ? 0 : L;
  int n_pages = (L + (1 << a.page_shift) - 1) >> a.page_shift;
  if (n_pages > row_pages) n_pages = row_pages;
  auto emit = [&](int pos, int page) { dst[pos] = page; };
  if (n_pages <= K) {
    choose_all(n_pages, K, emit);
    return;
  }
  select_top_k<R>(raw, n_pages, K, emit);
}

// ------------------------------------------------------------ streaming top-K

constexpr int kStreamTopkThreads = 1024;
constexpr int kStreamTopkWaves = kStreamTopkThreads / kWave;
constexpr int kStreamUnroll = 8;  // score loads in flight per thread

// key >> shift for shift in [0, 32]
__device__ __forceinline__ uint32_t key_prefix(uint32_t key, int shift) {
  return shift >= 32 ? 0u : key >> shift;
}

// One workgroup per (b, kv) for units with more pages than the register-held
// select takes (256 threads x 64).  The same choice -- the K largest keys,
// ties to the lower page, ascending pages -- from passes that re-read the
// unit's score row (an L2-resident 4 bytes per page) instead of holding it:
//   1. the smallest and largest key give the prefix every key shares;
//   2. radix passes of up to 11-bit digits below the resolved prefix: an LDS
//      histogram of the keys that still carry the prefix and a
//      digit-descending block scan for the boundary digit, which extends the
//      prefix; `need` counts the places left for keys that carry it;
//   3. keys above the final prefix are chosen, and of the keys equal to it the
//      `need` lowest pages (all of them when need covers them);
//   4. thread t owns a contiguous run of pages; a block scan of the chosen
//      counts of the runs gives each run its first output position.
__global__ void __launch_bounds__(kStreamTopkThreads)
    topk_stream_kernel(const float* __restrict__ scores, const int32_t* __restrict__ seqlens,
                       int hkv, int row_pages, ScoreLaunch a) {
  __shared__ uint32_t hist[1 << kRadixBits];
  __shared__ uint32_t red_min[kStreamTopkWaves], red_max[kStreamTopkWaves];
  __shared__ uint32_t scratch[kStreamTopkWaves];
  __shared__ uint32_t info[3];
  const int tid = threadIdx.x;
  const int lane = lane_in_wave();
  const int wave = tid / kWave;
  const int kv = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t unit = (int64_t)b * hkv + kv;
  const float* sc = scores + unit * row_pages;
  int L = seqlens[b];
  L = L < 0 ? 0 : L;
  const int64_t pages_l = ((int64_t)L + (1 << a.page_shift) - 1) >> a.page_shift;
  const int n_pages = pages_l < row_pages ? (int)pages_l : row_pages;
  const int K = a.num_sel;
  int32_t* dst = a.page_idx + unit * K;
  if (n_pages <= K) {
    for (int i = tid; i < K; i += kStreamTopkThreads) dst[i] = i < n_pages ? i : -1;
    return;
  }

  // 1. key range
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int i0 = 0; i0 < n_pages; i0 += kStreamTopkThreads * kStreamUnroll) {
    float x[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int i = i0 + u * kStreamTopkThreads + tid;
      x[u] = sc[i < n_pages ? i : n_pages - 1];
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const uint32_t k = order_key(x[u]);
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    }
  }
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  if (lane == 0) {
    red_min[wave] = kmin;
    red_max[wave] = kmax;
  }
  for (int i = tid; i < (1 << kRadixBits); i += kStreamTopkThreads) hist[i] = 0u;
  __syncthreads();
  kmin = red_min[0];
  kmax = red_max[0];
#pragma unroll
  for (int w = 1; w < kStreamTopkWaves; ++w) {
    kmin = min(kmin, red_min[w]);
    kmax = max(kmax, red_max[w]);
  }
  const uint32_t diff = kmin ^ kmax;
  int shift = diff ? 32 - __builtin_clz(diff) : 0;  // bits below the shared prefix
  uint32_t pre = key_prefix(kmax, shift);
  uint32_t need = (uint32_t)K;
  uint32_t ncand = (uint32_t)n_pages;

  // 2. radix passes over the keys that carry the prefix
  while (need > 0 && need < ncand && shift > 0) {
    const int nb = shift < kRadixBits ? shift : kRadixBits;
    const int lo = shift - nb;
    const uint32_t dmask = (1u << nb) - 1u;
    for (int i0 = 0; i0 < n_pages; i0 += kStreamTopkThreads * kStreamUnroll) {
      float x[kStreamUnroll];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const int i = i0 + u * kStreamTopkThreads + tid;
        x[u] = sc[i < n_pages ? i : n_pages - 1];
      }
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const uint32_t k = order_key(x[u]);
        const bool in = i0 + u * kStreamTopkThreads + tid < n_pages && key_prefix(k, shift) == pre;
        if (in) atomicAdd(&hist[(k >> lo) & dmask], 1u);
      }
    }
    __syncthreads();
    // thread t reads `per` digits from the top digit down
    constexpr int kPerMax = ((1 << kRadixBits) + kStreamTopkThreads - 1) / kStreamTopkThreads;
    const int nbins = 1 << nb;
    const int per = (nbins + kStreamTopkThreads - 1) / kStreamTopkThreads;
    uint32_t cnt[kPerMax];
    uint32_t run = 0;
#pragma unroll
    for (int q = 0; q < kPerMax; ++q) {
      const int dgt = nbins - 1 - (tid * per + q);
      cnt[q] = (q < per && dgt >= 0) ? hist[dgt] : 0u;
      run += cnt[q];
    }
    uint32_t total;
    const uint32_t before = block_exclusive_scan<kStreamTopkWaves>(run, scratch, &total);
    if (before < need && need <= before + run) {
      uint32_t acc = before;
      bool found = false;
#pragma unroll
      for (int q = 0; q < kPerMax; ++q) {
        if (!found && acc + cnt[q] >= need) {
          info[0] = (uint32_t)(nbins - 1 - (tid * per + q));  // boundary digit
          info[1] = acc;                                      // keys above it
          info[2] = cnt[q];                                   // keys on it
          found = true;
        }
        acc += cnt[q];
      }
    }
    __syncthreads();
    need -= info[1];
    ncand = info[2];
    pre = (pre << nb) | info[0];
    shift = lo;
    for (int i = tid; i < nbins; i += kStreamTopkThreads) hist[i] = 0u;
    __syncthreads();  // hist and info are reused by the next pass
  }

  // 3-4. chosen pages in page order, thread t owning pages [r0, r1)
  const int per_t = (n_pages + kStreamTopkThreads - 1) / kStreamTopkThreads;
  const int r0 = min(tid * per_t, n_pages);
  const int r1 = min(r0 + per_t, n_pages);
  uint32_t n_above = 0, n_tie = 0;
  for (int i0 = r0; i0 < r1; i0 += kStreamUnroll) {
    float x[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) x[u] = sc[min(i0 + u, r1 - 1)];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const uint32_t kp = key_prefix(order_key(x[u]), shift);
      const bool in = i0 + u < r1;
      n_above += (in && kp > pre) ? 1u : 0u;
      n_tie += (in && kp == pre) ? 1u : 0u;
    }
  }
  uint32_t tot_above, tot_tie;
  uint32_t above_before = block_exclusive_scan<kStreamTopkWaves>(n_above, scratch, &tot_above);
  uint32_t tie_before = block_exclusive_scan<kStreamTopkWaves>(n_tie, scratch, &tot_tie);
  for (int i0 = r0; i0 < r1; i0 += kStreamUnroll) {
    float x[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) x[u] = sc[min(i0 + u, r1 - 1)];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int i = i0 + u;
      const uint32_t kp = key_prefix(order_key(x[u]), shift);
      if (i < r1 && kp > pre) {
        // chosen pages below i: the keys above the prefix, and the tied
        // pages that fit
        dst[above_before + min(tie_before, need)] = i;
        ++above_before;
      } else if (i < r1 && kp == pre) {
        if (tie_before < need) dst[above_before + tie_before] = i;
        ++tie_before;
      }
    }
  }
}

template <int D, int G, int DEPTH>
int launch_score(const ScoreLaunch& in, hipStream_t s) {
  // passes per workgroup: enough workgroups to fill the chip (about 1,024),
  // each streaming as many pages as that allows (at most 8 passes)
  ScoreLaunch a = in;
  constexpr int per_pass = ScoreShape<D, DEPTH>::PAGES_PER_PASS;
  const int64_t total = (int64_t)a.batch * a.num_kv_heads * a.meta_max_pages;
  const int64_t passes = total / ((int64_t)kScoreTargetWorkgroups * per_pass);
  a.score_passes = (int)(passes < 1 ? 1 : (passes > 8 ? 8 : passes));
  const int per_wg = per_pass * a.score_passes;
  dim3 grid((a.meta_max_pages + per_wg - 1) / per_wg, a.num_kv_heads, a.batch);
  hipLaunchKernelGGL((page_score_kernel<D, G, DEPTH>), grid, dim3(kWave * kScoreWaves), 0, s,
                     a.seqlens, a.q, a.meta, a.k_new, a.num_kv_heads, a);
  return (int)hipGetLastError();
}

template <int D, int G>
int launch_score_dg(const ScoreLaunch& a, hipStream_t s) {
  const int64_t total = (int64_t)a.batch * a.num_kv_heads * a.meta_max_pages;
  const bool shallow =
      total < (int64_t)kScoreTargetWorkgroups * ScoreShape<D, kScoreDepth>::PAGES_PER_PASS;
  return shallow ? launch_score<D, G, kScoreDepthShallow>(a, s)
                 : launch_score<D, G, kScoreDepth>(a, s);
}

template <int D>
int launch_score_d(const ScoreLaunch& a, hipStream_t s) {
  switch (a.group) {
    case 1: return launch_score_dg<D, 1>(a, s);
    case 2: return launch_score_dg<D, 2>(a, s);
    case 4: return launch_score_dg<D, 4>(a, s);
    case 8: return launch_score_dg<D, 8>(a, s);
    default: return (int)hipErrorInvalidValue;
  }
}

template <int R>
int launch_topk(const ScoreLaunch& a, hipStream_t s) {
  dim3 grid(a.num_kv_heads, a.batch);
  hipLaunchKernelGGL((topk_kernel<R>), grid, dim3(kTopkThreads), 0, s, a.scores, a.seqlens,
                     a.num_kv_heads, a.meta_max_pages, a);
  return (int)hipGetLastError();
}

}  // namespace

int launch_meta_append(const MetaLaunch& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid(a.pages_per_seq, a.num_kv_heads, a.batch);
  if (a.head_dim == 64) {
    hipLaunchKernelGGL((meta_append_kernel<64>), grid, dim3(kWave), 0, s, a);
  } else if (a.head_dim == 128) {
    hipLaunchKernelGGL((meta_append_kernel<128>), grid, dim3(kWave), 0, s, a);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_topk_only(const ScoreLaunch& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int P = a.meta_max_pages;
  if (P <= kTopkThreads * 8) return launch_topk<8>(a, s);
  if (P <= kTopkThreads * 16) return launch_topk<16>(a, s);
  if (P <= kTopkThreads * 32) return launch_topk<32>(a, s);
  if (P <= kTopkThreads * 64) return launch_topk<64>(a, s);
  dim3 grid(a.num_kv_heads, a.batch);
  hipLaunchKernelGGL(topk_stream_kernel, grid, dim3(kStreamTopkThreads), 0, s, a.scores,
                     a.seqlens, a.num_kv_heads, a.meta_max_pages, a);
  return (int)hipGetLastError();
}

int launch_score_topk(const ScoreLaunch& in, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const ScoreLaunch& a = in;
  int err = a.head_dim == 64 ? launch_score_d<64>(a, s)
          : a.head_dim == 128 ? launch_score_d<128>(a, s)
                              : (int)hipErrorInvalidValue;
  if (err != 0 || a.page_idx == nullptr) return err;  // scores only
  return launch_topk_only(a, stream);
}

int topk_max_pages() { return kTopkThreads * 64; }

}  // namespace da
