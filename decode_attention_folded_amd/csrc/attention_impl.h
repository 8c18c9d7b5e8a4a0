// Split-context folded-GQA decode attention for gfx950 (MI355X): the kernel
// templates and their launch, included by the translation units that
// instantiate them (decode_kernel.hip: given page lists or none;
// decode_select.hip: pages selected in the kernel).
//
// What it computes -- [CoreML-GQA] section 3, "Fold Q Instead of Expanding KV"
// and "Implementation": for every (batch b, KV head kv) the G query heads
// h = G*kv + g are treated as G rows of one small matrix, so each K and V row
// is read from HBM once for all G rows (no repeat_kv copy).  Per row:
// s_t = scale * q.k_t for t < L_b, softmax over t, o = sum_t p_t v_t.
// With q_len > 1 query positions per head ([CoreML-GQA] section 5, "Prefill
// Needs Separate Design") the rows are the G * q_len (head, position) pairs of
// the KV head -- group and sequence axes merged -- and row g * q_len + i only
// sees keys t < L_b - q_len + 1 + i.  The template parameter G is the row
// count.  The Quest variant ([Quest-review], paper sections 3.3-3.5) runs the
// same loop over the tokens of the chosen pages only.
//
// Work decomposition (flash-decode): a 1-D grid of splits x (B * Hkv) units,
// unit index fastest.  A workgroup of 4 waves owns a contiguous chunk of
// `tiles_per_split` 16-key tiles of one (b, kv) unit; its waves take the
// chunk's tiles round robin.  (The paged dense stream instead takes its
// chunks from a flat list of real chunks, longest sequences first: one
// workgroup per chunk, or, for up to 64 sequences with rows x D >= 512,
// resident workgroups that take chunk after chunk from a work counter; see
// flat_chunk and Persist.)  Workgroups reach the 8 XCDs round robin, so with
// the unit index fastest every XCD receives the same KV heads of every
// sequence: sequences of different lengths load the XCDs evenly, which they
// do not when the split index runs fastest (short sequences would only feed
// the XCDs of the low split numbers).
// Each split writes a partial (running max m, sum l, unnormalised o) and a
// second, small launch merges them (log-sum-exp, in split order).  The kernel
// boundary is the only synchronisation: merging inside the attention kernel
// needs either device-scope release/acquire fences (which write back /
// invalidate the whole L2 of every XCD and cost a third of the runtime) or a
// hand-off through agent-scope (write-through) stores, an arrival counter and
// agent-scope loads, which measured no faster than the extra launch on small
// grids and about 5% slower on large ones (every workgroup must wait for its
// write-through stores before it retires).
//
// Lane layout of one 16-key tile (lane = 0..63):
//   K: lane holds key (lane % 16), 16-byte channel chunks 4*j + lane/16,
//      j < D/32 -- the B-operand layout of v_mfma_f32_16x16x16f16 (k =
//      channel, n = key), so a tile feeds the matrix core as loaded.
//   V: lane holds keys (lane % 8) and (lane % 8) + 8, chunks 8*h + lane/8,
//      h < D/64: each load instruction covers 128 contiguous bytes of each
//      of 8 keys, and a lane accumulates only D/8 channels per query row.
// Scores: the G query rows are replicated over the 16 rows of the MFMA A
// operand, so every lane receives all G scores of its K key.  One DPP
// exchange (lane ^ 8) hands each lane the scores of its two V keys.
// Each lane keeps its own online-softmax state (m, l, fp32 accumulators) over
// the keys that pass through its slots; the 8 slot states of a channel group
// are merged at the end of the chunk, then the 4 waves through LDS.
// Rescaling is lazy: the running max only moves when a score exceeds it by
// more than 2^8 (exp2 units), so steady-state tiles skip the rescale.
// Tiles are loaded into a ring of NS register stages, so NS - 1 tiles are in
// flight while one is computed.
//
// Keys at or past the valid length are never loaded from their own slots:
// their loads are redirected to a valid row of the same sequence and their
// scores forced to -inf, so whatever the cache holds there (even NaN) cannot
// leak into the result.  No floating-point atomics: results are bitwise
// reproducible.

#ifndef DA_ATTENTION_IMPL_H
#define DA_ATTENTION_IMPL_H

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"
#include "topk.h"

namespace da {
namespace {

typedef f16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kTileKeys = 16;
// Key tiles per workgroup chunk, at most: 160 when the chunk reads a page
// list (paged cache or chosen pages; the list is staged in LDS), 512 for a
// contiguous cache.  Measured on MI355X: contiguous 128K dense attention
// 672 us at 128, 642 at 256, 634 at 512, 636 at 1024 (fewer workgroup
// start-ups and partials); the variable-length paged batch in its persistent
// launch 701, 686.5, 678.6, 679.5, 693.8 and 688 us at 96, 128, 160, 192, 224
// and 256 (longer chunks mean fewer chunk changes, but a coarser tail of
// unequal sequences).
constexpr int kMaxTilesPerSplit = 160;
constexpr int kMaxTilesPerSplitContiguous = 512;
constexpr int kMinPageSize = 8;
// pages (or chosen-page entries) one chunk can touch
constexpr int kMaxChunkPages = kMaxTilesPerSplit * kTileKeys / kMinPageSize + 2;
constexpr float kRescaleThreshold = 8.0f;
constexpr float kNegBig = -1.0e30f;
constexpr int kStages = 3;

// Keys in the (b, kv) key stream and the number of splits that cover it;
// shared by the attention and the merge kernel.
struct StreamInfo {
  int L;        // valid length after clamping
  int n_keys;   // keys in the stream (dense: L; chosen pages: nsel * S)
  int nsplit;   // splits with at least one key
};

__device__ __forceinline__ StreamInfo stream_info(const AttnLaunch& a, const int32_t* seqlens, int b,
                                                  bool sparse) {
  StreamInfo si;
  const int L = seqlens[b];
  si.L = L < 0 ? 0 : (L > a.capacity ? a.capacity : L);
  si.n_keys = si.L;
  if (sparse) {
    const int pages = (si.L + (1 << a.page_shift) - 1) >> a.page_shift;
    const int nsel = pages < a.num_sel ? pages : a.num_sel;
    si.n_keys = nsel << a.page_shift;
  }
  const int n_tiles = (si.n_keys + kTileKeys - 1) / kTileKeys;
  si.nsplit = (n_tiles + a.tiles_per_split - 1) / a.tiles_per_split;
  return si;
}

template <int D>
struct Layout {
  static constexpr int NCK = D / 32;   // K chunks per lane per tile
  static constexpr int NCV = D / 64;   // V chunks per lane per key (2 keys)
  static constexpr int NV = NCV * 8;   // channels per lane
};

template <int D>
struct Stage {
  f16x8 k[Layout<D>::NCK];
  f16x8 v0[Layout<D>::NCV];  // key (lane % 8)
  f16x8 v1[Layout<D>::NCV];  // key (lane % 8) + 8
  bool kvalid;               // the K key of this lane
  int ktok;                  // its token position (causal limit of q_len > 1 rows)
};

// Merge the split partials of one unit into its G output rows:
// O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s over the splits, in split
// order (log-sum-exp).  One thread per output element; D is a multiple of 64,
// so every wave works on one row.  Lane s of a wave loads split s's (m, l) of
// that row and the values reach the other lanes through readlane, so a round
// of KB splits is 1 + KB loads per lane: within the 63 loads a wave can keep
// in flight, so the round costs one memory round trip.  The launch picks KB
// (8, 16 or 48) to cover the plan's splits with as few loads as possible.  The first
// round is read before `get_nsplit` is called (it may wait for the valid
// length).  Splits past the valid ones get zero weight, so stale workspace
// contents never enter the sums.
template <int D, int G, int NT, int KB, typename NSplitFn>
__device__ __forceinline__ void merge_partials(const AttnLaunch& a, const float* part_ml,
                                               const float* part_o, int max_splits, int64_t unit,
                                               NSplitFn get_nsplit) {
  static_assert(NT == G * D && D % kWave == 0, "one thread per output element, one row per wave");
  constexpr int kBatch = KB;  // splits per round of loads (at most 48)
  static_assert(KB >= 1 && KB <= 48, "splits per round");
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + unit * max_splits * G;
  const float* po = part_o + unit * max_splits * G * D;
  f16* out = reinterpret_cast<f16*>(a.out) + unit * G * D;
  const int i = (int)threadIdx.x;  // output element
  const int g = i / D;             // its row, the same for the whole wave
  const int lane = lane_in_wave();

  float M = kNegBig, O = 0.0f, S = 0.0f;
  float2 mlv;          // (m, l) of split s0 + lane
  float ov[kBatch];    // o of splits s0 .. s0 + kBatch - 1 at element i
  auto load_round = [&](int s0, auto load) {
    mlv = load(ml + min(s0 + lane, max_splits - 1) * G + g);
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      ov[u] = load(po + (int64_t)min(s0 + u, max_splits - 1) * G * D + i);
  };
  auto add_round = [&](int s0, int nsplit) {
    const bool mine = lane < kBatch && s0 + lane < nsplit;
    const float m_s = mine ? mlv.x : kNegBig;
    const float bm = fmaxf(M, wave_max_f32(m_s));
    const float w_s = mine ? fast_exp2(m_s - bm) : 0.0f;
    const float l_s = mine ? mlv.y : 0.0f;
    const float f = fast_exp2(M - bm);
    float o = O * f, l = S * f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = read_lane(w_s, u);
      o = fmaf(w, s0 + u < nsplit ? ov[u] : 0.0f, o);
      l = fmaf(w, read_lane(l_s, u), l);
    }
    M = bm;
    O = o;
    S = l;
  };
  // The first round is issued before anything else (its addresses need only
  // the leading arguments, and early loads are not moved past the exit
  // below); later rounds follow one by one.
  load_round(0, [](const auto* p) { return early_load(p); });
  const int nsplit = get_nsplit();
  if (nsplit <= 1) return;  // the attention kernel wrote the output
  add_round(0, nsplit);
  for (int s0 = kBatch; s0 < nsplit; s0 += kBatch) {
    load_round(s0, [](const auto* p) { return *p; });
    add_round(s0, nsplit);
  }
  out[i] = (f16)(S > 0.0f ? O / S : 0.0f);
}

// Persistent paged dense stream (batches of at most 64 sequences).  A launch
// of about as many workgroups as fit on the chip at once works through the
// flat work list (see flat_chunk: real chunks only, longest sequences first,
// the Hkv heads of a chunk on consecutive tickets).  Ticket t is the t-th
// (chunk, head) item; workgroup w starts with ticket w and takes the next one
// from a counter in the workspace while its current chunk still streams, then
// loads that chunk's page-table entries, so a new chunk starts with its page
// list already in LDS instead of three dependent memory round trips (valid
// lengths, page table, K/V) behind the saturated HBM stream.  The hardware
// dispatcher no longer balances the unequal sequences; the ticket order does.
//
// The counter starts at zero: a one-thread launch clears it just before (the
// workspace itself needs no initialisation).  A fetched value v names ticket
// grid + v when v < T - grid, T being the number of tickets; any other value
// ends the workgroup.  Values come in increasing order, so every valid one is
// handed out before the first that ends a workgroup, and every ticket is
// processed exactly once.  (From an arbitrary starting value that fails: the
// values that end workgroups can come first and stop them all before the low
// values are handed out.)
struct Persist {
  uint32_t* counter;          // the ticket counter (zero at the launch)
  uint32_t* next_slot;        // LDS [2]: the ticket after each buffer's chunk
  int32_t* phys0_slot;        // LDS [2]: page of token 0 of each list buffer's sequence
  const int32_t* flat_L;      // LDS [64]: clamped valid length of sequence b
  const int32_t* flat_start;  // LDS [64]: its first flat chunk
  const int32_t* flat_n;      // LDS [64]: its number of chunks
  uint32_t grid;              // workgroups in the launch (= static tickets)
  uint32_t total;             // T: flat chunks x Hkv
  int batch;
  int buf;                    // LDS list buffer of the current chunk
  bool staged;                // the current chunk's list is already in that buffer
};

// Ticket t -> (split, unit) of the flat work list; wave-uniform.
__device__ __forceinline__ void persist_lookup(const Persist& ps, int hkv, uint32_t t,
                                               uint32_t& split_u, uint32_t& unit_u) {
  const int lane = lane_in_wave();
  const uint32_t f = t / (uint32_t)hkv;
  const uint32_t kv = t - f * (uint32_t)hkv;
  const int st = ps.flat_start[lane];
  const int n = ps.flat_n[lane];
  const uint64_t hit = __ballot(lane < ps.batch && (uint32_t)st <= f && f < (uint32_t)(st + n));
  const int b = hit ? __builtin_ctzll(hit) : 0;
  split_u = f - (uint32_t)__builtin_amdgcn_readlane(st, b);
  unit_u = (uint32_t)b * (uint32_t)hkv + kv;
}

// The leading scalar arguments repeat the fields of `a` that the first
// instructions need (see `launch_one`); the rest of `a` is read from the
// kernel-argument segment while the valid-length load is in flight.  `list`
// is the first list the chunk reads (the chosen pages, the page scores when
// the kernel selects the pages itself, else the page table, else unused) and
// `list_width` its row width; `chunk_geom` packs the key tiles per chunk
// (bits 0-15) and log2 of the page size (bits 16 and up), which place the
// chunk's list entries.
//
// SEL_R > 0 (selected-page stream only): every workgroup of a unit runs the
// top-K over the unit's page scores itself (select_top_k, SEL_R scores per
// thread) and keeps the part of the ascending choice that its chunk covers;
// the first split also writes the choice out.  All workgroups of a unit make
// the same integer decisions on the same scores, so this equals a separate
// top-K launch followed by the selected-page attention, with one launch less.
//
// DRAIN (contiguous cache, chunks of at most two ring rounds per wave): the
// ring's last round issues no loads past the chunk.  The arithmetic is the
// same as without it, so both variants give bitwise equal results.
//
// PERSIST (paged dense stream in the persistent launch, `ps` given): the
// valid length comes from the flat list in LDS, the chunk's page list may
// already be staged (ps->staged), and wave 0 takes the workgroup's next ticket
// and prepares its page list (see Persist).
//
// attend_chunk runs chunk `split_u` of unit `unit_u` (unit = b * Hkv + kv)
// with the calling workgroup: it writes the unit's output when the unit has
// one split with keys, a partial when it has more and split_u is below that
// count, and nothing otherwise (split 0 of a unit without keys writes the
// zero output).
template <int D, int G, bool PAGED, bool SPARSE, int SEL_R, bool DRAIN, bool PERSIST = false>
__device__ __forceinline__ void attend_chunk(const int32_t* __restrict__ seqlens,
                                             const void* __restrict__ q, void* k, void* v,
                                             const void* __restrict__ list, int batch, int hkv,
                                             int list_width, int chunk_geom, const AttnLaunch& a,
                                             uint32_t split_u, uint32_t unit_u,
                                             Persist* ps = nullptr) {
  constexpr bool SELECT = SEL_R > 0;
  static_assert(!PERSIST || (PAGED && !SPARSE), "the persistent launch runs the paged dense stream");
  // The thread index, hidden from the optimiser in the persistent launch: the
  // values derived from it are then recomputed per chunk instead of being held
  // across the chunk loop (which took the kernel past 256 registers, half the
  // occupancy).
  int tid_ = (int)threadIdx.x;
  if constexpr (PERSIST) asm volatile("" : "+v"(tid_));
  static_assert(!SELECT || SPARSE, "page selection feeds the selected-page stream");
  static_assert(!DRAIN || !PAGED, "the draining ring is built for contiguous caches");
  static_assert(!SELECT || kThreads == kTopkThreads, "one workgroup shape for both parts");
  constexpr int NCK = Layout<D>::NCK;
  constexpr int NCV = Layout<D>::NCV;
  constexpr int NV = Layout<D>::NV;
  constexpr int GC = (G + 3) / 4;  // MFMA chains (4 query rows each)
  constexpr int NS = kStages;

  __shared__ float s_o[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  // chunk page lists (two in the persistent launch: the current chunk's and
  // the next one's)
  __shared__ int32_t s_page_mem[(PERSIST ? 2 : 1) * ((PAGED || SPARSE) ? kMaxChunkPages : 1)];
  int32_t* s_page = s_page_mem;
  if constexpr (PERSIST) s_page = s_page_mem + ps->buf * kMaxChunkPages;
  const bool stage_list = !PERSIST || !ps->staged;
  __shared__ int32_t s_phys[(PAGED && SPARSE) ? kMaxChunkPages : 1];

  const int lane = (tid_ & (kWave - 1));
  const int wave = tid_ / kWave;
  const int rk = lane & 15;        // K key slot
  const int ck = lane >> 4;        // K chunk group (0..3)
  const int rv = lane & 7;         // V key slots rv, rv + 8
  const int cv = lane >> 3;        // V chunk group (0..7)
  const bool upper = (lane & 8) != 0;
  const uint32_t b_u = unit_u / (uint32_t)hkv;
  const int split = (int)split_u;
  const int64_t unit = unit_u;
  const int b = (int)b_u;
  const int kv = (int)(unit_u - b_u * (uint32_t)hkv);
  const int tiles_per_split = chunk_geom & 0xFFFF;
  const int shift = chunk_geom >> 16;
  const int page_mask = (1 << shift) - 1;
  const int tile_begin = split * tiles_per_split;
  const int key_begin = tile_begin * kTileKeys;
  const int page0 = key_begin >> shift;

  // Inputs that do not depend on the valid length: the folded queries and the
  // raw page-list entries of the whole chunk (clamped indices; checked once
  // the length is known).
  const f16* qb = reinterpret_cast<const f16*>(q) + unit * G * D;
  // MFMA A operand: row i of chain c is query g = (4c + i % 4) mod G; the lane
  // holds row lane % 16 over the k-slots of chunk 4j + ck.
  f16x8 qa[GC][NCK];
#pragma unroll
  for (int cch = 0; cch < GC; ++cch) {
    const int g = (4 * cch + (rk & 3)) % G;
#pragma unroll
    for (int j = 0; j < NCK; ++j)
      qa[cch][j] = *reinterpret_cast<const f16x8*>(qb + g * D + 8 * (4 * j + ck));
  }
  // Entry i of the chunk's page list: the chosen logical page (selected-page
  // stream) and/or the physical page (paged cache), read with clamped indices.
  // The chosen pages are read with early loads, ahead of the valid-length
  // wait.  (The page table of a dense paged stream is left to the compiler,
  // which issues it after the wait: early loads there measured 2% slower on
  // the var-length batch, where half of the workgroups have no keys.)
  constexpr int kListIters =
      ((PAGED || SPARSE) && !SELECT) ? (kMaxChunkPages + kThreads - 1) / kThreads : 0;
  int raw_logical[kListIters > 0 ? kListIters : 1];
  int raw_phys[kListIters > 0 ? kListIters : 1];
  const int32_t* list_row =
      kListIters > 0
          ? reinterpret_cast<const int32_t*>(list) + (SPARSE ? unit : (int64_t)b) * list_width
          : nullptr;
  // Page scores of the unit (selecting mode), all loaded up front at indices
  // clamped to the row; entries past the valid pages are masked in the
  // selection.
  float sel_raw[SELECT ? SEL_R : 1];
  if constexpr (SELECT) {
    const float* srow = reinterpret_cast<const float*>(list) + unit * list_width;
#pragma unroll
    for (int r = 0; r < SEL_R; ++r)
      sel_raw[r] = early_load(srow + min(r * kThreads + (int)tid_, list_width - 1));
  }
#pragma unroll
  for (int r = 0; r < kListIters; ++r) {
    const int e = min(page0 + (int)tid_ + r * kThreads, list_width - 1);
    if constexpr (SPARSE) {
      raw_logical[r] = early_load(list_row + e);
    } else {
      raw_logical[r] = page0 + (int)tid_ + r * kThreads;
      if constexpr (PAGED) {
        if (stage_list) raw_phys[r] = list_row[e];
      }
    }
  }
  if constexpr (PAGED && SPARSE && !SELECT) {
#pragma unroll
    for (int r = 0; r < kListIters; ++r)
      raw_phys[r] = a.page_table[(int64_t)b * a.max_pages + min(max(raw_logical[r], 0), a.max_pages - 1)];
  }

  StreamInfo si;
  if constexpr (PERSIST) {
    si.L = ps->flat_L[b];
    si.n_keys = si.L;
    si.nsplit = ((si.L + kTileKeys - 1) / kTileKeys + a.tiles_per_split - 1) / a.tiles_per_split;
  } else {
    si = stream_info(a, seqlens, b, SPARSE);
  }
  const int L = si.L;
  const int n_keys = si.n_keys;
  const int nsplit = si.nsplit;
  const int n_pages_L = (L + page_mask) >> shift;
  f16* out = reinterpret_cast<f16*>(a.out) + unit * G * D;  // rows h = G*kv + g of batch b

  // Persistent launch, wave 0: the next ticket and its chunk's page list.
  // (A chunk starts on a 16-key tile, so it spans at most kMaxTilesPerSplit *
  // 16 / S pages for S = 8, and at most that many plus one for S >= 16.)
  constexpr int kNextIters =
      PERSIST ? (kMaxTilesPerSplit * kTileKeys / kMinPageSize + kWave - 1) / kWave : 1;
  uint32_t next_fetched = 0;          // lane 0: the counter value fetched
  uint32_t next_ticket = 0xFFFFFFFFu; // the next ticket, or none (>= total)
  int next_page0 = 0, next_npg = 0;
  int next_raw[kNextIters];
  int next_phys0 = 0;
  auto next_fetch = [&]() {
    if (lane == 0)
      next_fetched = __hip_atomic_fetch_add(ps->counter, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  };
  auto next_prepare = [&]() {
    const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)next_fetched, 0);
    next_ticket = (ps->total > ps->grid && v < ps->total - ps->grid) ? ps->grid + v : 0xFFFFFFFFu;
    if (next_ticket < ps->total) {
      uint32_t sp, un;
      persist_lookup(*ps, hkv, next_ticket, sp, un);
      const int bn = (int)(un / (uint32_t)hkv);
      const int Ln = ps->flat_L[bn];
      const int tb = (int)sp * tiles_per_split;
      const int te = min(tb + tiles_per_split, (Ln + kTileKeys - 1) / kTileKeys);
      const int klast = min(te * kTileKeys, Ln) - 1;
      next_page0 = (tb * kTileKeys) >> shift;
      next_npg = (klast >> shift) - next_page0 + 1;
      const int32_t* row = a.page_table + (int64_t)bn * a.max_pages;
#pragma unroll
      for (int r = 0; r < kNextIters; ++r)
        next_raw[r] = row[min(next_page0 + lane + r * kWave, a.max_pages - 1)];
      next_phys0 = row[0];
    }
  };
  auto next_stage = [&]() {  // into the other list buffer, checked as below
    if (next_ticket < ps->total) {
      int32_t* dst = s_page_mem + (ps->buf ^ 1) * kMaxChunkPages;
#pragma unroll
      for (int r = 0; r < kNextIters; ++r) {
        const int i = lane + r * kWave;
        if (i < next_npg) {
          int phys = next_raw[r];
          if (next_page0 + i >= a.max_pages || phys < 0 || phys >= a.num_pages) phys = -1;
          dst[i] = phys;
        }
      }
      if (lane == 0) ps->phys0_slot[ps->buf ^ 1] = next_phys0;
    }
    // (double-buffered like the lists: a chunk without keys writes this
    // before any barrier, while other waves may still read the last value)
    if (lane == 0) ps->next_slot[ps->buf ^ 1] = next_ticket;
  };

  if (split >= nsplit) {
    if constexpr (PERSIST) {
      if (wave == 0) {
        next_fetch();
        next_prepare();
        next_stage();
      }
    }
    if (split == 0) {  // no valid key at all: defined as a zero output
      for (int i = tid_; i < G * D; i += kThreads) out[i] = (f16)0.0f;
      if constexpr (SELECT) {  // and no page to choose
        if (a.sel_idx_out != nullptr)
          for (int i = tid_; i < a.num_sel; i += kThreads)
            a.sel_idx_out[unit * a.num_sel + i] = -1;
      }
    }
    return;
  }

  const int n_tiles = (n_keys + kTileKeys - 1) / kTileKeys;
  const int tile_end = min(tile_begin + tiles_per_split, n_tiles);
  const int key_last = min(tile_end * kTileKeys, n_keys) - 1;

  // Page lists of this chunk into LDS: the physical page of each logical page
  // (paged cache) and/or the chosen logical pages (selected-page stream).
  // Entries that do not name an existing page become -1.
  if constexpr (SELECT) {
    // The unit's choice, of which this chunk keeps positions [page0, page0 +
    // npg); the first split writes all of it out.
    const int npg = (key_last >> shift) - page0 + 1;
    const int K = a.num_sel;
    const int n_scored = min(n_pages_L, list_width);
    int32_t* idx_out =
        (split == 0 && a.sel_idx_out != nullptr) ? a.sel_idx_out + unit * K : nullptr;
    auto emit = [&](int pos, int page) {
      if (idx_out != nullptr) idx_out[pos] = page;
      const int li = pos - page0;
      if (li >= 0 && li < npg) s_page[li] = page;
    };
    if (n_scored <= K) {
      choose_all(n_scored, K, emit);
    } else {
      select_top_k<SEL_R>(sel_raw, n_scored, K, emit);
    }
    __syncthreads();
    if constexpr (PAGED) {
      for (int i = tid_; i < npg; i += kThreads) {
        const int logical = s_page[i];
        int phys = (logical >= 0 && logical < a.max_pages)
                       ? a.page_table[(int64_t)b * a.max_pages + logical]
                       : -1;
        if (phys < 0 || phys >= a.num_pages) phys = -1;
        s_phys[i] = phys;
      }
      __syncthreads();
    }
  } else if constexpr (PAGED || SPARSE) {
    if (stage_list) {
      const int npg = (key_last >> shift) - page0 + 1;
#pragma unroll
      for (int r = 0; r < kListIters; ++r) {
        const int i = (int)tid_ + r * kThreads;
        if (i < npg) {
          int logical = raw_logical[r];
          if constexpr (SPARSE) {
            if (logical < 0 || logical >= n_pages_L) logical = -1;
          }
          int entry = logical;
          if constexpr (PAGED) {
            int phys = raw_phys[r];
            if (logical < 0 || logical >= a.max_pages || phys < 0 || phys >= a.num_pages) phys = -1;
            if constexpr (SPARSE) {
              s_phys[i] = phys;
            } else {
              entry = phys;
            }
          }
          s_page[i] = entry;
        }
      }
      if constexpr (PERSIST) {
        if (tid_ == 0) ps->phys0_slot[ps->buf] = a.page_table[(int64_t)b * a.max_pages];
      }
      __syncthreads();
    }
  }

  // Masked keys, and the ring's loads past the chunk, read a row that holds
  // this sequence's data instead of their own slot, so the value multiplied
  // by their zero weight is finite.  Contiguous cache: the chunk's first row
  // (dense: row key_begin; chosen pages: the first row of the chunk's first
  // chosen page), which is valid and which this workgroup loads first, so
  // these loads hit in cache instead of waiting on a cold row at the end of
  // the loop.  Paged cache: token 0 of the sequence; a page-table entry
  // outside the pool falls back to pool page 0, which always exists.
  const bool has_new = a.k_new != nullptr;
  int64_t safe_off;
  // with an append, a redirected key reads k_new/v_new instead when the safe
  // row may be the slot this call is writing (L - 1)
  bool safe_is_new;
  if constexpr (PAGED) {
    int phys0;
    if constexpr (PERSIST) {
      phys0 = ps->phys0_slot[ps->buf];
    } else {
      phys0 = a.page_table[(int64_t)b * a.max_pages];
    }
    if (phys0 < 0 || phys0 >= a.num_pages) phys0 = 0;
    safe_off = (((int64_t)phys0 * hkv + kv) << shift) * D;
    safe_is_new = has_new;
  } else if constexpr (!SPARSE) {
    safe_off = (unit * a.cache_stride + key_begin) * D;
    safe_is_new = has_new && key_begin >= L - 1;
  } else {
    // the chunk's list was staged above; an entry that names no page falls
    // back to token 0
    const int first_page = s_page[0];
    safe_off = (unit * a.cache_stride + (first_page >= 0 ? (first_page << shift) : 0)) * D;
    safe_is_new = has_new;
  }

  const f16* kc = reinterpret_cast<const f16*>(k);
  const f16* vc = reinterpret_cast<const f16*>(v);
  const f16* knew_row = has_new ? reinterpret_cast<const f16*>(a.k_new) + unit * D : nullptr;
  const f16* vnew_row = has_new ? reinterpret_cast<const f16*>(a.v_new) + unit * D : nullptr;

  // Row r of the unit is query position r % q_len of head G * kv + r / q_len
  // (group and sequence axes merged); it sees keys t < L - q_len + 1 + r % q_len.
  // With q_len = 1 every row sees the whole valid length.
  int lim[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lim[g] = L - a.q_len + 1 + g % a.q_len;

  float m[G], l[G], acc[G][NV];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegBig;
    l[g] = 0.0f;
#pragma unroll
    for (int x = 0; x < NV; ++x) acc[g][x] = 0.0f;
  }

  // Append: the new row goes to slot L - 1 of the cache.  Only the workgroup
  // whose chunk holds that slot writes it, and its own loads of that key are
  // redirected to k_new/v_new, so no other read of the slot can race.
  if (has_new && !SPARSE && key_begin <= L - 1 && L - 1 <= key_last) {
    int64_t off;
    if constexpr (PAGED) {
      int phys = a.page_table[(int64_t)b * a.max_pages + ((L - 1) >> shift)];
      off = (phys >= 0 && phys < a.num_pages)
                ? (((int64_t)phys * hkv + kv) << shift) * D + (int64_t)((L - 1) & page_mask) * D
                : -1;
    } else {
      off = (unit * a.cache_stride + (L - 1)) * D;
    }
    if (off >= 0 && tid_ < 2 * (D / 8)) {
      const int c16 = tid_ % (D / 8);
      const f16* src = (tid_ < D / 8 ? knew_row : vnew_row) + 8 * c16;
      f16* dst = reinterpret_cast<f16*>(tid_ < D / 8 ? k : v) + off + 8 * c16;
      *reinterpret_cast<f16x8*>(dst) = *reinterpret_cast<const f16x8*>(src);
    }
  }

  // Element offset of stream position j (or the safe row), its validity and
  // its token index.  Positions outside this chunk (live = false) resolve to
  // the safe row: the stage ring issues its loads unconditionally so that the
  // compiler's wait counts stay exact, and such loads only touch that row.
  auto resolve = [&](int j, bool live, bool& valid, int& t) -> int64_t {
    t = j;
    valid = live && j < n_keys;
    int64_t off;
    // The list entries are read unconditionally (the index is in range
    // either way) and masked afterwards, so the reads of a stage issue
    // together instead of each behind a branch and a wait.
    if constexpr (SPARSE) {
      const int li = valid ? (j >> shift) - page0 : 0;  // in range of the LDS list
      const int logical_raw = s_page[li];
      const int phys_raw = PAGED ? s_phys[li] : 0;
      const int logical = valid ? logical_raw : -1;
      t = (logical << shift) + (j & page_mask);
      valid = valid && logical >= 0 && t < L;
      if constexpr (PAGED) {
        const int phys = valid ? phys_raw : -1;
        valid = valid && phys >= 0;
        off = (((int64_t)phys * hkv + kv) << shift) * D + (int64_t)(t & page_mask) * D;
      } else {
        off = (unit * a.cache_stride + t) * D;
      }
    } else if constexpr (PAGED) {
      const int phys_raw = s_page[valid ? (j >> shift) - page0 : 0];
      const int phys = valid ? phys_raw : -1;
      valid = valid && phys >= 0;
      off = (((int64_t)phys * hkv + kv) << shift) * D + (int64_t)(t & page_mask) * D;
    } else {
      off = (unit * a.cache_stride + t) * D;
    }
    return valid ? off : safe_off;
  };

  // Loads of one tile; no branches, so every stage issues the same number of
  // loads and the wait for a stage leaves the later stages in flight.
  auto load_stage = [&](int tile, Stage<D>& st) {
    const bool live = tile < tile_end;
    const int j0 = tile * kTileKeys;
    bool vk, v0, v1;
    int tk, t0, t1;
    const int64_t ok = resolve(j0 + rk, live, vk, tk);
    const int64_t o0 = resolve(j0 + rv, live, v0, t0);
    const int64_t o1 = resolve(j0 + rv + 8, live, v1, t1);
    st.kvalid = vk;
    st.ktok = tk;
    // The appended key reads k_new/v_new, and so does a redirected key when
    // its safe row may be the slot being written (not finite yet).
    const f16* kp = (has_new && (vk ? tk == L - 1 : safe_is_new)) ? knew_row : kc + ok;
    const f16* vp0 = (has_new && (v0 ? t0 == L - 1 : safe_is_new)) ? vnew_row : vc + o0;
    const f16* vp1 = (has_new && (v1 ? t1 == L - 1 : safe_is_new)) ? vnew_row : vc + o1;
    // K and V are streamed once: non-temporal loads (measured about 20%
    // more read bandwidth than default-policy loads on this part).
#pragma unroll
    for (int j = 0; j < NCK; ++j)
      st.k[j] = stream_load(kp + 8 * (4 * j + ck));
#pragma unroll
    for (int h = 0; h < NCV; ++h) {
      st.v0[h] = stream_load(vp0 + 8 * (8 * h + cv));
      st.v1[h] = stream_load(vp1 + 8 * (8 * h + cv));
    }
  };

  auto compute_stage = [&](const Stage<D>& st) {
    // scores of this lane's K key, all G rows
    float sk[G];
#pragma unroll
    for (int cch = 0; cch < GC; ++cch) {
      f32x4 d4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < NCK; ++j) {
        const f16x4 blo = {st.k[j][0], st.k[j][1], st.k[j][2], st.k[j][3]};
        const f16x4 bhi = {st.k[j][4], st.k[j][5], st.k[j][6], st.k[j][7]};
        const f16x4 alo = {qa[cch][j][0], qa[cch][j][1], qa[cch][j][2], qa[cch][j][3]};
        const f16x4 ahi = {qa[cch][j][4], qa[cch][j][5], qa[cch][j][6], qa[cch][j][7]};
        d4 = __builtin_amdgcn_mfma_f32_16x16x16f16(alo, blo, d4, 0, 0, 0);
        d4 = __builtin_amdgcn_mfma_f32_16x16x16f16(ahi, bhi, d4, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * cch + r < G) sk[4 * cch + r] = d4[r];
    }
    // scores of the two V keys of this lane: keys (lane % 8) and + 8
    float sa[G], sb[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mine = (st.kvalid && st.ktok < lim[g]) ? sk[g] * a.scale_log2 : -INFINITY;
      const float other = lane_xor<8>(mine);
      sa[g] = upper ? other : mine;
      sb[g] = upper ? mine : other;
    }
    bool need = false;
#pragma unroll
    for (int g = 0; g < G; ++g) need |= fmaxf(sa[g], sb[g]) > m[g] + kRescaleThreshold;
    if (need) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(m[g], fmaxf(sa[g], sb[g]));
        const float f = fast_exp2(m[g] - mn);
        l[g] *= f;
#pragma unroll
        for (int x = 0; x < NV; ++x) acc[g][x] *= f;
        m[g] = mn;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pa = fast_exp2(sa[g] - m[g]);
      const float pb = fast_exp2(sb[g] - m[g]);
      l[g] += pa + pb;
#pragma unroll
      for (int h = 0; h < NCV; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = fmaf(pa, (float)st.v0[h][e], acc[g][h * 8 + e]);
          acc[g][h * 8 + e] = fmaf(pb, (float)st.v1[h][e], x);
        }
    }
  };

  // Ring of NS register stages: stage s holds the wave's tiles first + s*4,
  // first + (s + NS)*4, ... (4 = waves per workgroup, the wave's stride).
  {
    Stage<D> st[NS];
    const int first = tile_begin + wave;
    // persistent launch: wave 0 takes the next ticket at the start of its
    // second-to-last ring round and loads the next page list at the end of
    // it (by then the fetch has returned along with that round's loads);
    // measured equal to the last round and to the third- or fourth-to-last
    int next_base = 0x7FFFFFFF;
    if constexpr (PERSIST) {
      const int rounds = (tile_end - tile_begin + NS * kWaves - 1) / (NS * kWaves);
      if (wave == 0) next_base = tile_begin + max(rounds - 2, 0) * NS * kWaves;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) load_stage(first + s * kWaves, st[s]);
    for (int base = first; base < tile_end; base += NS * kWaves) {
      if (!DRAIN || base + NS * kWaves < tile_end) {
        if constexpr (PERSIST) {
          if (base == next_base) next_fetch();
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int t = base + s * kWaves;
          if (t < tile_end) compute_stage(st[s]);
          load_stage(t + NS * kWaves, st[s]);
        }
        if constexpr (PERSIST) {
          if (base == next_base) next_prepare();
        }
      } else {
        // DRAIN: the last round issues no loads past the chunk, so the code
        // after the loop does not wait for them
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int t = base + s * kWaves;
          if (t < tile_end) compute_stage(st[s]);
        }
        break;
      }
    }
  }

  // Merge the 8 key slots of each V channel group (log-sum-exp).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = group_max<8>(m[g]);
    const float f = fast_exp2(m[g] - M);
    l[g] = group_sum<8>(l[g] * f);
#pragma unroll
    for (int x = 0; x < NV; ++x) acc[g][x] = group_sum<8>(acc[g][x] * f);
    m[g] = M;
  }
  if (rv == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int h = 0; h < NCV; ++h) {
        float* dst = &s_o[wave][g][8 * (8 * h + cv)];
        *reinterpret_cast<f32x4*>(dst) =
            f32x4{acc[g][h * 8 + 0], acc[g][h * 8 + 1], acc[g][h * 8 + 2], acc[g][h * 8 + 3]};
        *reinterpret_cast<f32x4*>(dst + 4) =
            f32x4{acc[g][h * 8 + 4], acc[g][h * 8 + 5], acc[g][h * 8 + 6], acc[g][h * 8 + 7]};
      }
      if (cv == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  if constexpr (PERSIST) {
    if (wave == 0) next_stage();  // the other buffer: nobody reads it now
  }

  // Merge the waves of this workgroup; write the output (single split) or
  // this split's partial.
  float* part_o = a.part_o + (unit * a.max_splits + split) * G * D;
  float* part_ml = a.part_ml + (unit * a.max_splits + split) * G * 2;
  for (int i = tid_; i < G * D; i += kThreads) {
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
}

// Flat work list of a dense stream over sequences of unequal lengths: chunk
// `w` of the grid (any workgroup, each wave computes the same answer) in an
// order that holds only chunks with keys -- a sequence without keys keeps one
// chunk, which writes its zero output -- longest sequences first (equal
// lengths in index order) when there are at most 64 sequences, in index order
// otherwise.  Consecutive workgroups take the Hkv heads of one chunk, so the
// heads of every chunk spread over the XCDs.  Returns false past the last
// chunk.  (The grid, max_splits * B * Hkv workgroups, is sized on the host,
// which does not know the lengths.)
__device__ __forceinline__ bool flat_chunk(const int32_t* __restrict__ seqlens, int batch, int hkv,
                                           int tiles_per_split, int capacity, uint32_t w,
                                           uint32_t& split_u, uint32_t& unit_u) {
  const int lane = lane_in_wave();
  const uint32_t f = w / (uint32_t)hkv;  // flat chunk index
  const uint32_t kv = w - f * (uint32_t)hkv;
  auto chunks = [&](int L) {
    L = L < 0 ? 0 : (L > capacity ? capacity : L);
    const int n = ((L + kTileKeys - 1) / kTileKeys + tiles_per_split - 1) / tiles_per_split;
    return n < 1 ? 1 : n;
  };
  if (batch <= kWave) {
    int L = lane < batch ? seqlens[lane] : -1;
    L = lane < batch ? (L < 0 ? 0 : (L > capacity ? capacity : L)) : -1;
    const int n = lane < batch ? chunks(L) : 0;
    int rank = 0;  // sequences before this one: longer, or as long with a lower index
    for (int j = 0; j < batch; ++j) {
      const int Lj = __builtin_amdgcn_readlane(L, j);
      rank += (Lj > L || (Lj == L && j < lane)) ? 1 : 0;
    }
    int start = 0;  // its first flat chunk: the chunks of every sequence before it
    for (int j = 0; j < batch; ++j) {
      const int rj = __builtin_amdgcn_readlane(rank, j);
      const int nj = __builtin_amdgcn_readlane(n, j);
      start += rj < rank ? nj : 0;
    }
    const uint64_t hit =
        __ballot(lane < batch && (uint32_t)start <= f && f < (uint32_t)(start + n));
    if (hit == 0) return false;
    const int b = __builtin_ctzll(hit);
    split_u = f - (uint32_t)__builtin_amdgcn_readlane(start, b);
    unit_u = (uint32_t)b * (uint32_t)hkv + kv;
    return true;
  }
  uint32_t base = 0;
  for (int b0 = 0; b0 < batch; b0 += kWave) {
    const int b = b0 + lane;
    const uint32_t n = b < batch ? (uint32_t)chunks(seqlens[b]) : 0u;
    const uint32_t inc = wave_inclusive_scan(n);
    const uint32_t start = base + inc - n;
    const uint64_t hit = __ballot(b < batch && start <= f && f < start + n);
    if (hit != 0) {
      const int l = __builtin_ctzll(hit);
      split_u = f - (uint32_t)__builtin_amdgcn_readlane((int)start, l);
      unit_u = (uint32_t)(b0 + l) * (uint32_t)hkv + kv;
      return true;
    }
    base += (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
  }
  return false;
}

// One workgroup per (split, unit).  The paged dense stream (the batched
// decode of sequences of unequal lengths) takes its chunk from the flat work
// list; the other streams use a 1-D grid of splits x units, unit index
// fastest.
template <int D, int G, bool PAGED, bool SPARSE, int SEL_R, bool DRAIN>
__global__ void __launch_bounds__(kThreads)
    decode_kernel(const int32_t* __restrict__ seqlens, const void* __restrict__ q, void* k,
                  void* v, const void* __restrict__ list, int batch, int hkv, int list_width,
                  int chunk_geom, AttnLaunch a) {
  uint32_t split_u, unit_u;
  if constexpr (PAGED && !SPARSE) {
    if (!flat_chunk(seqlens, batch, hkv, chunk_geom & 0xFFFF, a.capacity, blockIdx.x, split_u,
                    unit_u))
      return;
  } else {
    // grid < 2^31 workgroups (checked on the host): 32-bit index arithmetic
    const uint32_t n_units = (uint32_t)batch * (uint32_t)hkv;
    split_u = blockIdx.x / n_units;
    unit_u = blockIdx.x - split_u * n_units;
  }
  attend_chunk<D, G, PAGED, SPARSE, SEL_R, DRAIN>(seqlens, q, k, v, list, batch, hkv,
                                                  list_width, chunk_geom, a, split_u, unit_u);
}

// The persistent launch of the paged dense stream (see Persist): the flat
// list is built once per workgroup, then the workgroup runs ticket after
// ticket.  Every wave of a workgroup leaves the loop together (the ticket
// comes from LDS after a barrier); a workgroup ends at its first fetched
// value past the tickets, which every workgroup reaches after at most T
// fetches in all.
template <int D, int G>
__global__ void __launch_bounds__(kThreads)
    paged_persist_kernel(const int32_t* __restrict__ seqlens, const void* __restrict__ q, void* k,
                         void* v, const void* __restrict__ list, int batch, int hkv,
                         int list_width, int chunk_geom, AttnLaunch a) {
  __shared__ uint32_t s_next[2];
  __shared__ int32_t s_phys0[2];
  __shared__ int32_t s_fL[kWave], s_fstart[kWave], s_fn[kWave];
  const int lane = lane_in_wave();
  const int tps = chunk_geom & 0xFFFF;
  // lane b: sequence b's clamped length, chunk count and first flat chunk
  // (longest first, equal lengths in index order), as in flat_chunk
  int L = early_load(seqlens + min(lane, batch - 1));
  L = lane < batch ? (L < 0 ? 0 : (L > a.capacity ? a.capacity : L)) : -1;
  int n = 0;
  if (lane < batch) {
    n = ((L + kTileKeys - 1) / kTileKeys + tps - 1) / tps;
    n = n < 1 ? 1 : n;
  }
  int rank = 0;
  for (int j = 0; j < batch; ++j) {
    const int Lj = __builtin_amdgcn_readlane(L, j);
    rank += (Lj > L || (Lj == L && j < lane)) ? 1 : 0;
  }
  int start = 0;
  for (int j = 0; j < batch; ++j) {
    const int rj = __builtin_amdgcn_readlane(rank, j);
    const int nj = __builtin_amdgcn_readlane(n, j);
    start += rj < rank ? nj : 0;
  }
  const uint32_t chunks =
      (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan((uint32_t)n), kWave - 1);
  if (threadIdx.x < kWave) {
    s_fL[lane] = L;
    s_fstart[lane] = start;
    s_fn[lane] = n;
  }
  __syncthreads();
  Persist ps;
  ps.counter = a.work_counter;
  ps.next_slot = s_next;
  ps.phys0_slot = s_phys0;
  ps.flat_L = s_fL;
  ps.flat_start = s_fstart;
  ps.flat_n = s_fn;
  ps.grid = gridDim.x;
  ps.total = chunks * (uint32_t)hkv;
  ps.batch = batch;
  ps.buf = 0;
  ps.staged = false;
  uint32_t t = blockIdx.x;
  if (t >= ps.total) return;
  while (true) {
    uint32_t split_u, unit_u;
    persist_lookup(ps, hkv, t, split_u, unit_u);
    attend_chunk<D, G, true, false, 0, false, true>(seqlens, q, k, v, list, batch, hkv, list_width,
                                                    chunk_geom, a, split_u, unit_u, &ps);
    __syncthreads();
    t = s_next[ps.buf ^ 1];
    if (t >= ps.total) break;
    ps.buf ^= 1;
    ps.staged = true;
  }
}

// Clears the work counter of the persistent launch (a kernel rather than a
// memset, so that a captured graph replays it as such).
__global__ void __launch_bounds__(kWave) counter_clear_kernel(uint32_t* counter) {
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroups of the persistent launch: as many as are resident at once (its
// register use decides how many per CU), so that no workgroup waits for
// another to exit before it takes its first ticket.  The per-CU figure is a
// property of the compiled kernel, looked up once.
template <int D, int G>
uint32_t persist_grid() {
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(paged_persist_kernel<D, G>), kThreads, 0) !=
            hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 1;
  return (uint32_t)(per_cu * cus);
}

// Merge kernel: one workgroup per (b, kv) unit, one thread per output element
// of the unit's G rows (G * D threads, 64 to 1024); up to 48 splits are merged
// with one round of loads (merge_partials).
// Leading scalar arguments as in the attention kernel: what the first round
// of partial loads needs.
template <int D, int G, bool SPARSE, int KB>
__global__ void __launch_bounds__(G * D)
    merge_kernel(const float* __restrict__ part_ml, const float* __restrict__ part_o,
                 const int32_t* __restrict__ seqlens, int max_splits, int hkv, AttnLaunch a) {
  const int kv = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t unit = (int64_t)b * hkv + kv;
  merge_partials<D, G, G * D, KB>(a, part_ml, part_o, max_splits, unit,
                              [&] { return stream_info(a, seqlens, b, SPARSE).nsplit; });
}

template <int D, int G, bool PAGED, bool SPARSE, int SEL_R>
int launch_one(const AttnLaunch& a, hipStream_t stream) {
  const void* list = SEL_R > 0 ? static_cast<const void*>(a.sel_scores)
                   : SPARSE    ? static_cast<const void*>(a.page_idx)
                               : static_cast<const void*>(a.page_table);
  const int list_width = SEL_R > 0 ? a.sel_row : SPARSE ? a.num_sel : (PAGED ? a.max_pages : 1);
  // tiles per chunk < 2^16 (at most kMaxTilesPerSplitContiguous)
  const int chunk_geom = a.tiles_per_split | (a.page_shift << 16);
  const dim3 grid((uint32_t)a.max_splits * (uint32_t)a.batch * (uint32_t)a.num_kv_heads);
  // Short chunks of a contiguous cache (at most two ring rounds per wave,
  // such as a few thousand keys split over the chip) use the draining ring;
  // long chunks keep the plain one (the drain measured 1.5% slower on them),
  // and so does the paged cache (10% slower with it).  With 8 rows of D = 128
  // the draining ring does not fit in registers (the compiler spilled 170 to
  // 280 of them to scratch memory) and is not built: the plain ring, at 325
  // registers, measured 2.2x faster on such chunks (G = 8 at 4096 keys:
  // 43.2 -> 19.3 us).
  constexpr bool kDrainFits = !(D == 128 && G == 8);
  const bool drain = kDrainFits && !PAGED && a.tiles_per_split <= 2 * kStages * kWaves;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, a.seqlens, a.q, a.k, a.v, list,
                       a.batch, a.num_kv_heads, list_width, chunk_geom, a);
  };
  // The persistent launch of the paged dense stream pays where the rows times
  // the head dimension reach 512 (4 rows of D = 128, 8 of D = 64): it measured 1.5%
  // faster at D = 128, G = 4, 13.5% at D = 128, G = 8 and 8% at D = 64, G = 8
  // on the batch of 64 (lengths 1K-32K), and equal or 1-3% slower than one
  // workgroup per chunk below that (more workgroups fit on a CU there, and
  // the hardware dispatcher hides their start-up).
  constexpr bool kPersistent = PAGED && !SPARSE && SEL_R == 0 && G * D >= 512;
  if constexpr (kPersistent) {
    // where the work list can outnumber the resident workgroups (at most 64
    // sequences); otherwise one workgroup per item
    const uint32_t tickets = (uint32_t)a.max_splits * (uint32_t)a.batch * (uint32_t)a.num_kv_heads;
    const uint32_t resident = a.batch <= kWave ? persist_grid<D, G>() : 0u;
    if (tickets > resident && a.batch <= kWave) {
      hipLaunchKernelGGL(counter_clear_kernel, dim3(1), dim3(kWave), 0, stream, a.work_counter);
      hipLaunchKernelGGL((paged_persist_kernel<D, G>), dim3(resident), dim3(kThreads), 0, stream,
                         a.seqlens, a.q, a.k, a.v, list, a.batch, a.num_kv_heads, list_width,
                         chunk_geom, a);
    } else {
      go(decode_kernel<D, G, true, SPARSE, SEL_R, false>);
    }
  } else if constexpr (PAGED) {
    go(decode_kernel<D, G, true, SPARSE, SEL_R, false>);
  } else if (drain) {
    if constexpr (kDrainFits) go(decode_kernel<D, G, false, SPARSE, SEL_R, true>);
  } else {
    go(decode_kernel<D, G, false, SPARSE, SEL_R, false>);
  }
  const int err = (int)hipGetLastError();
  if (err != 0 || a.max_splits <= 1) return err;
  // a round of loads covers at most max_splits splits: no loads past them
  auto merge = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(a.num_kv_heads, a.batch), dim3(G * D), 0, stream, a.part_ml,
                       a.part_o, a.seqlens, a.max_splits, a.num_kv_heads, a);
  };
  if (a.max_splits <= 8) {
    merge(merge_kernel<D, G, SPARSE, 8>);
  } else if (a.max_splits <= 16) {
    merge(merge_kernel<D, G, SPARSE, 16>);
  } else {
    merge(merge_kernel<D, G, SPARSE, 48>);
  }
  return (int)hipGetLastError();
}

}  // namespace
}  // namespace da

#endif  // DA_ATTENTION_IMPL_H
