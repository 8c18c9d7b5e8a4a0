// Internal launch interface between the C ABI layer (api.cpp, plain C++) and
// the HIP kernels.  No HIP types appear here so the host layer compiles as
// ordinary C++.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace da {

// One launch of the split-context decode attention kernel (dense, paged or
// selected-page key stream).  All pointers are device pointers.
struct AttnLaunch {
  const void* q;             // fp16 [B, Hq, D]
  void* k;                   // fp16 cache [B, Hkv, cap, D] or pool [NP, Hkv, S, D]
  void* v;
  const int32_t* page_table; // [B, max_pages] or nullptr (contiguous cache)
  const int32_t* seqlens;    // [B]
  const int32_t* page_idx;   // [B, Hkv, num_sel] chosen pages, or nullptr (dense)
  const void* k_new;         // fp16 [B, Hkv, D] or nullptr
  const void* v_new;
  void* out;                 // fp16 [B, Hq, D]
  float* part_ml;            // [B * Hkv, max_splits, G, 2]
  float* part_o;             // [B * Hkv, max_splits, G, D]
  int32_t batch;
  int32_t num_kv_heads;
  int32_t group;             // rows per KV head: (Hq / Hkv) * q_len
  int32_t q_len;             // query positions per head (the last q_len of each sequence)
  int32_t head_dim;          // D
  int32_t capacity;          // valid-length clamp: cap (contiguous) or max_pages * S
  int32_t cache_stride;      // slots per (b, kv) row of a contiguous cache
  int32_t page_shift;        // log2(S) (paged cache and/or selected pages)
  int32_t max_pages;         // page-table row width
  int64_t num_pages;         // pool size; page-table entries outside [0, num_pages) are skipped
  int32_t num_sel;           // K pages per (b, kv) in the selected-page stream
  int32_t tiles_per_split;   // key tiles per workgroup chunk
  int32_t max_splits;        // splits per (b, kv) unit; the grid is max_splits * B * Hkv
  float scale_log2;          // scale * log2(e)
  // Pages chosen in the launch (sel_scores != nullptr, page_idx == nullptr):
  // every workgroup runs the top-K of its unit's page scores and attends over
  // its part of the choice; split 0 writes the choice to sel_idx_out.
  const float* sel_scores;   // [B, Hkv, sel_row] page scores, or nullptr
  int32_t* sel_idx_out;      // [B, Hkv, num_sel] or nullptr
  int32_t sel_row;           // score row width (<= 16384)
  // Ticket counter of the persistent paged launch: the workspace's first 4
  // bytes, cleared by the call before that launch (attention_impl.h, Persist).
  uint32_t* work_counter;
};

// Split plan shared by the workspace-size query and the launch.
struct SplitPlan {
  int32_t keys_per_tile;
  int32_t tiles_per_split;
  int32_t max_splits;
};

int keys_per_tile(int head_dim, int group);
int max_tiles_per_split(bool page_list);  // page_list: paged cache or chosen pages

int launch_decode(const AttnLaunch& p, void* stream);
// the selecting variant (p.sel_scores != nullptr); called by launch_decode
int launch_select_attention(const AttnLaunch& p, void* stream);

struct MetaLaunch {
  void* k;                   // cache or pool (written only when k_new != nullptr)
  void* v;
  const int32_t* page_table;
  const int32_t* seqlens;
  const void* k_new;
  const void* v_new;
  void* meta;                // fp16 [B, Hkv, meta_max_pages, 2, D]
  int32_t batch, num_kv_heads, head_dim;
  int32_t capacity, cache_stride, page_shift, max_pages;
  int64_t num_pages;
  int32_t meta_max_pages;
  int32_t n_new;
  int32_t pages_per_seq;     // grid.x: pages a single call can touch per sequence
};
int launch_meta_append(const MetaLaunch& p, void* stream);

struct ScoreLaunch {
  const void* q;             // fp16 [B, Hq, D]
  void* meta;                // fp16 [B, Hkv, P, 2, D]; written only with k_new
  const int32_t* seqlens;
  float* scores;             // [B, Hkv, P]
  int32_t* page_idx;         // [B, Hkv, K]
  int32_t batch, num_kv_heads, group, head_dim;
  int32_t page_shift, meta_max_pages, num_sel;
  int32_t score_passes;      // set by the launcher
  // Fused decode-step append (k_new != nullptr): row min(L_b, capacity) - 1 of
  // the cache receives k_new / v_new and its page's metadata is updated (reset
  // at a page start, min/max otherwise) before the page is scored.  (The
  // scalars come first: they share a kernel-argument cache line with the
  // fields above.)
  int32_t capacity, cache_stride, max_pages;
  const void* k_new;         // fp16 [B, Hkv, D] or nullptr
  const void* v_new;
  void* k;                   // cache or pool (written only with k_new)
  void* v;
  const int32_t* page_table; // [B, max_pages] or nullptr (contiguous cache)
  int64_t num_pages;
};
int launch_score_topk(const ScoreLaunch& p, void* stream);
// The top-K alone over p.scores (p.page_idx receives it), for any page count.
int launch_topk_only(const ScoreLaunch& p, void* stream);
// Pages per unit up to which the top-K holds the scores in registers (and the
// attention launch can select its own pages); above it the streaming select runs.
int topk_max_pages();

// Materialised repeat_kv: rows t < L_b of every KV head copied to its G query
// heads, out [B, Hq, out_capacity, D].
struct RepeatLaunch {
  const void* k;             // cache or pool
  const void* v;
  const int32_t* page_table;
  const int32_t* seqlens;
  void* k_out;               // fp16 [B, Hq, out_capacity, D]
  void* v_out;
  int32_t batch, num_kv_heads, group, head_dim;
  int32_t capacity, cache_stride, page_shift, max_pages;
  int64_t num_pages;
  int32_t out_capacity;
};
int launch_repeat_kv(const RepeatLaunch& p, void* stream);
int repeat_kv_rows_per_workgroup();

// The library's static scratch for the entry point that allocates nothing:
// its size, and its device address on the current device (looked up once per
// device; 0 or a HIP error code).
size_t noalloc_scratch_bytes();
int noalloc_scratch(void** ptr);

// Streaming-read calibration over `bytes` (a multiple of 16) at `src`.
int launch_read_calibration(const void* src, uint64_t bytes, uint32_t* sink, void* stream);

}  // namespace da
