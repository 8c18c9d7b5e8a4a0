// C ABI of libdecode_attn.so (declared in include/decode_attn.h): argument
// validation, workspace layout, split planning and kernel launches.
//
// Every check here runs before anything is enqueued, so a rejected call has no
// side effect.  This file is plain C++ (no HIP headers); the kernels sit behind
// the launch functions of kernels.h and report HIP errors as non-zero ints.

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/decode_attn.h"
#include "check.h"
#include "kernels.h"

namespace {

constexpr int kMaxGridDim = 65535;
// Pages per (b, kv) row of the Quest metadata and scores: keeps the kernels'
// 32-bit page arithmetic (index plus a few thousand) clear of overflow.
constexpr int kMaxMetaPages = 1 << 28;
// Split plan: enough key tiles per workgroup that the grid is about one
// workgroup per CU (256 CUs), longer chunks where the stream allows.  Measured
// against 384, 512, 768 and 1024: equal on the dense and paged workloads
// (their chunks are at the chunk cap or the 8-tile floor) and best on the
// 128K selected-page stream (34.4 us vs 35.2 at 512, 37.0 at 768, 40 at 384).
constexpr int kTargetWorkgroups = 256;
constexpr int kMinTilesPerSplit = 8;     // at least 2 tiles per wave

bool is_pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

int log2i(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct Shape {
  int batch, hkv, hq, group, d;
  int capacity;      // valid-length clamp
  int stride;        // contiguous slots per (b, kv)
  bool paged;
  int page_size;     // paged pool or Quest page size
  int max_pages;
};

// Checks shared by the attention entry points.
int check_cache(const da_kv_cache* kv, int32_t num_q_heads, Shape* s) {
  if (kv == nullptr) return DA_ERR_NULL;
  if (kv->batch < 0 || kv->num_kv_heads < 1 || num_q_heads < 1) return DA_ERR_SHAPE;
  if (kv->batch > kMaxGridDim || kv->num_kv_heads > kMaxGridDim) return DA_ERR_SHAPE;
  if (num_q_heads % kv->num_kv_heads != 0) return DA_ERR_SHAPE;
  const int group = num_q_heads / kv->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return DA_ERR_UNSUPPORTED;
  if (kv->head_dim != 64 && kv->head_dim != 128) return DA_ERR_UNSUPPORTED;
  s->batch = kv->batch;
  s->hkv = kv->num_kv_heads;
  s->hq = num_q_heads;
  s->group = group;
  s->d = kv->head_dim;
  s->paged = kv->page_table != nullptr;
  s->page_size = kv->page_size;
  if (s->paged) {
    if (!is_pow2_in(kv->page_size, 8, 64)) return DA_ERR_UNSUPPORTED;
    if (kv->max_pages < 1 || kv->num_pages < 1) return DA_ERR_SHAPE;
    if ((int64_t)kv->max_pages * kv->page_size > INT32_MAX / 2) return DA_ERR_SHAPE;
    s->max_pages = kv->max_pages;
    s->capacity = kv->max_pages * kv->page_size;
    s->stride = 0;
  } else {
    if (kv->capacity < 1 || kv->capacity > INT32_MAX / 2) return DA_ERR_SHAPE;
    s->max_pages = 0;
    s->capacity = kv->capacity;
    s->stride = kv->capacity;
  }
  return DA_OK;
}

// page_list: the stream reads a page list (paged cache or chosen pages).
da::SplitPlan plan_splits(const Shape& s, int max_keys, int num_splits, bool page_list) {
  da::SplitPlan p;
  p.keys_per_tile = da::keys_per_tile(s.d, s.group);
  const int64_t max_tiles = max_keys < 1 ? 1 : (max_keys + p.keys_per_tile - 1) / p.keys_per_tile;
  int64_t tps;
  if (num_splits > 0) {
    tps = (max_tiles + num_splits - 1) / num_splits;
  } else {
    const int64_t total = (int64_t)s.batch * s.hkv * max_tiles;
    tps = (total + kTargetWorkgroups - 1) / kTargetWorkgroups;
    if (tps < kMinTilesPerSplit) tps = kMinTilesPerSplit;
  }
  if (tps < 1) tps = 1;
  if (tps > da::max_tiles_per_split(page_list)) tps = da::max_tiles_per_split(page_list);
  if (tps > max_tiles) tps = max_tiles;
  p.tiles_per_split = (int32_t)tps;
  p.max_splits = (int32_t)((max_tiles + tps - 1) / tps);
  return p;
}

constexpr size_t kCounterBytes = 256;

struct WsLayout {
  size_t ml, o, idx, total;
};

// Workspace: the first 256 bytes hold the work counter of the persistent
// paged launch (cleared by the call before that launch, so the workspace
// needs no initialisation); then per (b, kv, split) partial softmax state (m, l)
// and unnormalised output o, all fp32; for the selected-page stream (k_sel > 0
// chosen pages per unit) also room for the choice [B, Hkv, k_sel] int32,
// which the page-selecting call fills when the unit has more pages than the
// attention launch selects itself and the caller keeps no copy.
WsLayout ws_layout(const Shape& s, const da::SplitPlan& p, int k_sel) {
  const size_t units = (size_t)s.batch * s.hkv;
  WsLayout w;
  w.ml = kCounterBytes;
  w.o = w.ml + align256(units * p.max_splits * s.group * 2 * sizeof(float));
  const size_t o_bytes = units * p.max_splits * s.group * s.d * sizeof(float);
  w.idx = w.o + align256(o_bytes);
  w.total = k_sel > 0 ? w.idx + units * (size_t)k_sel * sizeof(int32_t) : w.o + o_bytes;
  return w;
}

// Longest key stream one (b, kv) unit can have: the valid length for dense
// attention; for the chosen pages, at most budget tokens and at most every
// page of the sequence (a partial last page still occupies S stream slots).
int max_stream_keys(const Shape& s, int budget_tokens) {
  if (budget_tokens <= 0) return s.capacity;
  const int64_t all_pages = ((int64_t)s.capacity + s.page_size - 1) / s.page_size * s.page_size;
  return (int)(budget_tokens < all_pages ? budget_tokens : all_pages);
}

int check_budget(const Shape& s, int budget_tokens) {
  if (!is_pow2_in(s.page_size, 8, 64)) return DA_ERR_UNSUPPORTED;
  if (budget_tokens <= 0 || budget_tokens % s.page_size != 0) return DA_ERR_BUDGET;
  return DA_OK;
}

// num_rows = Hq * q_len: the kernel reads Q [B, Hq, q_len, D] as
// [B, Hkv, G * q_len, D] rows.
// Pages chosen inside the attention launch from the page scores (the
// selected-page stream without a given page list).
struct PageSelect {
  const float* scores;  // [B, Hkv, row] fp32
  int32_t row;          // pages with a score per (b, kv)
  int32_t* idx_out;     // [B, Hkv, K] the choice, or nullptr
};

// Where the split partials go: the caller's workspace, or (kLibraryScratch)
// the library's static device scratch, whose address is fetched only after
// every argument check has passed.
enum WsSource { kCallerWorkspace, kLibraryScratch };

int run_attention(const void* q, const da_kv_cache* kv, const int32_t* seqlens,
                  const int32_t* page_idx, int32_t budget_tokens, int32_t num_rows,
                  int32_t q_len, float scale, const void* k_new, const void* v_new, void* out,
                  void* workspace, size_t workspace_bytes, int32_t num_splits, void* stream,
                  const PageSelect* select = nullptr, WsSource ws_source = kCallerWorkspace) {
  Shape s;
  int st = check_cache(kv, num_rows, &s);
  if (st != DA_OK) return st;
  if ((k_new == nullptr) != (v_new == nullptr)) return DA_ERR_NULL;
  if (!isfinite(scale)) return DA_ERR_SHAPE;
  if (num_splits < 0) return DA_ERR_SHAPE;
  const bool sparse = page_idx != nullptr || select != nullptr;
  if (sparse) {
    st = check_budget(s, budget_tokens);
    if (st != DA_OK) return st;
  }
  if (s.batch == 0) return DA_OK;  // nothing to read or write (empty tensors may be NULL)
  if (q == nullptr || seqlens == nullptr || out == nullptr || kv->k == nullptr ||
      kv->v == nullptr)
    return DA_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(kv->k) || !aligned16(kv->v) ||
      !aligned16(k_new) || !aligned16(v_new))
    return DA_ERR_SHAPE;
  const da::SplitPlan plan = plan_splits(s, max_stream_keys(s, sparse ? budget_tokens : 0),
                                         num_splits, s.paged || sparse);
  // one workgroup per (split, b, kv) on a 1-D grid
  if ((int64_t)plan.max_splits * s.batch * s.hkv > INT32_MAX) return DA_ERR_SHAPE;
  const int k_sel = sparse ? budget_tokens / s.page_size : 0;
  const WsLayout w = ws_layout(s, plan, k_sel);
  if (ws_source == kLibraryScratch) {
    if (w.total > da::noalloc_scratch_bytes()) return DA_ERR_TOO_LARGE;
    if (da::noalloc_scratch(&workspace) != 0) return DA_ERR_HIP;
    workspace_bytes = da::noalloc_scratch_bytes();
  }
  if (workspace == nullptr) return DA_ERR_NULL;
  if (!aligned16(workspace)) return DA_ERR_SHAPE;
  if (workspace_bytes < w.total) return DA_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  da::AttnLaunch a;
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.page_table = kv->page_table;
  a.seqlens = seqlens;
  a.page_idx = page_idx;
  a.k_new = k_new;
  a.v_new = v_new;
  a.out = out;
  a.work_counter = reinterpret_cast<uint32_t*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + w.ml);
  a.part_o = reinterpret_cast<float*>(ws + w.o);
  a.batch = s.batch;
  a.num_kv_heads = s.hkv;
  a.group = s.group;
  a.q_len = q_len;
  a.head_dim = s.d;
  a.capacity = s.capacity;
  a.cache_stride = s.stride;
  a.page_shift = (s.paged || sparse) ? log2i(s.page_size) : 0;
  a.max_pages = s.max_pages;
  a.num_pages = kv->num_pages;
  a.num_sel = k_sel;
  a.sel_scores = select != nullptr ? select->scores : nullptr;
  a.sel_row = select != nullptr ? select->row : 0;
  a.sel_idx_out = select != nullptr ? select->idx_out : nullptr;
  a.tiles_per_split = plan.tiles_per_split;
  a.max_splits = plan.max_splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  if (select != nullptr && select->row > da::topk_max_pages()) {
    // More pages per unit than the attention launch selects itself: the
    // streaming top-K writes the choice (to page_idx, else the workspace),
    // then the attention reads it as a given list.
    if (s.batch > kMaxGridDim || s.hkv > kMaxGridDim) return DA_ERR_SHAPE;  // its (Hkv, B) grid
    int32_t* idx = select->idx_out != nullptr ? select->idx_out
                                              : reinterpret_cast<int32_t*>(ws + w.idx);
    da::ScoreLaunch t{};
    t.seqlens = seqlens;
    t.scores = const_cast<float*>(select->scores);
    t.page_idx = idx;
    t.batch = s.batch;
    t.num_kv_heads = s.hkv;
    t.group = s.group;
    t.head_dim = s.d;
    t.page_shift = log2i(s.page_size);
    t.meta_max_pages = select->row;
    t.num_sel = k_sel;
    if (da::launch_topk_only(t, stream) != 0) return DA_ERR_HIP;
    a.page_idx = idx;
    a.sel_scores = nullptr;
    a.sel_row = 0;
    a.sel_idx_out = nullptr;
  }
  return da::launch_decode(a, stream) == 0 ? DA_OK : DA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* da_status_string(int status) {
  switch (status) {
    case DA_OK: return "DA_OK";
    case DA_ERR_NULL: return "DA_ERR_NULL: a required pointer is NULL";
    case DA_ERR_SHAPE: return "DA_ERR_SHAPE: inconsistent or misaligned arguments";
    case DA_ERR_UNSUPPORTED: return "DA_ERR_UNSUPPORTED: head_dim, group or page size not supported";
    case DA_ERR_BUDGET: return "DA_ERR_BUDGET: token budget must be a positive multiple of the page size";
    case DA_ERR_WORKSPACE: return "DA_ERR_WORKSPACE: workspace too small";
    case DA_ERR_HIP: return "DA_ERR_HIP: HIP launch or runtime error";
    case DA_ERR_TOO_LARGE:
      return "DA_ERR_TOO_LARGE: the call needs more split-partial scratch than the library's "
             "static buffer holds (DA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int da_workspace_size(const da_kv_cache* kv, int32_t num_q_heads, int32_t budget_tokens,
                      int32_t num_splits, size_t* bytes_out) {
  if (bytes_out == nullptr) return DA_ERR_NULL;
  Shape s;
  int st = check_cache(kv, num_q_heads, &s);
  if (st != DA_OK) return st;
  if (num_splits < 0) return DA_ERR_SHAPE;
  if (budget_tokens > 0) {
    st = check_budget(s, budget_tokens);
    if (st != DA_OK) return st;
  } else if (budget_tokens < 0) {
    return DA_ERR_BUDGET;
  }
  const da::SplitPlan plan = plan_splits(s, max_stream_keys(s, budget_tokens), num_splits,
                                         s.paged || budget_tokens > 0);
  // the same grid limit as the calls: one workgroup per (split, b, kv)
  if ((int64_t)plan.max_splits * s.batch * s.hkv > INT32_MAX) return DA_ERR_SHAPE;
  *bytes_out = ws_layout(s, plan, budget_tokens > 0 ? budget_tokens / s.page_size : 0).total;
  return DA_OK;
}

int gqa_decode_attn(const void* q, const da_kv_cache* kv, const int32_t* seqlens,
                    int32_t num_q_heads, float scale, const void* k_new, const void* v_new,
                    void* out, void* workspace, size_t workspace_bytes, int32_t num_splits,
                    void* stream) {
  return run_attention(q, kv, seqlens, nullptr, 0, num_q_heads, 1, scale, k_new, v_new, out,
                       workspace, workspace_bytes, num_splits, stream);
}

int gqa_decode_attn_noalloc(const void* q, const da_kv_cache* kv, const int32_t* seqlens,
                            int32_t num_q_heads, float scale, const void* k_new,
                            const void* v_new, void* out, int32_t num_splits, void* stream) {
  return run_attention(q, kv, seqlens, nullptr, 0, num_q_heads, 1, scale, k_new, v_new, out,
                       nullptr, 0, num_splits, stream, nullptr, kLibraryScratch);
}

int gqa_decode_attn_multi(const void* q, const da_kv_cache* kv, const int32_t* seqlens,
                          int32_t num_q_heads, int32_t q_len, float scale, void* out,
                          void* workspace, size_t workspace_bytes, int32_t num_splits,
                          void* stream) {
  if (kv == nullptr) return DA_ERR_NULL;
  if (q_len < 1 || num_q_heads < 1 || kv->num_kv_heads < 1) return DA_ERR_SHAPE;
  if (num_q_heads % kv->num_kv_heads != 0) return DA_ERR_SHAPE;
  if ((int64_t)num_q_heads * q_len > INT32_MAX / 2) return DA_ERR_SHAPE;
  return run_attention(q, kv, seqlens, nullptr, 0, num_q_heads * q_len, q_len, scale, nullptr,
                       nullptr, out, workspace, workspace_bytes, num_splits, stream);
}

int quest_sparse_decode_attn(const void* q, const da_kv_cache* kv, const int32_t* seqlens,
                             const int32_t* page_idx, int32_t budget_tokens,
                             int32_t num_q_heads, float scale, void* out, void* workspace,
                             size_t workspace_bytes, int32_t num_splits, void* stream) {
  if (page_idx == nullptr) return DA_ERR_NULL;
  return run_attention(q, kv, seqlens, page_idx, budget_tokens, num_q_heads, 1, scale, nullptr,
                       nullptr, out, workspace, workspace_bytes, num_splits, stream);
}

int gqa_repeat_kv(const da_kv_cache* kv, int32_t num_q_heads, const int32_t* seqlens,
                  void* k_out, void* v_out, void* stream) {
  Shape s;
  int st = check_cache(kv, num_q_heads, &s);
  if (st != DA_OK) return st;
  if (s.paged && !is_pow2_in(s.page_size, 8, 64)) return DA_ERR_UNSUPPORTED;
  const int64_t rows = da::repeat_kv_rows_per_workgroup();
  if ((s.capacity + rows - 1) / rows * s.batch * s.hkv > INT32_MAX) return DA_ERR_SHAPE;
  if (s.batch == 0) return DA_OK;  // nothing to read or write
  if (seqlens == nullptr || kv->k == nullptr || kv->v == nullptr || k_out == nullptr ||
      v_out == nullptr)
    return DA_ERR_NULL;
  if (!aligned16(kv->k) || !aligned16(kv->v) || !aligned16(k_out) || !aligned16(v_out))
    return DA_ERR_SHAPE;
  da::RepeatLaunch a;
  a.k = kv->k;
  a.v = kv->v;
  a.page_table = kv->page_table;
  a.seqlens = seqlens;
  a.k_out = k_out;
  a.v_out = v_out;
  a.batch = s.batch;
  a.num_kv_heads = s.hkv;
  a.group = s.group;
  a.head_dim = s.d;
  a.capacity = s.capacity;
  a.cache_stride = s.stride;
  a.page_shift = s.paged ? log2i(s.page_size) : 0;
  a.max_pages = s.max_pages;
  a.num_pages = kv->num_pages;
  a.out_capacity = s.capacity;
  return da::launch_repeat_kv(a, stream) == 0 ? DA_OK : DA_ERR_HIP;
}

int quest_meta_append(const da_kv_cache* kv, void* meta, int32_t meta_max_pages,
                      const int32_t* seqlens, int32_t n_new, const void* k_new,
                      const void* v_new, void* stream) {
  if (kv == nullptr) return DA_ERR_NULL;
  Shape s;
  // the group size does not matter for metadata; pass Hq = Hkv
  int st = check_cache(kv, kv->num_kv_heads, &s);
  if (st != DA_OK) return st;
  if (!is_pow2_in(s.page_size, 8, 64)) return DA_ERR_UNSUPPORTED;
  if ((k_new == nullptr) != (v_new == nullptr)) return DA_ERR_NULL;
  if (k_new != nullptr && n_new != 1) return DA_ERR_SHAPE;
  if (n_new < 1) return DA_ERR_SHAPE;
  if (meta_max_pages < 1 || meta_max_pages > kMaxMetaPages ||
      (int64_t)meta_max_pages * s.page_size < s.capacity)
    return DA_ERR_SHAPE;
  if (s.batch == 0) return DA_OK;  // nothing to read or write
  if (meta == nullptr || seqlens == nullptr || kv->k == nullptr) return DA_ERR_NULL;
  if (k_new != nullptr && kv->v == nullptr) return DA_ERR_NULL;
  if (!aligned16(meta) || !aligned16(kv->k) || !aligned16(kv->v) || !aligned16(k_new) ||
      !aligned16(v_new))
    return DA_ERR_SHAPE;
  const int n = n_new < s.capacity ? n_new : s.capacity;
  int pages = (n - 1 + s.page_size - 1) / s.page_size + 1;
  if (pages > meta_max_pages) pages = meta_max_pages;
  da::MetaLaunch a;
  a.k = kv->k;
  a.v = kv->v;
  a.page_table = kv->page_table;
  a.seqlens = seqlens;
  a.k_new = k_new;
  a.v_new = v_new;
  a.meta = meta;
  a.batch = s.batch;
  a.num_kv_heads = s.hkv;
  a.head_dim = s.d;
  a.capacity = s.capacity;
  a.cache_stride = s.stride;
  a.page_shift = log2i(s.page_size);
  a.max_pages = s.max_pages;
  a.num_pages = kv->num_pages;
  a.meta_max_pages = meta_max_pages;
  a.n_new = n_new;
  a.pages_per_seq = pages;
  return da::launch_meta_append(a, stream) == 0 ? DA_OK : DA_ERR_HIP;
}

int da_quest_workspace_size(int32_t batch, int32_t num_kv_heads, int32_t meta_max_pages,
                            size_t* bytes_out) {
  if (bytes_out == nullptr) return DA_ERR_NULL;
  if (batch < 0 || num_kv_heads < 1 || meta_max_pages < 1 || meta_max_pages > kMaxMetaPages)
    return DA_ERR_SHAPE;
  *bytes_out = align256((size_t)batch * num_kv_heads * meta_max_pages * sizeof(float));
  if (*bytes_out == 0) *bytes_out = 256;
  return DA_OK;
}

int quest_page_score_topk(const void* q, const void* meta, int32_t meta_max_pages,
                          const int32_t* seqlens, int32_t batch, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                          int32_t budget_tokens, int32_t* page_idx, float* page_scores,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || num_kv_heads < 1 || num_q_heads < 1 || meta_max_pages < 1 ||
      meta_max_pages > kMaxMetaPages)
    return DA_ERR_SHAPE;
  if (batch > kMaxGridDim || num_kv_heads > kMaxGridDim) return DA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return DA_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return DA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return DA_ERR_UNSUPPORTED;
  if (!is_pow2_in(page_size, 8, 64)) return DA_ERR_UNSUPPORTED;
  if (budget_tokens <= 0 || budget_tokens % page_size != 0) return DA_ERR_BUDGET;
  if (batch == 0) return DA_OK;  // nothing to read or write
  if (q == nullptr || meta == nullptr || seqlens == nullptr) return DA_ERR_NULL;
  if (page_idx == nullptr && page_scores == nullptr) return DA_ERR_NULL;  // nothing to output
  if (!aligned16(q) || !aligned16(meta)) return DA_ERR_SHAPE;
  float* scores = page_scores;
  if (scores == nullptr) {
    size_t need = 0;
    da_quest_workspace_size(batch, num_kv_heads, meta_max_pages, &need);
    if (workspace == nullptr) return DA_ERR_NULL;
    if (!aligned16(workspace)) return DA_ERR_SHAPE;
    if (workspace_bytes < need) return DA_ERR_WORKSPACE;
    scores = static_cast<float*>(workspace);
  }
  da::ScoreLaunch a;
  a.q = q;
  a.meta = const_cast<void*>(meta);  // read only: no append on this path
  a.seqlens = seqlens;
  a.scores = scores;
  a.page_idx = page_idx;
  a.batch = batch;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.head_dim = head_dim;
  a.page_shift = log2i(page_size);
  a.meta_max_pages = meta_max_pages;
  a.num_sel = budget_tokens / page_size;
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.k = nullptr;
  a.v = nullptr;
  a.page_table = nullptr;
  a.capacity = 0;
  a.cache_stride = 0;
  a.max_pages = 0;
  a.num_pages = 0;
  return da::launch_score_topk(a, stream) == 0 ? DA_OK : DA_ERR_HIP;
}

int quest_append_score_topk(const void* q, const da_kv_cache* kv, void* meta,
                            int32_t meta_max_pages, const int32_t* seqlens, int32_t num_q_heads,
                            int32_t budget_tokens, const void* k_new, const void* v_new,
                            int32_t* page_idx, float* page_scores, void* workspace,
                            size_t workspace_bytes, void* stream) {
  Shape s;
  int st = check_cache(kv, num_q_heads, &s);
  if (st != DA_OK) return st;
  if (!is_pow2_in(s.page_size, 8, 64)) return DA_ERR_UNSUPPORTED;
  if (budget_tokens <= 0 || budget_tokens % s.page_size != 0) return DA_ERR_BUDGET;
  if (meta_max_pages < 1 || meta_max_pages > kMaxMetaPages ||
      (int64_t)meta_max_pages * s.page_size < s.capacity)
    return DA_ERR_SHAPE;
  if (s.batch == 0) return DA_OK;  // nothing to read or write
  if (q == nullptr || meta == nullptr || seqlens == nullptr || k_new == nullptr ||
      v_new == nullptr || kv->k == nullptr || kv->v == nullptr)
    return DA_ERR_NULL;
  if (page_idx == nullptr && page_scores == nullptr) return DA_ERR_NULL;  // nothing to output
  if (!aligned16(q) || !aligned16(meta) || !aligned16(k_new) || !aligned16(v_new) ||
      !aligned16(kv->k) || !aligned16(kv->v))
    return DA_ERR_SHAPE;
  float* scores = page_scores;
  if (scores == nullptr) {
    size_t need = 0;
    da_quest_workspace_size(s.batch, s.hkv, meta_max_pages, &need);
    if (workspace == nullptr) return DA_ERR_NULL;
    if (!aligned16(workspace)) return DA_ERR_SHAPE;
    if (workspace_bytes < need) return DA_ERR_WORKSPACE;
    scores = static_cast<float*>(workspace);
  }
  da::ScoreLaunch a;
  a.q = q;
  a.meta = meta;
  a.seqlens = seqlens;
  a.scores = scores;
  a.page_idx = page_idx;
  a.batch = s.batch;
  a.num_kv_heads = s.hkv;
  a.group = s.group;
  a.head_dim = s.d;
  a.page_shift = log2i(s.page_size);
  a.meta_max_pages = meta_max_pages;
  a.num_sel = budget_tokens / s.page_size;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k = kv->k;
  a.v = kv->v;
  a.page_table = kv->page_table;
  a.capacity = s.capacity;
  a.cache_stride = s.stride;
  a.max_pages = s.max_pages;
  a.num_pages = kv->num_pages;
  return da::launch_score_topk(a, stream) == 0 ? DA_OK : DA_ERR_HIP;
}

int quest_select_sparse_decode_attn(const void* q, const da_kv_cache* kv,
                                    const int32_t* seqlens, const float* page_scores,
                                    int32_t meta_max_pages, int32_t budget_tokens,
                                    int32_t num_q_heads, float scale, int32_t* page_idx,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    int32_t num_splits, void* stream) {
  Shape s;
  int st = check_cache(kv, num_q_heads, &s);
  if (st != DA_OK) return st;
  st = check_budget(s, budget_tokens);
  if (st != DA_OK) return st;
  if (meta_max_pages < 1 || meta_max_pages > kMaxMetaPages ||
      (int64_t)meta_max_pages * s.page_size < s.capacity)
    return DA_ERR_SHAPE;  // every page that can hold a valid token has a score
  if (s.batch > 0 && page_scores == nullptr) return DA_ERR_NULL;
  PageSelect sel;
  sel.scores = page_scores;
  sel.row = meta_max_pages;
  sel.idx_out = page_idx;
  return run_attention(q, kv, seqlens, nullptr, budget_tokens, num_q_heads, 1, scale, nullptr,
                       nullptr, out, workspace, workspace_bytes, num_splits, stream, &sel);
}

int da_check_cache(const da_kv_cache* kv, const int32_t* seqlens, int32_t* report,
                   void* stream) {
  Shape s;
  // the group size does not matter here; pass Hq = Hkv
  const int st = check_cache(kv, kv != nullptr ? kv->num_kv_heads : 1, &s);
  if (st != DA_OK) return st;
  if (s.batch == 0) return DA_OK;  // nothing to check
  if (seqlens == nullptr || report == nullptr) return DA_ERR_NULL;
  da::CheckLaunch a;
  a.seqlens = seqlens;
  a.page_table = kv->page_table;
  a.report = report;
  a.batch = s.batch;
  a.capacity = s.capacity;
  a.page_shift = s.paged ? log2i(s.page_size) : 0;
  a.max_pages = s.max_pages;
  a.num_pages = kv->num_pages;
  return da::launch_check(a, stream) == 0 ? DA_OK : DA_ERR_HIP;
}

int da_read_calibration(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr) return DA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return DA_ERR_SHAPE;
  return da::launch_read_calibration(buf, bytes, sink, stream) == 0 ? DA_OK : DA_ERR_HIP;
}

}  // extern "C"
