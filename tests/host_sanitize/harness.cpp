// Drives every entry point of include/decode_attn.h through its argument
// checks, with the kernel launchers replaced by recording stubs, in a build
// with AddressSanitizer and UndefinedBehaviorSanitizer (see
// tests/test_host_sanitize.py).  Device pointers are fake, aligned and never
// dereferenced: the host layer only checks them for NULL and alignment.
//
// Three parts:
//   1. the documented status code of each rejected argument, entry point by
//      entry point, and the launch a valid call asks for;
//   2. a seeded fuzz of every entry point over extreme and random sizes (the
//      sanitizers report any overflow or out-of-bounds access in the host
//      arithmetic; the harness checks that a call either is rejected or asks
//      for a launch whose grid and workspace fit what was validated);
//   3. workspace sizes of a fixed list of shapes, printed as JSON for the
//      test to compare with the real library.
// Prints "ok" and exits 0 when every check passes.

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>

#include "../../include/decode_attn.h"
#include "stubs.h"

namespace {

int g_failures = 0;

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                        \
    }                                                                      \
  } while (0)

#define EXPECT_STATUS(call, want)                                                       \
  do {                                                                                  \
    const int got_ = (call);                                                            \
    if (got_ != (want)) {                                                               \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
              got_, (int)(want));                                                       \
      ++g_failures;                                                                     \
    }                                                                                   \
  } while (0)

void* fake(uintptr_t i) { return reinterpret_cast<void*>(uintptr_t(1) << 20 | (i << 12)); }
int32_t* fake_i(uintptr_t i) { return static_cast<int32_t*>(fake(i)); }
void* misaligned() { return reinterpret_cast<void*>((uintptr_t(1) << 20) + 8); }
constexpr size_t kBigWs = size_t(1) << 40;

da_kv_cache contiguous(int b = 2, int hkv = 8, int d = 128, int cap = 4096, int s = 16) {
  da_kv_cache kv{};
  kv.k = fake(1);
  kv.v = fake(2);
  kv.page_table = nullptr;
  kv.batch = b;
  kv.num_kv_heads = hkv;
  kv.head_dim = d;
  kv.capacity = cap;
  kv.page_size = s;
  kv.max_pages = 0;
  kv.num_pages = 0;
  return kv;
}

da_kv_cache paged(int b = 2, int hkv = 8, int d = 128, int s = 16, int max_pages = 256,
                  int64_t pool = 1024) {
  da_kv_cache kv = contiguous(b, hkv, d, 0, s);
  kv.page_table = fake_i(3);
  kv.max_pages = max_pages;
  kv.num_pages = pool;
  return kv;
}

// ------------------------------------------------------------ part 1

void status_strings() {
  for (int c = 0; c >= -7; --c) CHECK(strncmp(da_status_string(c), "DA_", 3) == 0);
  CHECK(strcmp(da_status_string(-99), "unknown status") == 0);
  CHECK(strstr(da_status_string(DA_ERR_TOO_LARGE), "DA_ERR_TOO_LARGE") != nullptr);
}

int attn(const da_kv_cache& kv, int hq = 32, const void* q = fake(4), const void* out = fake(5),
         void* ws = fake(6), size_t ws_bytes = kBigWs, const void* kn = nullptr,
         const void* vn = nullptr, int splits = 0, float scale = 0.125f) {
  return gqa_decode_attn(q, &kv, fake_i(7), hq, scale, kn, vn, const_cast<void*>(out), ws,
                         ws_bytes, splits, nullptr);
}

void decode_checks() {
  da_kv_cache kv = contiguous();
  EXPECT_STATUS(attn(kv, 32, nullptr), DA_ERR_NULL);
  EXPECT_STATUS(attn(kv, 32, fake(4), nullptr), DA_ERR_NULL);
  EXPECT_STATUS(attn(kv, 32, fake(4), fake(5), nullptr), DA_ERR_NULL);
  EXPECT_STATUS(attn(kv, 32, fake(4), fake(5), fake(6), kBigWs, fake(8)), DA_ERR_NULL);
  EXPECT_STATUS(attn(kv, 30), DA_ERR_SHAPE);                        // Hq % Hkv
  EXPECT_STATUS(attn(kv, 24), DA_ERR_UNSUPPORTED);                  // G = 3
  EXPECT_STATUS(attn(kv, 128), DA_ERR_UNSUPPORTED);                 // G = 16
  EXPECT_STATUS(attn(kv, 32, misaligned()), DA_ERR_SHAPE);
  EXPECT_STATUS(attn(kv, 32, fake(4), fake(5), misaligned()), DA_ERR_SHAPE);
  EXPECT_STATUS(attn(kv, 32, fake(4), fake(5), fake(6), 16), DA_ERR_WORKSPACE);
  EXPECT_STATUS(attn(kv, 32, fake(4), fake(5), fake(6), kBigWs, nullptr, nullptr, -1),
                DA_ERR_SHAPE);
  EXPECT_STATUS(attn(kv, 32, fake(4), fake(5), fake(6), kBigWs, nullptr, nullptr, 0,
                     __builtin_nanf("")),
                DA_ERR_SHAPE);
  EXPECT_STATUS(gqa_decode_attn(fake(4), nullptr, fake_i(7), 32, 1.0f, nullptr, nullptr,
                                fake(5), fake(6), kBigWs, 0, nullptr),
                DA_ERR_NULL);
  da_kv_cache bad = kv;
  bad.head_dim = 96;
  EXPECT_STATUS(attn(bad), DA_ERR_UNSUPPORTED);
  bad = kv;
  bad.capacity = 0;
  EXPECT_STATUS(attn(bad), DA_ERR_SHAPE);
  bad = kv;
  bad.batch = -1;
  EXPECT_STATUS(attn(bad), DA_ERR_SHAPE);
  bad = kv;
  bad.k = nullptr;
  EXPECT_STATUS(attn(bad), DA_ERR_NULL);
  bad = paged();
  bad.page_size = 12;
  EXPECT_STATUS(attn(bad), DA_ERR_UNSUPPORTED);
  bad = paged();
  bad.num_pages = 0;
  EXPECT_STATUS(attn(bad), DA_ERR_SHAPE);
  // batch 0: nothing to do, even with NULL tensors
  da_kv_cache empty = kv;
  empty.batch = 0;
  empty.k = empty.v = nullptr;
  EXPECT_STATUS(attn(empty, 32, nullptr, nullptr, nullptr, 0), DA_OK);

  // a valid call: the launch it asks for
  const long before = da::g_stub.launches;
  size_t need = 0;
  EXPECT_STATUS(da_workspace_size(&kv, 32, 0, 0, &need), DA_OK);
  EXPECT_STATUS(attn(kv, 32, fake(4), fake(5), fake(6), need), DA_OK);
  CHECK(da::g_stub.launches == before + 1 && da::g_stub.last == da::StubRecord::kAttn);
  const da::AttnLaunch& a = da::g_stub.attn;
  CHECK(a.group == 4 && a.head_dim == 128 && a.capacity == 4096 && a.cache_stride == 4096);
  CHECK(a.tiles_per_split >= 8 && a.max_splits * a.tiles_per_split * 16 >= 4096);
  CHECK(a.page_idx == nullptr && a.sel_scores == nullptr && a.num_sel == 0);
  CHECK(a.scale_log2 > 0.18f && a.scale_log2 < 0.181f);   // 0.125 * log2(e)
  // the workspace: the work counter first, the partials after 256 bytes
  CHECK(a.work_counter == reinterpret_cast<uint32_t*>(fake(6)));
  CHECK(reinterpret_cast<const char*>(a.part_ml) == static_cast<const char*>(fake(6)) + 256);
  EXPECT_STATUS(attn(kv, 32, fake(4), fake(5), fake(6), need - 1), DA_ERR_WORKSPACE);
  // an explicit split count
  EXPECT_STATUS(attn(kv, 32, fake(4), fake(5), fake(6), kBigWs, nullptr, nullptr, 5), DA_OK);
  CHECK(da::g_stub.attn.max_splits == 5);
  // a paged cache
  da_kv_cache pk = paged();
  EXPECT_STATUS(attn(pk), DA_OK);
  CHECK(da::g_stub.attn.page_table != nullptr && da::g_stub.attn.capacity == 256 * 16);
  CHECK(da::g_stub.attn.page_shift == 4 && da::g_stub.attn.max_pages == 256);
}

void noalloc_checks() {
  da_kv_cache kv = contiguous();
  auto call = [&](const da_kv_cache& c, const void* q, const void* out, int hq = 32) {
    return gqa_decode_attn_noalloc(q, &c, fake_i(7), hq, 0.1f, nullptr, nullptr,
                                   const_cast<void*>(out), 0, nullptr);
  };
  EXPECT_STATUS(call(kv, nullptr, fake(5)), DA_ERR_NULL);
  EXPECT_STATUS(call(kv, fake(4), nullptr), DA_ERR_NULL);
  EXPECT_STATUS(call(kv, fake(4), fake(5), 30), DA_ERR_SHAPE);
  EXPECT_STATUS(call(kv, fake(4), fake(5)), DA_OK);
  CHECK(da::g_stub.attn.work_counter == reinterpret_cast<uint32_t*>(uintptr_t(0x7f0000000000ull)));
  CHECK(da::g_stub.attn.part_ml == reinterpret_cast<float*>(uintptr_t(0x7f0000000000ull + 256)));
  da_kv_cache huge = contiguous(64, 8, 128, 1 << 20);
  EXPECT_STATUS(call(huge, fake(4), fake(5)), DA_ERR_TOO_LARGE);
}

void multi_checks() {
  da_kv_cache kv = contiguous();
  auto call = [&](int hq, int q_len, size_t ws = kBigWs) {
    return gqa_decode_attn_multi(fake(4), &kv, fake_i(7), hq, q_len, 0.1f, fake(5), fake(6), ws,
                                 0, nullptr);
  };
  EXPECT_STATUS(call(32, 0), DA_ERR_SHAPE);
  EXPECT_STATUS(call(30, 2), DA_ERR_SHAPE);
  EXPECT_STATUS(call(32, 3), DA_ERR_UNSUPPORTED);   // 12 rows
  EXPECT_STATUS(call(32, 2, 16), DA_ERR_WORKSPACE);
  EXPECT_STATUS(call(8, 8), DA_OK);                  // G = 1, 8 rows
  CHECK(da::g_stub.attn.group == 8 && da::g_stub.attn.q_len == 8);
  EXPECT_STATUS(call(INT32_MAX, INT32_MAX), DA_ERR_SHAPE);
}

void repeat_checks() {
  da_kv_cache kv = contiguous();
  EXPECT_STATUS(gqa_repeat_kv(&kv, 32, fake_i(7), fake(8), fake(9), nullptr), DA_OK);
  CHECK(da::g_stub.last == da::StubRecord::kRepeat && da::g_stub.repeat.group == 4);
  EXPECT_STATUS(gqa_repeat_kv(&kv, 32, nullptr, fake(8), fake(9), nullptr), DA_ERR_NULL);
  EXPECT_STATUS(gqa_repeat_kv(&kv, 32, fake_i(7), nullptr, fake(9), nullptr), DA_ERR_NULL);
  EXPECT_STATUS(gqa_repeat_kv(&kv, 32, fake_i(7), misaligned(), fake(9), nullptr), DA_ERR_SHAPE);
  EXPECT_STATUS(gqa_repeat_kv(&kv, 24, fake_i(7), fake(8), fake(9), nullptr), DA_ERR_UNSUPPORTED);
  EXPECT_STATUS(gqa_repeat_kv(nullptr, 32, fake_i(7), fake(8), fake(9), nullptr), DA_ERR_NULL);
}

void meta_checks() {
  da_kv_cache kv = contiguous();
  auto call = [&](const da_kv_cache& c, int mp, int n_new, const void* kn = nullptr,
                  const void* vn = nullptr, void* meta = fake(10)) {
    return quest_meta_append(&c, meta, mp, fake_i(7), n_new, kn, vn, nullptr);
  };
  EXPECT_STATUS(call(kv, 256, 1), DA_OK);
  CHECK(da::g_stub.last == da::StubRecord::kMeta && da::g_stub.meta.pages_per_seq == 1);
  EXPECT_STATUS(call(kv, 256, 4096), DA_OK);
  CHECK(da::g_stub.meta.pages_per_seq == 256);
  EXPECT_STATUS(call(kv, 255, 1), DA_ERR_SHAPE);          // 255 * 16 < 4096
  EXPECT_STATUS(call(kv, 256, 0), DA_ERR_SHAPE);
  EXPECT_STATUS(call(kv, 256, 2, fake(11), fake(12)), DA_ERR_SHAPE);   // append needs n_new 1
  EXPECT_STATUS(call(kv, 256, 1, fake(11)), DA_ERR_NULL);
  EXPECT_STATUS(call(kv, 256, 1, nullptr, nullptr, nullptr), DA_ERR_NULL);
  da_kv_cache bad = kv;
  bad.page_size = 7;
  EXPECT_STATUS(call(bad, 1024, 1), DA_ERR_UNSUPPORTED);
  EXPECT_STATUS(call(paged(), 256, 1), DA_OK);
}

void score_checks() {
  auto call = [&](int b, int hq, int hkv, int d, int s, int budget, int mp, int32_t* idx,
                  float* scores, void* ws, size_t ws_bytes) {
    return quest_page_score_topk(fake(4), fake(10), mp, fake_i(7), b, hq, hkv, d, s, budget, idx,
                                 scores, ws, ws_bytes, nullptr);
  };
  size_t need = 0;
  EXPECT_STATUS(da_quest_workspace_size(2, 8, 256, &need), DA_OK);
  CHECK(need >= 2 * 8 * 256 * 4);
  EXPECT_STATUS(da_quest_workspace_size(-1, 8, 256, &need), DA_ERR_SHAPE);
  EXPECT_STATUS(da_quest_workspace_size(2, 8, 256, nullptr), DA_ERR_NULL);
  EXPECT_STATUS(call(2, 32, 8, 128, 16, 256, 256, fake_i(13), nullptr, fake(6), need), DA_OK);
  CHECK(da::g_stub.last == da::StubRecord::kScore && da::g_stub.score.num_sel == 16);
  EXPECT_STATUS(call(2, 32, 8, 128, 16, 256, 256, fake_i(13), nullptr, fake(6), need - 1),
                DA_ERR_WORKSPACE);
  EXPECT_STATUS(call(2, 32, 8, 128, 16, 100, 256, fake_i(13), nullptr, fake(6), need),
                DA_ERR_BUDGET);
  EXPECT_STATUS(call(2, 32, 8, 128, 16, 0, 256, fake_i(13), nullptr, fake(6), need),
                DA_ERR_BUDGET);
  EXPECT_STATUS(call(2, 32, 8, 96, 16, 256, 256, fake_i(13), nullptr, fake(6), need),
                DA_ERR_UNSUPPORTED);
  EXPECT_STATUS(call(2, 32, 8, 128, 16, 256, (1 << 28) + 1, fake_i(13), nullptr, fake(6), kBigWs),
                DA_ERR_SHAPE);  // more pages than the kernels' index arithmetic allows
  // above 16384 pages per unit the same call runs the streaming top-K
  EXPECT_STATUS(call(2, 32, 8, 128, 16, 256, 16385, fake_i(13), nullptr, fake(6), kBigWs), DA_OK);
  CHECK(da::g_stub.last == da::StubRecord::kScore && da::g_stub.score.meta_max_pages == 16385);
  EXPECT_STATUS(call(2, 32, 8, 128, 16, 256, 256, nullptr, nullptr, fake(6), need),
                DA_ERR_NULL);   // nothing to output
  EXPECT_STATUS(call(2, 32, 8, 128, 16, 256, 256, nullptr, static_cast<float*>(fake(14)),
                     nullptr, 0),
                DA_OK);         // scores only, into the caller's buffer
  EXPECT_STATUS(call(0, 32, 8, 128, 16, 256, 256, nullptr, nullptr, nullptr, 0), DA_OK);

  da_kv_cache kv = contiguous();
  auto app = [&](const da_kv_cache& c, const void* kn, const void* vn, int budget = 256) {
    return quest_append_score_topk(fake(4), &c, fake(10), 256, fake_i(7), 32, budget, kn, vn,
                                   fake_i(13), nullptr, fake(6), need, nullptr);
  };
  EXPECT_STATUS(app(kv, fake(11), fake(12)), DA_OK);
  CHECK(da::g_stub.score.k_new == fake(11) && da::g_stub.score.capacity == 4096);
  EXPECT_STATUS(app(kv, nullptr, fake(12)), DA_ERR_NULL);
  EXPECT_STATUS(app(kv, fake(11), fake(12), 24), DA_ERR_BUDGET);
  EXPECT_STATUS(app(paged(), fake(11), fake(12)), DA_OK);
  CHECK(da::g_stub.score.page_table != nullptr);
}

void sparse_checks() {
  da_kv_cache kv = contiguous();
  auto sparse = [&](const da_kv_cache& c, const int32_t* idx, int budget, size_t ws = kBigWs) {
    return quest_sparse_decode_attn(fake(4), &c, fake_i(7), idx, budget, 32, 0.1f, fake(5),
                                    fake(6), ws, 0, nullptr);
  };
  EXPECT_STATUS(sparse(kv, fake_i(13), 256), DA_OK);
  CHECK(da::g_stub.attn.num_sel == 16 && da::g_stub.attn.page_idx == fake_i(13));
  EXPECT_STATUS(sparse(kv, nullptr, 256), DA_ERR_NULL);
  EXPECT_STATUS(sparse(kv, fake_i(13), 20), DA_ERR_BUDGET);
  EXPECT_STATUS(sparse(kv, fake_i(13), 256, 16), DA_ERR_WORKSPACE);
  auto select = [&](const da_kv_cache& c, const float* scores, int mp, int budget) {
    return quest_select_sparse_decode_attn(fake(4), &c, fake_i(7), scores, mp, budget, 32, 0.1f,
                                           nullptr, fake(5), fake(6), kBigWs, 0, nullptr);
  };
  EXPECT_STATUS(select(kv, static_cast<float*>(fake(14)), 256, 256), DA_OK);
  CHECK(da::g_stub.attn.sel_scores != nullptr && da::g_stub.attn.sel_row == 256);
  EXPECT_STATUS(select(kv, nullptr, 256, 256), DA_ERR_NULL);
  EXPECT_STATUS(select(kv, static_cast<float*>(fake(14)), 255, 256), DA_ERR_SHAPE);
  // more pages per unit than the attention launch selects itself: the
  // streaming top-K writes the choice to the workspace (no page_idx), then
  // the attention reads it as a given list
  const long before = da::g_stub.launches;
  EXPECT_STATUS(select(contiguous(2, 8, 128, 1 << 20), static_cast<float*>(fake(14)), 1 << 16,
                       256),
                DA_OK);
  CHECK(da::g_stub.launches == before + 2 && da::g_stub.last == da::StubRecord::kAttn);
  CHECK(da::g_stub.topk.meta_max_pages == 1 << 16 && da::g_stub.topk.num_sel == 16);
  CHECK(da::g_stub.topk.scores == static_cast<float*>(fake(14)));
  CHECK(da::g_stub.attn.sel_scores == nullptr && da::g_stub.attn.page_idx != nullptr);
  CHECK(da::g_stub.attn.page_idx == da::g_stub.topk.page_idx);
  {
    // the choice sits after the partials, inside the workspace the size query asks for
    da_kv_cache big = contiguous(2, 8, 128, 1 << 20);
    size_t need = 0;
    EXPECT_STATUS(da_workspace_size(&big, 32, 256, 0, &need), DA_OK);
    const char* ws0 = static_cast<const char*>(fake(6));
    const char* idx = reinterpret_cast<const char*>(da::g_stub.topk.page_idx);
    CHECK(idx >= ws0 + 2 * 8 * da::g_stub.attn.max_splits * 4 * 2 * sizeof(float));
    CHECK(idx + 2 * 8 * 16 * sizeof(int32_t) == ws0 + need);
  }
  // with page_idx the choice goes there
  EXPECT_STATUS(quest_select_sparse_decode_attn(fake(4), &kv, fake_i(7),
                                                static_cast<float*>(fake(14)), 1 << 16, 256, 32,
                                                0.1f, fake_i(15), fake(5), fake(6), kBigWs, 0,
                                                nullptr),
                DA_OK);
  CHECK(da::g_stub.topk.page_idx == fake_i(15) && da::g_stub.attn.page_idx == fake_i(15));
}

void check_checks() {
  da_kv_cache kv = contiguous();
  int32_t* report = fake_i(17);
  EXPECT_STATUS(da_check_cache(&kv, fake_i(7), report, nullptr), DA_OK);
  CHECK(da::g_stub.last == da::StubRecord::kCheck);
  EXPECT_STATUS(da_check_cache(&kv, nullptr, report, nullptr), DA_ERR_NULL);
  EXPECT_STATUS(da_check_cache(&kv, fake_i(7), nullptr, nullptr), DA_ERR_NULL);
  EXPECT_STATUS(da_check_cache(nullptr, fake_i(7), report, nullptr), DA_ERR_NULL);
  da_kv_cache pk = paged();
  EXPECT_STATUS(da_check_cache(&pk, fake_i(7), report, nullptr), DA_OK);
  da_kv_cache bad = paged();
  bad.page_size = 24;
  EXPECT_STATUS(da_check_cache(&bad, fake_i(7), report, nullptr), DA_ERR_UNSUPPORTED);
  da_kv_cache empty = kv;
  empty.batch = 0;
  EXPECT_STATUS(da_check_cache(&empty, nullptr, nullptr, nullptr), DA_OK);
}

void calibration_checks() {
  uint32_t* sink = static_cast<uint32_t*>(fake(15));
  EXPECT_STATUS(da_read_calibration(fake(16), 1 << 20, sink, nullptr), DA_OK);
  EXPECT_STATUS(da_read_calibration(nullptr, 1 << 20, sink, nullptr), DA_ERR_NULL);
  EXPECT_STATUS(da_read_calibration(fake(16), 1000, sink, nullptr), DA_ERR_SHAPE);
  EXPECT_STATUS(da_read_calibration(misaligned(), 1 << 20, sink, nullptr), DA_ERR_SHAPE);
}

// ------------------------------------------------------------ part 2

int pick(std::mt19937_64& rng, const int* v, int n) { return v[rng() % n]; }

void fuzz(uint64_t seed, int rounds) {
  std::mt19937_64 rng(seed);
  static const int kInts[] = {-1, 0, 1, 2, 3, 7, 8, 16, 17, 64, 100, 128, 4096, 65535, 65536,
                              1 << 20, 1 << 26, INT32_MAX / 2, INT32_MAX / 2 + 1, INT32_MAX};
  static const int kHeads[] = {-1, 0, 1, 2, 4, 8, 16, 32, 64, 65535, 65536};
  static const int kDims[] = {0, 64, 96, 128, 256};
  static const int kPages[] = {0, 7, 8, 16, 32, 64, 128};
  const int n_ints = sizeof(kInts) / sizeof(kInts[0]);
  for (int r = 0; r < rounds; ++r) {
    da_kv_cache kv = contiguous(pick(rng, kInts, n_ints), pick(rng, kHeads, 11),
                                pick(rng, kDims, 5), pick(rng, kInts, n_ints),
                                pick(rng, kPages, 7));
    if (rng() % 3 == 0) {
      kv.page_table = fake_i(3);
      kv.max_pages = pick(rng, kInts, n_ints);
      kv.num_pages = (int64_t)pick(rng, kInts, n_ints) * (1 + rng() % 4);
    }
    const int hq = pick(rng, kHeads, 11) * (1 + (int)(rng() % 8));
    const int budget = pick(rng, kInts, n_ints);
    const int mp = pick(rng, kInts, n_ints);
    const int splits = (int)(rng() % 4 == 0 ? pick(rng, kInts, n_ints) : 0);
    size_t need = 0;
    const long before = da::g_stub.launches;
    // a size query that succeeds must admit the call it sizes
    const bool as_sparse = budget > 0 && rng() % 2;
    int st = da_workspace_size(&kv, hq, as_sparse ? budget : 0, splits, &need);
    if (st == DA_OK) {
      if (as_sparse)
        st = quest_sparse_decode_attn(fake(4), &kv, fake_i(7), fake_i(13), budget, hq, 0.1f,
                                      fake(5), fake(6), need, splits, nullptr);
      else
        st = gqa_decode_attn(fake(4), &kv, fake_i(7), hq, 0.1f, nullptr, nullptr, fake(5),
                             fake(6), need, splits, nullptr);
      CHECK(st == DA_OK);
      if (kv.batch > 0) {
        const da::AttnLaunch& a = da::g_stub.attn;
        CHECK((int64_t)a.max_splits * a.batch * a.num_kv_heads <= INT32_MAX);
        CHECK(a.tiles_per_split >= 1 && a.tiles_per_split <= 512 && a.max_splits >= 1);
      }
    }
    (void)gqa_decode_attn_noalloc(fake(4), &kv, fake_i(7), hq, 0.1f, nullptr, nullptr, fake(5),
                                  splits, nullptr);
    (void)gqa_decode_attn_multi(fake(4), &kv, fake_i(7), hq, 1 + (int)(rng() % 9), 0.1f,
                                fake(5), fake(6), kBigWs, splits, nullptr);
    (void)gqa_repeat_kv(&kv, hq, fake_i(7), fake(8), fake(9), nullptr);
    (void)da_check_cache(&kv, fake_i(7), fake_i(17), nullptr);
    (void)quest_meta_append(&kv, fake(10), mp, fake_i(7), pick(rng, kInts, n_ints), nullptr,
                            nullptr, nullptr);
    (void)quest_meta_append(&kv, fake(10), mp, fake_i(7), 1, fake(11), fake(12), nullptr);
    size_t qneed = 0;
    if (da_quest_workspace_size(kv.batch, kv.num_kv_heads, mp, &qneed) == DA_OK)
      (void)quest_page_score_topk(fake(4), fake(10), mp, fake_i(7), kv.batch, hq,
                                  kv.num_kv_heads, kv.head_dim, kv.page_size, budget,
                                  fake_i(13), nullptr, fake(6), qneed, nullptr);
    (void)quest_append_score_topk(fake(4), &kv, fake(10), mp, fake_i(7), hq, budget, fake(11),
                                  fake(12), fake_i(13), nullptr, fake(6), kBigWs, nullptr);
    (void)quest_sparse_decode_attn(fake(4), &kv, fake_i(7), fake_i(13), budget, hq, 0.1f,
                                   fake(5), fake(6), kBigWs, splits, nullptr);
    (void)quest_select_sparse_decode_attn(fake(4), &kv, fake_i(7),
                                          static_cast<float*>(fake(14)), mp, budget, hq, 0.1f,
                                          nullptr, fake(5), fake(6), kBigWs, splits, nullptr);
    CHECK(da::g_stub.launches >= before);
  }
}

// ------------------------------------------------------------ part 3

void print_sizes() {
  printf("{\"attention\": [");
  const int shapes[][6] = {  // batch, hkv, d, capacity, hq, budget
      {1, 8, 64, 4096, 32, 0},     {8, 8, 128, 131072, 32, 0},  {64, 8, 128, 32768, 32, 0},
      {1, 32, 128, 32768, 32, 0},  {8, 8, 128, 131072, 32, 4096}, {1, 32, 128, 32768, 32, 2048},
      {3, 2, 64, 1000, 16, 256},   {2, 4, 128, 6000, 8, 0}};
  bool first = true;
  for (const auto& s : shapes) {
    da_kv_cache kv = contiguous(s[0], s[1], s[2], s[3], 16);
    size_t need = 0;
    const int st = da_workspace_size(&kv, s[4], s[5], 0, &need);
    printf("%s[%d, %d, %d, %d, %d, %d, %d, %zu]", first ? "" : ", ", s[0], s[1], s[2], s[3], s[4],
           s[5], st, need);
    first = false;
  }
  printf("]}\n");
}

}  // namespace

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? atoi(argv[1]) : 20000;
  status_strings();
  decode_checks();
  noalloc_checks();
  multi_checks();
  repeat_checks();
  meta_checks();
  score_checks();
  sparse_checks();
  check_checks();
  calibration_checks();
  fuzz(20261202, rounds);
  print_sizes();
  if (g_failures != 0) {
    fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
