/*
 * Drives libdecode_attn.so through its C ABI from a plain C program (no
 * Python, no torch): HIP runtime calls for memory and streams, the library's
 * entry points for the work.  Test infrastructure: each result is checked
 * against a direct fp64 evaluation on the host, written here from the
 * definitions the entry points document in include/decode_attn.h.
 *
 *   1. gqa_decode_attn with the step's K/V append, on a contiguous cache of
 *      two sequences (one ragged), G = 4: softmax(scale q.k) v over t < L_b,
 *      row L_b - 1 replaced by the appended one; the row is also in the cache.
 *   2. The Quest pipeline on one sequence with a partial last page:
 *      quest_meta_append (bulk) -> per-page min/max, exact;
 *      quest_page_score_topk -> U = sum_g sum_i max(q m, q M) within an fp32
 *      summation bound, and the chosen pages the exact top-K of the returned
 *      scores (ties to the lower page, ascending, -1 padded);
 *      quest_sparse_decode_attn -> attention over the chosen pages' tokens;
 *      quest_select_sparse_decode_attn -> the same choice and the same output
 *      bit for bit.
 *   3. da_check_cache on the clean cache reports nothing.
 *
 * Prints one line per check and exits 0 when all pass, 1 otherwise, 2 when
 * no device is present.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/decode_attn.h"

static int g_failures = 0;

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #call,             \
              hipGetErrorString(e_));                                             \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

#define DA_OK_CALL(call)                                                          \
  do {                                                                            \
    int s_ = (call);                                                              \
    if (s_ != DA_OK) {                                                            \
      fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #call,             \
              da_status_string(s_));                                              \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

static void check(int ok, const char* what, double value, double bound) {
  printf("%-58s %s (%.3g, bound %.3g)\n", what, ok ? "ok" : "FAILED", value, bound);
  if (!ok) ++g_failures;
}

/* ------------------------------------------------------------ fp16 */

/* IEEE binary16 from binary32, round to nearest even (normal and subnormal
 * results; the inputs here are small normal numbers). */
static uint16_t to_half(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const int exp = (int)((x >> 23) & 0xFF);
  uint32_t man = x & 0x7FFFFFu;
  if (exp == 0xFF) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
  const int e = exp - 127 + 15;
  if (e >= 31) return (uint16_t)(sign | 0x7C00u);
  if (e <= 0) {
    if (e < -10) return (uint16_t)sign;
    man |= 0x800000u;
    const int shift = 14 - e;
    uint32_t h = man >> shift;
    const uint32_t rem = man & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (h & 1u))) ++h;
    return (uint16_t)(sign | h);
  }
  uint32_t h = ((uint32_t)e << 10) | (man >> 13);
  const uint32_t rem = man & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;  /* a carry raises the exponent */
  return (uint16_t)(sign | h);
}

static double from_half(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int exp = (h >> 10) & 0x1F;
  const int man = h & 0x3FF;
  double v;
  if (exp == 0) {
    v = ldexp((double)man, -24);
  } else if (exp == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexp((double)(man | 0x400), exp - 25);
  }
  return sign ? -v : v;
}

/* ------------------------------------------------------------ inputs */

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;

static double uniform01(void) {  /* xorshift64*, 53-bit mantissa in (0, 1) */
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  const uint64_t r = g_rng * 0x2545F4914F6CDD1Dull;
  return ((double)(r >> 11) + 0.5) / 9007199254740992.0;
}

static float normal01(void) {  /* Box-Muller */
  const double u = uniform01(), v = uniform01();
  return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}

static uint16_t* random_half(size_t n) {
  uint16_t* p = (uint16_t*)malloc(n * sizeof(uint16_t));
  for (size_t i = 0; i < n; ++i) p[i] = to_half(normal01());
  return p;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes));
  HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

/* ------------------------------------------------------------ references */

/* Attention of query row qrow over the keys t of one (b, kv) row for which
 * use(t) holds, K/V rows given by key(t) / val(t) (fp16), in fp64. */
typedef const uint16_t* (*RowFn)(const void* ctx, int t);
typedef int (*UseFn)(const void* ctx, int t);

static void attend_ref(const uint16_t* qrow, int d, int n, RowFn key, RowFn val, UseFn use,
                       const void* ctx, double scale, double* out) {
  double m = -INFINITY, l = 0.0;
  double* s = (double*)malloc((size_t)n * sizeof(double));
  for (int t = 0; t < n; ++t) {
    s[t] = -INFINITY;
    if (!use(ctx, t)) continue;
    const uint16_t* k = key(ctx, t);
    double dot = 0.0;
    for (int i = 0; i < d; ++i) dot += from_half(qrow[i]) * from_half(k[i]);
    s[t] = scale * dot;
    if (s[t] > m) m = s[t];
  }
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  for (int t = 0; t < n; ++t) {
    if (s[t] == -INFINITY) continue;
    const double p = exp(s[t] - m);
    l += p;
    const uint16_t* v = val(ctx, t);
    for (int i = 0; i < d; ++i) out[i] += p * from_half(v[i]);
  }
  for (int i = 0; i < d; ++i) out[i] = l > 0.0 ? out[i] / l : 0.0;
  free(s);
}

typedef struct {
  const uint16_t* k;  /* row 0 of this (b, kv) */
  const uint16_t* v;
  const uint16_t* k_new;  /* replaces row L - 1, or NULL */
  const uint16_t* v_new;
  int d, L;
  const int32_t* pages;  /* chosen pages (-1 padded), or NULL for all */
  int n_pages, page_size;
} RowCtx;

static const uint16_t* row_k(const void* c, int t) {
  const RowCtx* r = (const RowCtx*)c;
  return (r->k_new && t == r->L - 1) ? r->k_new : r->k + (size_t)t * r->d;
}
static const uint16_t* row_v(const void* c, int t) {
  const RowCtx* r = (const RowCtx*)c;
  return (r->v_new && t == r->L - 1) ? r->v_new : r->v + (size_t)t * r->d;
}
static int row_use(const void* c, int t) {
  const RowCtx* r = (const RowCtx*)c;
  if (t >= r->L) return 0;
  if (!r->pages) return 1;
  for (int j = 0; j < r->n_pages; ++j)
    if (r->pages[j] == t / r->page_size) return 1;
  return 0;
}

/* ------------------------------------------------------------ 1. dense */

static void dense_with_append(hipStream_t stream) {
  enum { B = 2, HQ = 8, HKV = 2, G = 4, D = 64, CAP = 320 };
  const int32_t lens[B] = {CAP, 77};
  const double scale = 1.0 / sqrt((double)D);
  uint16_t* q = random_half((size_t)B * HQ * D);
  uint16_t* k = random_half((size_t)B * HKV * CAP * D);
  uint16_t* v = random_half((size_t)B * HKV * CAP * D);
  uint16_t* k_new = random_half((size_t)B * HKV * D);
  uint16_t* v_new = random_half((size_t)B * HKV * D);
  void* dq = to_device(q, (size_t)B * HQ * D * 2);
  void* dk = to_device(k, (size_t)B * HKV * CAP * D * 2);
  void* dv = to_device(v, (size_t)B * HKV * CAP * D * 2);
  void* dkn = to_device(k_new, (size_t)B * HKV * D * 2);
  void* dvn = to_device(v_new, (size_t)B * HKV * D * 2);
  void* dl = to_device(lens, sizeof(lens));
  void* dout = NULL;
  HIP_OK(hipMalloc(&dout, (size_t)B * HQ * D * 2));

  da_kv_cache kv;
  memset(&kv, 0, sizeof(kv));
  kv.k = dk;
  kv.v = dv;
  kv.batch = B;
  kv.num_kv_heads = HKV;
  kv.head_dim = D;
  kv.capacity = CAP;
  kv.page_size = 16;
  size_t ws_bytes = 0;
  DA_OK_CALL(da_workspace_size(&kv, HQ, 0, 0, &ws_bytes));
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  DA_OK_CALL(gqa_decode_attn(dq, &kv, (const int32_t*)dl, HQ, (float)scale, dkn, dvn, dout, ws,
                             ws_bytes, 0, stream));
  HIP_OK(hipStreamSynchronize(stream));

  uint16_t* out = (uint16_t*)malloc((size_t)B * HQ * D * 2);
  HIP_OK(hipMemcpy(out, dout, (size_t)B * HQ * D * 2, hipMemcpyDeviceToHost));
  double err = 0.0, ref[D];
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < HQ; ++h) {
      const int kvh = h / G;  /* head h reads KV head h / G */
      const size_t row = ((size_t)b * HKV + kvh) * CAP * D;
      RowCtx c = {k + row, v + row, k_new + ((size_t)b * HKV + kvh) * D,
                  v_new + ((size_t)b * HKV + kvh) * D, D, lens[b], NULL, 0, 16};
      attend_ref(q + ((size_t)b * HQ + h) * D, D, CAP, row_k, row_v, row_use, &c, scale, ref);
      for (int i = 0; i < D; ++i) {
        const double e = fabs(from_half(out[((size_t)b * HQ + h) * D + i]) - ref[i]);
        if (e > err || e != e) err = e;
      }
    }
  check(err <= 2e-3, "gqa_decode_attn with append: max |out - fp64|", err, 2e-3);

  /* the appended rows are in the cache */
  uint16_t* kc = (uint16_t*)malloc((size_t)B * HKV * CAP * D * 2);
  HIP_OK(hipMemcpy(kc, dk, (size_t)B * HKV * CAP * D * 2, hipMemcpyDeviceToHost));
  int stored = 1;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < HKV; ++h)
      if (memcmp(kc + (((size_t)b * HKV + h) * CAP + lens[b] - 1) * D,
                 k_new + ((size_t)b * HKV + h) * D, D * 2) != 0)
        stored = 0;
  check(stored, "gqa_decode_attn with append: k_new stored at L - 1", stored, 1);

  free(q); free(k); free(v); free(k_new); free(v_new); free(out); free(kc);
  HIP_OK(hipFree(dq)); HIP_OK(hipFree(dk)); HIP_OK(hipFree(dv)); HIP_OK(hipFree(dkn));
  HIP_OK(hipFree(dvn)); HIP_OK(hipFree(dl)); HIP_OK(hipFree(dout)); HIP_OK(hipFree(ws));
}

/* ------------------------------------------------------------ 2. Quest */

static void quest_pipeline(hipStream_t stream) {
  enum { B = 1, HQ = 8, HKV = 2, G = 4, D = 128, S = 16, P = 64, CAP = P * S, KSEL = 8 };
  const int32_t lens[B] = {1000};  /* 63 pages, the last one partial */
  const int n_pages = (lens[0] + S - 1) / S;
  const double scale = 1.0 / sqrt((double)D);
  uint16_t* q = random_half((size_t)B * HQ * D);
  uint16_t* k = random_half((size_t)B * HKV * CAP * D);
  uint16_t* v = random_half((size_t)B * HKV * CAP * D);
  void* dq = to_device(q, (size_t)B * HQ * D * 2);
  void* dk = to_device(k, (size_t)B * HKV * CAP * D * 2);
  void* dv = to_device(v, (size_t)B * HKV * CAP * D * 2);
  void* dl = to_device(lens, sizeof(lens));
  void *dmeta = NULL, *dscores = NULL, *didx = NULL, *didx2 = NULL, *dout = NULL, *dout2 = NULL;
  HIP_OK(hipMalloc(&dmeta, (size_t)B * HKV * P * 2 * D * 2));
  HIP_OK(hipMalloc(&dscores, (size_t)B * HKV * P * 4));
  HIP_OK(hipMalloc(&didx, (size_t)B * HKV * KSEL * 4));
  HIP_OK(hipMalloc(&didx2, (size_t)B * HKV * KSEL * 4));
  HIP_OK(hipMalloc(&dout, (size_t)B * HQ * D * 2));
  HIP_OK(hipMalloc(&dout2, (size_t)B * HQ * D * 2));

  da_kv_cache kv;
  memset(&kv, 0, sizeof(kv));
  kv.k = dk;
  kv.v = dv;
  kv.batch = B;
  kv.num_kv_heads = HKV;
  kv.head_dim = D;
  kv.capacity = CAP;
  kv.page_size = S;
  DA_OK_CALL(quest_meta_append(&kv, dmeta, P, (const int32_t*)dl, CAP, NULL, NULL, stream));
  DA_OK_CALL(quest_page_score_topk(dq, dmeta, P, (const int32_t*)dl, B, HQ, HKV, D, S, KSEL * S,
                                   (int32_t*)didx, (float*)dscores, NULL, 0, stream));
  size_t ws_bytes = 0;
  DA_OK_CALL(da_workspace_size(&kv, HQ, KSEL * S, 0, &ws_bytes));
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  DA_OK_CALL(quest_sparse_decode_attn(dq, &kv, (const int32_t*)dl, (const int32_t*)didx,
                                      KSEL * S, HQ, (float)scale, dout, ws, ws_bytes, 0, stream));
  DA_OK_CALL(quest_select_sparse_decode_attn(dq, &kv, (const int32_t*)dl, (const float*)dscores,
                                             P, KSEL * S, HQ, (float)scale, (int32_t*)didx2,
                                             dout2, ws, ws_bytes, 0, stream));
  HIP_OK(hipStreamSynchronize(stream));

  uint16_t* meta = (uint16_t*)malloc((size_t)B * HKV * P * 2 * D * 2);
  float* scores = (float*)malloc((size_t)B * HKV * P * 4);
  int32_t* idx = (int32_t*)malloc((size_t)B * HKV * KSEL * 4);
  int32_t* idx2 = (int32_t*)malloc((size_t)B * HKV * KSEL * 4);
  uint16_t* out = (uint16_t*)malloc((size_t)B * HQ * D * 2);
  uint16_t* out2 = (uint16_t*)malloc((size_t)B * HQ * D * 2);
  HIP_OK(hipMemcpy(meta, dmeta, (size_t)B * HKV * P * 2 * D * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(scores, dscores, (size_t)B * HKV * P * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(idx, didx, (size_t)B * HKV * KSEL * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(idx2, didx2, (size_t)B * HKV * KSEL * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out, dout, (size_t)B * HQ * D * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out2, dout2, (size_t)B * HQ * D * 2, hipMemcpyDeviceToHost));

  /* metadata: min / max over the page's valid keys, exact */
  int meta_ok = 1;
  for (int h = 0; h < HKV; ++h)
    for (int p = 0; p < n_pages; ++p)
      for (int i = 0; i < D; ++i) {
        double mn = INFINITY, mx = -INFINITY;
        for (int t = p * S; t < (p + 1) * S && t < lens[0]; ++t) {
          const double x = from_half(k[((size_t)h * CAP + t) * D + i]);
          if (x < mn) mn = x;
          if (x > mx) mx = x;
        }
        const size_t base = (((size_t)h * P + p) * 2) * D;
        if (from_half(meta[base + i]) != mn || from_half(meta[base + D + i]) != mx) meta_ok = 0;
      }
  check(meta_ok, "quest_meta_append: page min/max exact", meta_ok, 1);

  /* scores: U = sum over the group's heads and channels of max(q m, q M) */
  double score_excess = 0.0;
  for (int h = 0; h < HKV; ++h)
    for (int p = 0; p < n_pages; ++p) {
      double u = 0.0, mag = 0.0;
      const size_t base = (((size_t)h * P + p) * 2) * D;
      for (int g = 0; g < G; ++g)
        for (int i = 0; i < D; ++i) {
          const double qi = from_half(q[((size_t)h * G + g) * D + i]);
          const double a = qi * from_half(meta[base + i]), c = qi * from_half(meta[base + D + i]);
          u += a > c ? a : c;
          mag += fabs(a) + fabs(c);
        }
      /* fp32 accumulation of 2 * G * D terms: a loose first-order bound */
      const double bound = 2.0 * G * D * 6e-8 * mag + 1e-6;
      const double e = fabs((double)scores[h * P + p] - u) / bound;
      if (e > score_excess || e != e) score_excess = e;
    }
  check(score_excess <= 1.0, "quest_page_score_topk: |U - fp64| / fp32 bound", score_excess, 1.0);

  /* the choice: the exact top-K of the returned scores, ascending */
  int choice_ok = 1;
  for (int h = 0; h < HKV; ++h) {
    int chosen[P];
    memset(chosen, 0, sizeof(chosen));
    for (int r = 0; r < KSEL; ++r) {  /* K times: the best page not taken yet */
      int best = -1;
      for (int p = 0; p < n_pages; ++p) {
        if (chosen[p]) continue;
        if (best < 0 || scores[h * P + p] > scores[h * P + best]) best = p;
      }
      chosen[best] = 1;
    }
    int j = 0;
    for (int p = 0; p < n_pages && j < KSEL; ++p)
      if (chosen[p]) {
        if (idx[h * KSEL + j] != p) choice_ok = 0;
        ++j;
      }
  }
  check(choice_ok, "quest_page_score_topk: exact top-K of its scores", choice_ok, 1);

  /* attention over the chosen pages */
  double err = 0.0, ref[D];
  for (int h = 0; h < HQ; ++h) {
    const int kvh = h / G;
    const size_t row = (size_t)kvh * CAP * D;
    RowCtx c = {k + row, v + row, NULL, NULL, D, lens[0], idx + kvh * KSEL, KSEL, S};
    attend_ref(q + (size_t)h * D, D, CAP, row_k, row_v, row_use, &c, scale, ref);
    for (int i = 0; i < D; ++i) {
      const double e = fabs(from_half(out[(size_t)h * D + i]) - ref[i]);
      if (e > err || e != e) err = e;
    }
  }
  check(err <= 2e-3, "quest_sparse_decode_attn: max |out - fp64|", err, 2e-3);

  const int same_idx = memcmp(idx, idx2, (size_t)B * HKV * KSEL * 4) == 0;
  const int same_out = memcmp(out, out2, (size_t)B * HQ * D * 2) == 0;
  check(same_idx && same_out, "quest_select_sparse_decode_attn: same choice and output",
        same_idx && same_out, 1);

  /* 3. the input check on the clean cache */
  void* drep = NULL;
  HIP_OK(hipMalloc(&drep, 16));
  DA_OK_CALL(da_check_cache(&kv, (const int32_t*)dl, (int32_t*)drep, stream));
  int32_t rep[4];
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(rep, drep, 16, hipMemcpyDeviceToHost));
  const int clean = rep[0] == 0 && rep[1] == 0 && rep[2] == -1;
  check(clean, "da_check_cache: nothing to report", clean, 1);

  free(q); free(k); free(v); free(meta); free(scores); free(idx); free(idx2); free(out);
  free(out2);
  HIP_OK(hipFree(dq)); HIP_OK(hipFree(dk)); HIP_OK(hipFree(dv)); HIP_OK(hipFree(dl));
  HIP_OK(hipFree(dmeta)); HIP_OK(hipFree(dscores)); HIP_OK(hipFree(didx));
  HIP_OK(hipFree(didx2)); HIP_OK(hipFree(dout)); HIP_OK(hipFree(dout2)); HIP_OK(hipFree(ws));
  HIP_OK(hipFree(drep));
}

int main(void) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
    fprintf(stderr, "no HIP device\n");
    return 2;
  }
  HIP_OK(hipSetDevice(0));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  dense_with_append(stream);
  quest_pipeline(stream);
  HIP_OK(hipStreamDestroy(stream));
  printf("%s\n", g_failures == 0 ? "c abi checks passed" : "c abi checks FAILED");
  return g_failures == 0 ? 0 : 1;
}
