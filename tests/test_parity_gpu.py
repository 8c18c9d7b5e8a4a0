"""GPU parity: the HIP path, called through the C ABI binding, against the
fp64 CPU oracle on the same seeded fp16 inputs.

Bars (stated here and in the design notes):
* attention outputs: max |gpu - oracle| <= 2e-3 (fp16 inputs, fp32
  accumulation, fp16 output);
* metadata: bit-exact (min/max of fp16 values);
* page scores: |gpu - oracle| <= 2e-6 * sum_i |w_i| |extreme_i| (a bound on
  fp32 accumulation of 2D products with at most ~25 roundings each);
* chosen pages: identical, except that a page may be swapped for another
  when both oracle scores lie within 1e-5 relative of the oracle's K-th
  score; the GPU choice must also be an exact top-K of its own fp32 scores.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import quest as oquest
from decode_attention_folded_amd import workloads

pytestmark = pytest.mark.gpu

ATOL = 2e-3
DEV = "cuda:0"


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


@pytest.fixture(scope="module")
def da():
    import decode_attention_folded_amd as pkg
    pkg.load_library()
    return pkg


def run_dense(da, case, num_splits=0, with_new=False):
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    kn = vn = None
    if with_new:
        kn, vn = dev(case.k_new), dev(case.v_new)
    pt = dev(case.page_table) if case.page_table is not None else None
    out = da.gqa_decode_attn(q, k, v, dev(case.seqlens), k_new=kn, v_new=vn, page_table=pt,
                             page_size=case.page_size, num_splits=num_splits)
    torch.cuda.synchronize()
    return host(out).astype(np.float64), k, v


def max_err(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


# ------------------------------------------------------------ dense attention

DENSE_SHAPES = [
    # (D, G, Hkv, cap, lengths)
    (64, 4, 8, 1100, [1100, 517, 1]),
    (64, 1, 4, 700, [700, 16, 17]),
    (64, 2, 2, 400, [15, 400, 399]),
    (64, 8, 2, 600, [600, 333]),
    (128, 4, 8, 1100, [1100, 517, 1]),
    (128, 1, 4, 700, [700, 16, 17]),
    (128, 2, 2, 400, [15, 400, 399]),
    (128, 8, 2, 600, [600, 333, 8, 9]),
]


@pytest.mark.parametrize("d,g,hkv,cap,lens", DENSE_SHAPES)
def test_dense_parity(da, d, g, hkv, cap, lens):
    case = workloads.dense_case(100 + d + g, len(lens), hkv * g, hkv, d, cap, lens)
    got, _, _ = run_dense(da, case)
    want = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    assert np.all(np.isfinite(got))
    assert max_err(got, want) <= ATOL


@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_dense_split_counts(da, splits):
    case = workloads.dense_case(7, 2, 32, 8, 128, 2000, [2000, 1234])
    got, _, _ = run_dense(da, case, num_splits=splits)
    want = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    assert max_err(got, want) <= ATOL


@pytest.mark.parametrize("d,g,splits", [(64, 1, 100), (64, 8, 40), (128, 8, 50), (128, 2, 33)])
def test_merge_many_splits(da, d, g, splits):
    """Split counts above one merge batch (32, 16 or 8 partials per load
    batch depending on G * D), with one sequence too short to fill them."""
    case = workloads.dense_case(9 + g, 3, 2 * g, 2, d, 1600, [1600, 1111, 20])
    got, _, _ = run_dense(da, case, num_splits=splits)
    want = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    assert max_err(got, want) <= ATOL


def test_dense_bitwise_deterministic(da):
    case = workloads.dense_case(8, 2, 32, 8, 128, 3000, [3000, 2047])
    a, _, _ = run_dense(da, case)
    b, _, _ = run_dense(da, case)
    assert np.array_equal(a, b)


def test_dense_append(da):
    """Fused append: the new row lands at slot L_b - 1, attention includes it."""
    lens = [1000, 17, 1]
    case = workloads.dense_case(9, 3, 32, 8, 64, 1024, lens, with_new=True)
    got, k_dev, v_dev = run_dense(da, case, with_new=True)
    k2, v2 = oracle.append_kv(case.k, case.v, case.seqlens, case.k_new, case.v_new)
    want = oracle.decode_attention(case.q, k2, v2, case.seqlens, case.scale)
    assert max_err(got, want) <= ATOL
    kh, vh = host(k_dev), host(v_dev)
    for b, lb in enumerate(lens):
        assert np.array_equal(kh[b, :, lb - 1], case.k_new[b])
        assert np.array_equal(vh[b, :, lb - 1], case.v_new[b])
        assert np.array_equal(kh[b, :, :lb - 1], case.k[b, :, :lb - 1])


@pytest.mark.parametrize("with_new", [True, False])
@pytest.mark.parametrize("num_splits", [32, 11, 10])
def test_chunk_edges_and_the_appended_slot(da, with_new, num_splits):
    """Chunks of 8 and 24 tiles (the draining ring for short chunks) and of 26
    (the plain ring), with sequences whose appended slot L - 1 is exactly the
    first key of a chunk (L = 1, 129, 257 with 128-key chunks) or inside one.
    Masked keys and the ring's loads past a chunk read the chunk's first row,
    except where that row is the slot being written; the slot L - 1 is
    poisoned with NaN before the append, so reading it there would show."""
    lens = [4096, 3000, 257, 129, 200, 1]
    case = workloads.dense_case(990 + num_splits, len(lens), 16, 4, 64, 4096, lens,
                                with_new=with_new)
    if with_new:
        for b, lb in enumerate(lens):
            case.k[b, :, lb - 1] = np.nan
            case.v[b, :, lb - 1] = np.nan
    got, _, _ = run_dense(da, case, num_splits=num_splits, with_new=with_new)
    if with_new:
        k2, v2 = oracle.append_kv(case.k, case.v, case.seqlens, case.k_new, case.v_new)
    else:
        k2, v2 = case.k, case.v
    want = oracle.decode_attention(case.q, k2, v2, case.seqlens, case.scale)
    assert np.all(np.isfinite(got))
    assert max_err(got, want) <= ATOL


@pytest.mark.parametrize("num_splits", [1, 2, 3])
def test_chunks_at_the_contiguous_cap(da, num_splits):
    """Contiguous-cache chunks of the full 512-tile cap (8192 keys; one or two
    requested splits of 16384 keys give two such chunks) and of 342 tiles,
    with a ragged last chunk, an appended slot that is the first key of the
    second chunk (L = 8193) or inside a chunk, and a one-key sequence."""
    lens = [16384, 8193, 12000, 513, 1]
    case = workloads.dense_case(980 + num_splits, len(lens), 8, 2, 128, 16384, lens,
                                with_new=True)
    for b, lb in enumerate(lens):
        case.k[b, :, lb - 1] = np.nan
        case.v[b, :, lb - 1] = np.nan
    got, _, _ = run_dense(da, case, num_splits=num_splits, with_new=True)
    k2, v2 = oracle.append_kv(case.k, case.v, case.seqlens, case.k_new, case.v_new)
    want = oracle.decode_attention(case.q, k2, v2, case.seqlens, case.scale)
    assert np.all(np.isfinite(got))
    assert max_err(got, want) <= ATOL


def test_dense_empty_and_zero_batch(da):
    case = workloads.dense_case(10, 3, 8, 2, 64, 64, [0, 5, 0])
    got, _, _ = run_dense(da, case)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    want = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    assert max_err(got, want) <= ATOL
    q = torch.zeros((0, 8, 64), dtype=torch.float16, device=DEV)
    k = torch.zeros((0, 2, 64, 64), dtype=torch.float16, device=DEV)
    out = da.gqa_decode_attn(q, k, k, torch.zeros(0, dtype=torch.int32, device=DEV))
    assert out.shape == (0, 8, 64)


def test_dense_single_key_is_exact(da):
    case = workloads.dense_case(11, 2, 32, 8, 128, 64, [1, 1])
    got, _, _ = run_dense(da, case)
    for h in range(32):
        assert np.array_equal(got[:, h], case.v[:, h // 4, 0].astype(np.float64))


def test_fold_equals_materialised_repeat_kv(da):
    """The fold on [B, Hkv, G, D] against the same library at G = 1 on an
    explicitly repeated cache (the page's repeat_kv form)."""
    case = workloads.dense_case(12, 2, 32, 8, 128, 900, [900, 300])
    got, _, _ = run_dense(da, case)
    rep = workloads.Case(q=case.q, k=np.repeat(case.k, 4, axis=1), v=np.repeat(case.v, 4, axis=1),
                         seqlens=case.seqlens, num_kv_heads=32, head_dim=128, capacity=900)
    got_rep, _, _ = run_dense(da, rep)
    assert max_err(got, got_rep) <= ATOL


@pytest.mark.parametrize("page_size", [8, 16, 32, 64])
@pytest.mark.parametrize("d,g", [(128, 4), (64, 4), (128, 8), (64, 1)])
def test_paged_parity(da, page_size, d, g):
    hkv, max_pages = 4, (1500 + page_size - 1) // page_size
    lens = [1500, 37, 1, page_size * 3]
    case = workloads.paged_case(200 + page_size + d + g, len(lens), hkv * g, hkv, d, page_size,
                                max_pages, lens, spare_pages=3)
    got, _, _ = run_dense(da, case)
    kc = oracle.gather_paged(case.k, case.page_table, page_size, case.capacity)
    vc = oracle.gather_paged(case.v, case.page_table, page_size, case.capacity)
    want = oracle.decode_attention(case.q, kc, vc, case.seqlens, case.scale)
    assert np.all(np.isfinite(got))
    assert max_err(got, want) <= ATOL


@pytest.mark.parametrize("page_size", [8, 16])
def test_paged_append(da, page_size):
    """Fused append on a paged cache: the new row lands in slot (L - 1) mod S
    of the sequence's page (L - 1) / S in the pool (poisoned with NaN before),
    and attention includes it; splits forced so chunks start at page starts."""
    hkv, g, d = 4, 4, 64
    lens = [1500, 129, 17, 1]
    max_pages = (1500 + page_size - 1) // page_size
    case = workloads.paged_case(260 + page_size, len(lens), hkv * g, hkv, d, page_size,
                                max_pages, lens, spare_pages=2)
    rng = np.random.default_rng([260, page_size])
    k_new = rng.standard_normal((len(lens), hkv, d), dtype=np.float32).astype(np.float16)
    v_new = rng.standard_normal((len(lens), hkv, d), dtype=np.float32).astype(np.float16)
    k_pool, v_pool = case.k.copy(), case.v.copy()
    for b, lb in enumerate(lens):
        phys = case.page_table[b, (lb - 1) // page_size]
        k_pool[phys, :, (lb - 1) % page_size] = np.nan
        v_pool[phys, :, (lb - 1) % page_size] = np.nan
    k_dev, v_dev = dev(k_pool), dev(v_pool)
    for splits in (0, 16):
        out = da.gqa_decode_attn(dev(case.q), k_dev, v_dev, dev(case.seqlens), k_new=dev(k_new),
                                 v_new=dev(v_new), page_table=dev(case.page_table),
                                 page_size=page_size, num_splits=splits)
        torch.cuda.synchronize()
        kc = oracle.gather_paged(case.k, case.page_table, page_size, case.capacity)
        vc = oracle.gather_paged(case.v, case.page_table, page_size, case.capacity)
        k2, v2 = oracle.append_kv(kc, vc, case.seqlens, k_new, v_new)
        want = oracle.decode_attention(case.q, k2, v2, case.seqlens, case.scale)
        got = host(out).astype(np.float64)
        assert np.all(np.isfinite(got)), splits
        assert max_err(got, want) <= ATOL, splits
    kh, vh = host(k_dev), host(v_dev)
    for b, lb in enumerate(lens):
        phys = case.page_table[b, (lb - 1) // page_size]
        assert np.array_equal(kh[phys, :, (lb - 1) % page_size], k_new[b])
        assert np.array_equal(vh[phys, :, (lb - 1) % page_size], v_new[b])


# ------------------------------------------------------------ quest metadata


def run_meta_bulk(da, case, page_size, max_pages):
    meta = torch.zeros((case.batch, case.num_kv_heads, max_pages, 2, case.head_dim),
                       dtype=torch.float16, device=DEV)
    k, v = dev(case.k), dev(case.v)
    pt = dev(case.page_table) if case.page_table is not None else None
    da.quest_meta_append(k, v, meta, dev(case.seqlens), n_new=case.capacity,
                         page_size=page_size, page_table=pt)
    torch.cuda.synchronize()
    return meta


@pytest.mark.parametrize("page_size", [8, 16, 64])
@pytest.mark.parametrize("d", [64, 128])
def test_metadata_bulk_bit_exact(da, page_size, d):
    lens = [1000, 33, 1, 64]
    cap = 1024
    case = workloads.dense_case(300 + page_size, len(lens), 8, 2, d, cap, lens)
    max_pages = cap // page_size
    meta = host(run_meta_bulk(da, case, page_size, max_pages))
    want = oquest.build_metadata(case.k, case.seqlens, page_size, max_pages)
    for b, lb in enumerate(lens):
        n = oquest.page_count(lb, page_size)
        assert np.array_equal(meta[b, :, :n], want[b, :, :n])


def test_metadata_step_append_matches_bulk(da):
    """Token-by-token append with the fused cache write equals the bulk build,
    bit for bit, and writes the rows into the cache."""
    page_size, cap, d = 16, 80, 128
    case = workloads.dense_case(310, 2, 8, 2, d, cap, [cap, cap], poison=False)
    k = torch.zeros_like(dev(case.k))
    v = torch.zeros_like(dev(case.v))
    meta = torch.zeros((2, 2, cap // page_size, 2, d), dtype=torch.float16, device=DEV)
    for step in range(1, 71):
        lens = dev(np.array([step, max(1, step - 5)], np.int32))
        kn = dev(np.stack([case.k[0, :, step - 1], case.k[1, :, max(1, step - 5) - 1]]))
        vn = dev(np.stack([case.v[0, :, step - 1], case.v[1, :, max(1, step - 5) - 1]]))
        da.quest_meta_append(k, v, meta, lens, 1, page_size=page_size, k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    final = np.array([70, 65], np.int32)
    want = oquest.build_metadata(case.k, final, page_size, cap // page_size)
    got = host(meta)
    for b in range(2):
        n = oquest.page_count(final[b], page_size)
        assert np.array_equal(got[b, :, :n], want[b, :, :n])
        assert np.array_equal(host(k)[b, :, :final[b]], case.k[b, :, :final[b]])
        assert np.array_equal(host(v)[b, :, :final[b]], case.v[b, :, :final[b]])


def test_metadata_paged(da):
    page_size, d = 16, 128
    lens = [500, 16, 3]
    case = workloads.paged_case(320, 3, 8, 2, d, page_size, 40, lens)
    meta = host(run_meta_bulk(da, case, page_size, 40))
    kc = oracle.gather_paged(case.k, case.page_table, page_size, case.capacity)
    want = oquest.build_metadata(kc, case.seqlens, page_size, 40)
    for b, lb in enumerate(lens):
        n = oquest.page_count(lb, page_size)
        assert np.array_equal(meta[b, :, :n], want[b, :, :n])


# ------------------------------------------------------------ scores and top-K


def check_selection(gpu_idx, gpu_scores, want_idx, want_scores, seqlens, page_size, k_pages):
    """Compare chosen pages under the near-tie rule; also check the GPU set is
    an exact top-K (ties to lower index) of its own fp32 scores."""
    bsz, hkv, _ = gpu_idx.shape
    swaps = 0
    for b in range(bsz):
        n = oquest.page_count(seqlens[b], page_size)
        for kv in range(hkv):
            g = [int(p) for p in gpu_idx[b, kv] if p >= 0]
            w = [int(p) for p in want_idx[b, kv] if p >= 0]
            assert g == sorted(g) and len(g) == min(k_pages, n)
            assert list(gpu_idx[b, kv, len(g):]) == [-1] * (k_pages - len(g))
            if g != w:
                ws = want_scores[b, kv, :n]
                kth = np.sort(ws)[::-1][min(k_pages, n) - 1]
                for p in set(g) ^ set(w):
                    assert abs(ws[p] - kth) <= 1e-5 * abs(kth), (b, kv, p, ws[p], kth)
                swaps += len(set(g) ^ set(w)) // 2
            if gpu_scores is not None and n > k_pages:
                s = gpu_scores[b, kv, :n]
                chosen = set(g)
                worst = min((s[p], -p) for p in chosen)
                best_out = max(((s[p], -p) for p in range(n) if p not in chosen))
                assert worst > best_out
    return swaps


def score_tolerance(q, meta, seqlens, page_size):
    """2e-6 * sum_i |w+_i| |M_i| + |w-_i| |m_i| per page."""
    q64 = q.astype(np.float64)
    bsz, hq, d = q64.shape
    hkv = meta.shape[1]
    g = hq // hkv
    tol = np.zeros(meta.shape[:3])
    for b in range(bsz):
        for kv in range(hkv):
            qs = q64[b, kv * g:(kv + 1) * g]
            wpos = np.where(qs >= 0, qs, 0).sum(0)
            wneg = np.where(qs < 0, qs, 0).sum(0)
            mag = (np.abs(meta[b, kv, :, 1].astype(np.float64)) @ np.abs(wpos)
                   + np.abs(meta[b, kv, :, 0].astype(np.float64)) @ np.abs(wneg))
            tol[b, kv] = 2e-6 * mag + 1e-30
    return tol


@pytest.mark.parametrize("page_size,budget,g,d,cap,lens", [
    (16, 256, 4, 128, 4096, [4096, 1000, 200, 17]),
    (16, 64, 1, 128, 2048, [2048, 2047]),
    (8, 64, 2, 64, 1024, [1024, 900]),
    (32, 512, 8, 128, 8192, [8192, 5000]),
    (64, 128, 4, 64, 4096, [4096, 100]),
    (16, 2048, 4, 128, 32768, [32768]),
])
def test_score_topk_parity(da, page_size, budget, g, d, cap, lens):
    hkv = 2
    case = workloads.dense_case(400 + page_size + g, len(lens), hkv * g, hkv, d, cap, lens,
                                plant_pages=4, plant_page_size=page_size)
    max_pages = cap // page_size
    k_pages = budget // page_size
    meta_dev = run_meta_bulk(da, case, page_size, max_pages)
    meta = host(meta_dev)
    scores = torch.full((len(lens), hkv, max_pages), float("nan"), dtype=torch.float32,
                        device=DEV)
    idx = da.quest_page_score_topk(dev(case.q), meta_dev, dev(case.seqlens), page_size=page_size,
                                   budget_tokens=budget, page_scores=scores)
    torch.cuda.synchronize()
    want_meta = oquest.build_metadata(case.k, case.seqlens, page_size, max_pages)
    want_scores = oquest.page_scores(case.q, want_meta, case.seqlens, page_size)
    want_idx = oquest.select_pages(want_scores, case.seqlens, page_size, k_pages)
    got_scores = host(scores).astype(np.float64)
    tol = score_tolerance(case.q, want_meta, case.seqlens, page_size)
    for b, lb in enumerate(lens):
        n = oquest.page_count(lb, page_size)
        assert np.all(np.abs(got_scores[b, :, :n] - want_scores[b, :, :n]) <= tol[b, :, :n])
    check_selection(host(idx), got_scores, want_idx, want_scores, case.seqlens, page_size,
                    k_pages)
    # the same call without a score buffer uses the workspace and agrees
    idx2 = da.quest_page_score_topk(dev(case.q), meta_dev, dev(case.seqlens),
                                    page_size=page_size, budget_tokens=budget)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx2), host(idx))


@pytest.mark.parametrize("n_pages,k_pages,seqlen_pages", [
    (4096, 300, 4096),      # 16 items per thread
    (3001, 64, 2999),       # 16 items per thread, ragged
    (16384, 1000, 16384),   # the maximum: 64 items per thread
    (12000, 5, 11111),      # 64 items per thread, ragged, small K
    (16385, 300, 16385),    # one page past the register-held select: streaming top-K
    (65536, 256, 65536),    # 1M tokens at S = 16
    (40000, 2000, 39001),   # ragged, large K
    (50000, 3, 49999),      # small K
])
def test_topk_large_page_counts(da, n_pages, k_pages, seqlen_pages):
    """Score + top-K on random metadata: every item-per-thread width of the
    register-held select (up to 16384 pages per (b, kv)) and the streaming
    select above it."""
    s, d, g, hkv = 8, 64, 2, 2
    rng = np.random.default_rng(n_pages)
    a = rng.standard_normal((1, hkv, n_pages, d), dtype=np.float32)
    b = rng.standard_normal((1, hkv, n_pages, d), dtype=np.float32)
    meta = np.stack([np.minimum(a, b), np.maximum(a, b)], axis=3).astype(np.float16)
    q = rng.standard_normal((1, hkv * g, d), dtype=np.float32).astype(np.float16)
    seqlens = np.array([seqlen_pages * s - 3], np.int32)
    scores = torch.empty((1, hkv, n_pages), dtype=torch.float32, device=DEV)
    idx = da.quest_page_score_topk(dev(q), dev(meta), dev(seqlens), page_size=s,
                                   budget_tokens=k_pages * s, page_scores=scores)
    torch.cuda.synchronize()
    want_scores = oquest.page_scores(q, meta, seqlens, s)
    want_idx = oquest.select_pages(want_scores, seqlens, s, k_pages)
    got_scores = host(scores).astype(np.float64)
    n = oquest.page_count(seqlens[0], s)
    tol = score_tolerance(q, meta, seqlens, s)
    assert np.all(np.abs(got_scores[0, :, :n] - want_scores[0, :, :n]) <= tol[0, :, :n])
    check_selection(host(idx), got_scores, want_idx, want_scores, seqlens, s, k_pages)


def test_topk_exact_ties_lower_index(da):
    """Pages with identical keys tie exactly in fp32 too; the lower index is
    chosen.  Many ties straddle the K-th position here."""
    page_size, cap, d = 16, 2048, 128
    case = workloads.dense_case(410, 1, 4, 1, d, cap, [cap], poison=False)
    # 40 copies of one page, pushed along the sign of the summed query so they
    # outscore every other page; K = 24 must then split the tied copies
    qsum = case.q[0].astype(np.float32).sum(axis=0)
    hot = (case.k[0, 0, 0:16].astype(np.float32) + 2.0 * np.sign(qsum)).astype(np.float16)
    copies = list(range(3, 128, 3))[:40]
    for p in copies:
        case.k[0, 0, p * 16:(p + 1) * 16] = hot
    meta_dev = run_meta_bulk(da, case, page_size, cap // page_size)
    idx = host(da.quest_page_score_topk(dev(case.q), meta_dev, dev(case.seqlens),
                                        page_size=page_size, budget_tokens=24 * 16))
    want_meta = oquest.build_metadata(case.k, case.seqlens, page_size, cap // page_size)
    want_scores = oquest.page_scores(case.q, want_meta, case.seqlens, page_size)
    want = oquest.select_pages(want_scores, case.seqlens, page_size, 24)
    assert np.array_equal(idx, want)


def test_topk_fewer_pages_than_budget(da):
    case = workloads.dense_case(420, 2, 8, 2, 128, 512, [100, 512])
    meta_dev = run_meta_bulk(da, case, 16, 32)
    idx = host(da.quest_page_score_topk(dev(case.q), meta_dev, dev(case.seqlens), page_size=16,
                                        budget_tokens=64 * 16))
    assert list(idx[0, 0, :7]) == list(range(7)) and np.all(idx[0, :, 7:] == -1)
    assert list(idx[1, 1, :32]) == list(range(32)) and np.all(idx[1, :, 32:] == -1)


# ------------------------------------------------------------ sparse attention


@pytest.mark.parametrize("page_size,budget,g,d,lens", [
    (16, 256, 4, 128, [4096, 1000, 200, 17]),
    (16, 2048, 1, 128, [2048, 2047]),
    (8, 64, 2, 64, [1024, 900]),
    (32, 512, 8, 128, [3000, 64]),
    (64, 128, 4, 64, [4096, 100]),
])
def test_sparse_parity(da, page_size, budget, g, d, lens):
    hkv, cap = 2, max(lens)
    cap = ((cap + 63) // 64) * 64
    case = workloads.dense_case(500 + page_size + g, len(lens), hkv * g, hkv, d, cap, lens,
                                plant_pages=4, plant_page_size=page_size)
    k_pages = budget // page_size
    meta = oquest.build_metadata(case.k, case.seqlens, page_size, cap // page_size)
    idx = oquest.select_pages(oquest.page_scores(case.q, meta, case.seqlens, page_size),
                              case.seqlens, page_size, k_pages)
    out = da.quest_sparse_decode_attn(dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens),
                                      dev(idx), budget_tokens=budget, page_size=page_size)
    torch.cuda.synchronize()
    want = oquest.sparse_decode_attention(case.q, case.k, case.v, case.seqlens, idx, page_size,
                                          case.scale)
    assert max_err(host(out), want) <= ATOL


def test_sparse_all_pages_equals_dense(da):
    lens = [1000, 333]
    case = workloads.dense_case(510, 2, 32, 8, 128, 1024, lens)
    idx = np.full((2, 8, 64), -1, np.int32)
    for b, lb in enumerate(lens):
        idx[b, :, :oquest.page_count(lb, 16)] = np.arange(oquest.page_count(lb, 16))
    sparse = host(da.quest_sparse_decode_attn(dev(case.q), dev(case.k), dev(case.v),
                                              dev(case.seqlens), dev(idx), budget_tokens=1024,
                                              page_size=16)).astype(np.float64)
    dense, _, _ = run_dense(da, case)
    want = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    assert max_err(sparse, want) <= ATOL
    assert max_err(sparse, dense) <= ATOL


def test_sparse_over_paged_cache(da):
    page_size, lens = 16, [1500, 200]
    case = workloads.paged_case(520, 2, 32, 8, 128, page_size, 100, lens)
    kc = oracle.gather_paged(case.k, case.page_table, page_size, case.capacity)
    vc = oracle.gather_paged(case.v, case.page_table, page_size, case.capacity)
    meta = oquest.build_metadata(kc, case.seqlens, page_size, 100)
    idx = oquest.select_pages(oquest.page_scores(case.q, meta, case.seqlens, page_size),
                              case.seqlens, page_size, 16)
    out = da.quest_sparse_decode_attn(dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens),
                                      dev(idx), budget_tokens=256, page_size=page_size,
                                      page_table=dev(case.page_table))
    torch.cuda.synchronize()
    want = oquest.sparse_decode_attention(case.q, kc, vc, case.seqlens, idx, page_size,
                                          case.scale)
    assert max_err(host(out), want) <= ATOL


def test_quest_pipeline_end_to_end(da):
    """Metadata -> score/top-K -> sparse attention, all on the GPU, against
    the oracle running the same steps from the same inputs.  The chosen pages
    must agree under the near-tie rule, and the output must match the oracle's
    attention over the pages the GPU chose (so a legitimate near-tie swap
    still has its output checked)."""
    page_size, budget, lens = 16, 512, [8192, 3000]
    case = workloads.dense_case(530, 2, 32, 8, 128, 8192, lens, plant_pages=8)
    meta_dev = run_meta_bulk(da, case, page_size, 512)
    idx = da.quest_page_score_topk(dev(case.q), meta_dev, dev(case.seqlens), page_size=page_size,
                                   budget_tokens=budget)
    out = da.quest_sparse_decode_attn(dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens),
                                      idx, budget_tokens=budget, page_size=page_size)
    torch.cuda.synchronize()
    meta = oquest.build_metadata(case.k, case.seqlens, page_size, 512)
    scores = oquest.page_scores(case.q, meta, case.seqlens, page_size)
    want_idx = oquest.select_pages(scores, case.seqlens, page_size, budget // page_size)
    check_selection(host(idx), None, want_idx, scores, case.seqlens, page_size,
                    budget // page_size)
    want = oquest.sparse_decode_attention(case.q, case.k, case.v, case.seqlens, host(idx),
                                          page_size, case.scale)
    assert max_err(host(out), want) <= ATOL


# ------------------------------------------------------------ q_len > 1


@pytest.mark.parametrize("d,g,lq,cap,lens,splits", [
    (64, 4, 2, 700, [700, 130, 2, 1], 0),
    (128, 2, 4, 600, [600, 4, 3, 257], 0),
    (128, 1, 8, 500, [500, 8, 5, 33], 0),
    (64, 1, 2, 300, [300, 17], 7),
    (128, 4, 2, 1100, [1100, 999], 1),
    (64, 8, 1, 400, [400, 2], 0),
])
def test_multi_query_parity(da, d, g, lq, cap, lens, splits):
    """G * q_len rows per KV head, causal alignment per row, against the
    oracle; includes sequences shorter than q_len (leading rows see no key)
    and split counts from 1 to several."""
    hkv = 2
    case = workloads.dense_case(950 + g * lq, len(lens), hkv * g, hkv, d, cap, lens)
    rng = np.random.default_rng(951)
    q = rng.standard_normal((len(lens), hkv * g, lq, d), dtype=np.float32).astype(np.float16)
    out = da.gqa_decode_attn_multi(dev(q), dev(case.k), dev(case.v), dev(case.seqlens),
                                   num_splits=splits)
    torch.cuda.synchronize()
    got = host(out).astype(np.float64)
    want = oracle.multi_query_attention(q, case.k, case.v, case.seqlens, case.scale)
    assert np.all(np.isfinite(got))
    assert max_err(got, want) <= ATOL


def test_multi_query_paged_and_q1_equals_decode(da):
    """Paged cache with q_len = 4; and q_len = 1 gives the decode result
    bitwise."""
    case = workloads.paged_case(960, 3, 8, 2, 128, 16, 40, [640, 4, 300])
    rng = np.random.default_rng(961)
    q = rng.standard_normal((3, 8, 2, 128), dtype=np.float32).astype(np.float16)
    out = da.gqa_decode_attn_multi(dev(q), dev(case.k), dev(case.v), dev(case.seqlens),
                                   page_table=dev(case.page_table), page_size=16)
    torch.cuda.synchronize()
    kc = oracle.gather_paged(case.k, case.page_table, 16, 40 * 16)
    vc = oracle.gather_paged(case.v, case.page_table, 16, 40 * 16)
    want = oracle.multi_query_attention(q, kc, vc, case.seqlens, case.scale)
    assert max_err(host(out), want) <= ATOL
    dc = workloads.dense_case(962, 2, 32, 8, 64, 900, [900, 77])
    one = da.gqa_decode_attn_multi(dev(dc.q[:, :, None, :]), dev(dc.k), dev(dc.v),
                                   dev(dc.seqlens))
    dec = da.gqa_decode_attn(dev(dc.q), dev(dc.k), dev(dc.v), dev(dc.seqlens))
    torch.cuda.synchronize()
    assert np.array_equal(host(one)[:, :, 0], host(dec))


# ------------------------------------------------------------ fused append + score


@pytest.mark.parametrize("page_size,d,g,lens,paged", [
    (16, 128, 4, [4096, 1000, 17, 33], False),   # mid-page, start of page (L-1 = 16, 32)
    (8, 64, 2, [1024, 9, 0], False),              # page start (L-1 = 8), empty sequence
    (16, 128, 4, [2000, 1601, 300], True),         # paged cache, L-1 = 1600 starts a page
    (64, 64, 1, [640, 65], False),
])
def test_fused_append_score_matches_two_calls(da, page_size, d, g, lens, paged):
    """quest_append_score_topk equals quest_meta_append (one step) followed by
    quest_page_score_topk: cache, metadata, scores and chosen pages bitwise."""
    hkv, cap = 2, max(lens) + 64
    cap = (cap + page_size - 1) // page_size * page_size
    if paged:
        case = workloads.paged_case(900 + d, len(lens), hkv * g, hkv, d, page_size,
                                    cap // page_size, lens, poison=False, spare_pages=3)
        kw = dict(page_table=dev(case.page_table))
    else:
        case = workloads.dense_case(900 + d, len(lens), hkv * g, hkv, d, cap, lens)
        kw = {}
    rng = np.random.default_rng(901)
    kn = rng.standard_normal((len(lens), hkv, d), dtype=np.float32).astype(np.float16)
    vn = rng.standard_normal((len(lens), hkv, d), dtype=np.float32).astype(np.float16)
    max_pages = cap // page_size
    budget = 4 * page_size
    sl = dev(case.seqlens)
    outs = []
    for fused in (False, True):
        k, v = dev(case.k), dev(case.v)
        meta = torch.zeros((len(lens), hkv, max_pages, 2, d), dtype=torch.float16, device=DEV)
        # metadata of the lengths before the step (the new key not yet in it)
        sl_before = dev(np.maximum(case.seqlens - 1, 0).astype(np.int32))
        da.quest_meta_append(k, v, meta, sl_before, n_new=cap, page_size=page_size, **kw)
        scores = torch.full((len(lens), hkv, max_pages), float("nan"), dtype=torch.float32,
                            device=DEV)
        if fused:
            idx = da.quest_append_score_topk(dev(case.q), k, v, meta, sl, dev(kn), dev(vn),
                                             page_size=page_size, budget_tokens=budget,
                                             page_scores=scores, **kw)
        else:
            da.quest_meta_append(k, v, meta, sl, 1, page_size=page_size, k_new=dev(kn),
                                 v_new=dev(vn), **kw)
            idx = da.quest_page_score_topk(dev(case.q), meta, sl, page_size=page_size,
                                           budget_tokens=budget, page_scores=scores)
        torch.cuda.synchronize()
        outs.append((host(k), host(v), host(meta), host(scores), host(idx)))
    (k0, v0, m0, s0, i0), (k1, v1, m1, s1, i1) = outs
    # slots past L hold NaN poison in both caches
    assert np.array_equal(k0, k1, equal_nan=True) and np.array_equal(v0, v1, equal_nan=True)
    assert np.array_equal(m0, m1, equal_nan=True)
    for b, lb in enumerate(lens):
        n = oquest.page_count(lb, page_size)
        assert np.array_equal(s0[b, :, :n], s1[b, :, :n])
    assert np.array_equal(i0, i1)
    # and against the oracle: the metadata was built over [0, L - 1) before the
    # step, so after it the pages hold the min/max of the final cache's keys
    kc = oracle.gather_paged(k1, case.page_table, page_size, cap) if paged else k1
    want = oquest.build_metadata(kc, case.seqlens, page_size, max_pages)
    for b, lb in enumerate(lens):
        n = oquest.page_count(lb, page_size)
        assert np.array_equal(m1[b, :, :n], want[b, :, :n])


# ------------------------------------------------------------ repeat_kv A/B


@pytest.mark.parametrize("d,g,cap,lens", [(64, 4, 700, [700, 129, 1]), (128, 8, 300, [300, 65]),
                                          (128, 1, 200, [200, 0])])
def test_repeat_kv_copy_and_g1_attention(da, d, g, cap, lens):
    """The materialised copy equals the oracle's repeat_kv on every valid row
    (bit-exact), leaves rows past L_b untouched, and attention on it at G = 1
    matches the oracle and the folded kernel."""
    hkv = 2
    case = workloads.dense_case(810 + g, len(lens), hkv * g, hkv, d, cap, lens)
    k, v, sl = dev(case.k), dev(case.v), dev(case.seqlens)
    sentinel = torch.full((len(lens), hkv * g, cap, d), 7.0, dtype=torch.float16, device=DEV)
    kr, vr = da.gqa_repeat_kv(k, v, sl, hkv * g, k_out=sentinel.clone(), v_out=sentinel.clone())
    torch.cuda.synchronize()
    want_k, want_v = oracle.repeat_kv(case.k, g), oracle.repeat_kv(case.v, g)
    kr_h, vr_h = host(kr), host(vr)
    for b, lb in enumerate(lens):
        assert np.array_equal(kr_h[b, :, :lb], want_k[b, :, :lb])
        assert np.array_equal(vr_h[b, :, :lb], want_v[b, :, :lb])
        assert np.all(kr_h[b, :, lb:] == 7.0) and np.all(vr_h[b, :, lb:] == 7.0)
    out_g1 = host(da.gqa_decode_attn(dev(case.q), kr, vr, sl)).astype(np.float64)
    out_fold = host(da.gqa_decode_attn(dev(case.q), k, v, sl)).astype(np.float64)
    want = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    assert max_err(out_g1, want) <= ATOL
    assert max_err(out_fold, want) <= ATOL


def test_repeat_kv_from_paged_cache(da):
    """A paged pool is materialised into the contiguous [B, Hq, cap, D] layout."""
    case = workloads.paged_case(820, 3, 16, 4, 64, 16, 40, [640, 17, 300])
    k, v = dev(case.k), dev(case.v)
    kr, vr = da.gqa_repeat_kv(k, v, dev(case.seqlens), 16, page_table=dev(case.page_table),
                              page_size=16)
    torch.cuda.synchronize()
    kc = oracle.gather_paged(case.k, case.page_table, 16, 40 * 16)
    vc = oracle.gather_paged(case.v, case.page_table, 16, 40 * 16)
    want_k, want_v = oracle.repeat_kv(kc, 4), oracle.repeat_kv(vc, 4)
    for b, lb in enumerate(case.seqlens):
        assert np.array_equal(host(kr)[b, :, :lb], want_k[b, :, :lb])
        assert np.array_equal(host(vr)[b, :, :lb], want_v[b, :, :lb])


def _paged_items(lens, capacity, num_splits, hkv):
    """Items of the paged flat work list for an explicit split count: chunks
    of ceil(ceil(capacity / 16) / num_splits) 16-key tiles per sequence (one
    for a sequence without keys), times the KV heads."""
    tps = -(-(-(-capacity // 16)) // num_splits)
    return hkv * sum(max(1, -(-(-(-int(l) // 16)) // tps)) for l in lens)


def _as_i32(v):
    return int(np.array(v, dtype=np.uint32).view(np.int32))


@pytest.mark.parametrize("page_size", [16, 64])
def test_paged_counter_start_does_not_matter(da, page_size):
    """A paged call on at most 64 sequences runs resident workgroups that take
    their (chunk, head) items from a counter in the workspace, which the call
    clears first.  With small chunks (far more items than resident
    workgroups; 48-key chunks that do not start on 64-token page boundaries),
    whatever the counter holds before the call -- what the allocation held,
    zero, around the item count, the largest value -- the result is the
    oracle's, bitwise the same each time.  The split partials are poisoned
    with NaN before every call, so a chunk that no workgroup attended would
    show instead of reusing the previous call's partial."""
    hkv, g, d, splits = 8, 4, 128, 100
    lens = [4096, 3001, 64, 0, 1, 2500, 17, 4000]
    case = workloads.paged_case(270 + page_size, len(lens), hkv * g, hkv, d, page_size,
                                4096 // page_size, lens, spare_pages=2)
    kc = oracle.gather_paged(case.k, case.page_table, page_size, case.capacity)
    vc = oracle.gather_paged(case.v, case.page_table, page_size, case.capacity)
    want = oracle.decode_attention(case.q, kc, vc, case.seqlens, case.scale)
    items = _paged_items(lens, case.capacity, splits, hkv)
    assert items > 2 * 512
    q, k, v, sl, pt = (dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens),
                       dev(case.page_table))
    ws = da.Workspace()
    first = None
    for start in (None, 0, 1, items - 1, items, items + 1, 2**31, 2**32 - 1):
        if start is not None:
            ws.buf[:4].view(torch.int32).fill_(_as_i32(start))
            ws.buf[256:].fill_(0xFF)  # NaN in every partial
        out = da.gqa_decode_attn(q, k, v, sl, page_table=pt, page_size=page_size,
                                 num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        got = host(out)
        assert np.all(np.isfinite(got)), start
        assert max_err(got, want) <= ATOL, start
        if first is None:
            first = got.copy()
        assert np.array_equal(got.view(np.uint16), first.view(np.uint16)), start


@pytest.mark.parametrize("page_size", [8, 32])
@pytest.mark.parametrize("d,g", [(64, 1), (64, 2), (64, 4), (64, 8), (128, 1), (128, 2),
                                 (128, 4), (128, 8)])
def test_paged_persistent_launch_shapes(da, d, g, page_size):
    """Every (D, rows) combination of the paged dense stream with many small
    chunks (64 splits per sequence: more (chunk, head) items than resident
    workgroups; where rows * D >= 512 the persistent launch runs and some
    items come from the work counter), against the oracle; ragged lengths, a sequence
    without keys, chunks not aligned to 32-token pages, NaN in unused pool
    pages and in every split partial before the call."""
    hkv, splits = 8, 64  # 1,712 items; at most 1,024 resident workgroups (4 per CU)
    lens = [4096, 2047, 0, 3333, 1, 4000]
    case = workloads.paged_case(300 + d + g + page_size, len(lens), hkv * g, hkv, d, page_size,
                                4096 // page_size, lens, spare_pages=3)
    assert _paged_items(lens, case.capacity, splits, hkv) > 1024
    kc = oracle.gather_paged(case.k, case.page_table, page_size, case.capacity)
    vc = oracle.gather_paged(case.v, case.page_table, page_size, case.capacity)
    want = oracle.decode_attention(case.q, kc, vc, case.seqlens, case.scale)
    q, k, v, sl, pt = (dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens),
                       dev(case.page_table))
    ws = da.Workspace()
    for rep in range(2):
        if rep:
            ws.buf[256:].fill_(0xFF)  # NaN in every partial
        out = da.gqa_decode_attn(q, k, v, sl, page_table=pt, page_size=page_size,
                                 num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        got = host(out)
        assert np.all(np.isfinite(got)), rep
        assert max_err(got, want) <= ATOL, rep


def test_paged_batch_above_64_sequences(da):
    """More than 64 sequences take the flat grid of one workgroup per chunk
    instead of the resident workgroups; against the oracle."""
    hkv, g, d, page_size = 2, 4, 64, 16
    lens = workloads.draw_seqlens(280, 70, 1, 700)
    case = workloads.paged_case(281, len(lens), hkv * g, hkv, d, page_size, 700 // 16 + 1, lens)
    got, _, _ = run_dense(da, case, num_splits=4)
    kc = oracle.gather_paged(case.k, case.page_table, page_size, case.capacity)
    vc = oracle.gather_paged(case.v, case.page_table, page_size, case.capacity)
    want = oracle.decode_attention(case.q, kc, vc, case.seqlens, case.scale)
    assert np.all(np.isfinite(got))
    assert max_err(got, want) <= ATOL


def test_paged_graph_replays(da):
    """The paged call with its work counter, captured in a HIP graph and
    replayed with eager work in between (which also poisons the split
    partials): every replay gives the eager result bitwise."""
    hkv, g, d, page_size, splits = 8, 4, 128, 16, 64
    lens = [4096, 1000, 3333, 16]
    case = workloads.paged_case(290, len(lens), hkv * g, hkv, d, page_size, 4096 // page_size,
                                lens)
    q, k, v, sl, pt = (dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens),
                       dev(case.page_table))
    ws = da.Workspace()
    out = torch.empty_like(q)

    def step():
        da.gqa_decode_attn(q, k, v, sl, page_table=pt, page_size=page_size, num_splits=splits,
                           out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    want = host(out).copy()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        step()
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            step()
    torch.cuda.synchronize()
    noise = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        out.zero_()
        ws.buf[256:].fill_(0xFF)
        noise.mul_(1.0001).add_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint16), want.view(np.uint16)), rep


def test_graph_replays_match_eager(da):
    """The calls captured in a HIP graph (dense decode with append, the fused
    Quest step with a top-K launch and sparse attention, and the Quest step
    as launched by default: scores only, then the attention that selects its
    own pages) give the eager results on every replay, with unrelated eager
    work and synchronisations between the replays."""
    case = workloads.dense_case(980, 2, 32, 8, 128, 2048, [2048, 1500], with_new=True)
    s, budget = 16, 256
    q, sl = dev(case.q), dev(case.seqlens)
    kn, vn = dev(case.k_new), dev(case.v_new)

    def fresh():
        k, v = dev(case.k), dev(case.v)
        meta = torch.zeros((2, 8, 2048 // s, 2, 128), dtype=torch.float16, device=DEV)
        sl_before = dev(case.seqlens - 1)
        da.quest_meta_append(k, v, meta, sl_before, n_new=2048, page_size=s)
        return k, v, meta

    ws, qws = da.Workspace(), da.Workspace()
    idx = torch.empty((2, 8, budget // s), dtype=torch.int32, device=DEV)
    idx_f = torch.empty_like(idx)
    scores = torch.empty((2, 8, 2048 // s), dtype=torch.float32, device=DEV)
    out_d = torch.empty_like(q)
    out_s = torch.empty_like(q)
    out_f = torch.empty_like(q)

    def step(k, v, meta):
        da.gqa_decode_attn(q, k, v, sl, k_new=kn, v_new=vn, out=out_d, workspace=ws)
        da.quest_append_score_topk(q, k, v, meta, sl, kn, vn, page_size=s, budget_tokens=budget,
                                   page_idx=idx, workspace=qws)
        da.quest_sparse_decode_attn(q, k, v, sl, idx, budget_tokens=budget, page_size=s,
                                    out=out_s, workspace=ws)
        # the append again (idempotent), scores only, then the selecting attention
        da.quest_append_score_topk(q, k, v, meta, sl, kn, vn, page_size=s, budget_tokens=budget,
                                   page_scores=scores, select=False, workspace=qws)
        da.quest_select_sparse_decode_attn(q, k, v, sl, scores, budget_tokens=budget,
                                           page_size=s, page_idx=idx_f, out=out_f, workspace=ws)

    k, v, meta = fresh()
    step(k, v, meta)                       # eager reference (appends are idempotent)
    torch.cuda.synchronize()
    want = (host(out_d).copy(), host(out_s).copy(), host(idx).copy(), host(meta).copy(),
            host(out_f).copy(), host(idx_f).copy())
    # the two Quest paths choose the same pages and give the same output
    assert np.array_equal(want[5], want[2])
    assert np.array_equal(want[4].view(np.uint16), want[1].view(np.uint16))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        step(k, v, meta)                   # warm-up on the capture stream
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            step(k, v, meta)
    torch.cuda.synchronize()
    noise = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        out_d.zero_()
        out_s.zero_()
        out_f.zero_()
        idx.fill_(-7)
        idx_f.fill_(-7)
        scores.fill_(float("nan"))
        noise.mul_(1.0001).add_(1.0)        # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (host(out_d), host(out_s), host(idx), host(meta), host(out_f), host(idx_f))
        for a, b in zip(got, want):
            assert np.array_equal(a, b), rep


def test_split_merge_reads_fresh_partials(da):
    """Calls alternate between different inputs and split counts on one
    workspace: every merge must see this call's partials, never the previous
    call's."""
    cases = [workloads.dense_case(600 + i, 2, 32, 8, 128, 4096, [4096, 3001 - 500 * i])
             for i in range(3)]
    wants = [oracle.decode_attention(c.q, c.k, c.v, c.seqlens, c.scale) for c in cases]
    devs = [(dev(c.q), dev(c.k), dev(c.v), dev(c.seqlens)) for c in cases]
    ws = da.Workspace()
    for rep in range(4):
        for i, (q, k, v, sl) in enumerate(devs):
            out = da.gqa_decode_attn(q, k, v, sl, workspace=ws, num_splits=[64, 7, 32][i])
            torch.cuda.synchronize()
            assert max_err(host(out), wants[i]) <= ATOL, (rep, i)


def _topk_case(da, scores_kind, n_pages=2048, k_pages=128, seed=700):
    """Top-K on hand-made metadata: 'equal' makes every page identical (all
    scores tie), 'many_ties' makes 100 identical pages outscore the rest with
    K = 50, so more than 64 candidates tie on the boundary."""
    d, s = 128, 16
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 4, d), dtype=np.float32).astype(np.float16)
    meta = np.zeros((1, 1, n_pages, 2, d), np.float16)
    base = rng.standard_normal((2, d), dtype=np.float32).astype(np.float16)
    lo, hi = np.minimum(base[0], base[1]), np.maximum(base[0], base[1])
    if scores_kind == "equal":
        meta[0, 0, :, 0], meta[0, 0, :, 1] = lo, hi
    else:
        noise = rng.standard_normal((n_pages, 2, d), dtype=np.float32).astype(np.float16)
        meta[0, 0, :, 0] = np.minimum(noise[:, 0], noise[:, 1])
        meta[0, 0, :, 1] = np.maximum(noise[:, 0], noise[:, 1])
        hot = rng.choice(n_pages, 100, replace=False)
        sign = np.sign(q[0].astype(np.float32).sum(0)).astype(np.float16)
        meta[0, 0, hot, 0] = lo + 3 * sign
        meta[0, 0, hot, 1] = hi + 3 * sign
    lens = np.array([n_pages * s], np.int32)
    idx = host(da.quest_page_score_topk(dev(q), dev(meta), dev(lens), page_size=s,
                                        budget_tokens=k_pages * s))
    want = oquest.select_pages(oquest.page_scores(q, meta, lens, s), lens, s, k_pages)
    return idx, want


def test_topk_all_scores_equal(da):
    idx, want = _topk_case(da, "equal")
    assert list(want[0, 0]) == list(range(128))
    assert np.array_equal(idx, want)


def test_topk_many_boundary_ties(da):
    idx, want = _topk_case(da, "many_ties", k_pages=50)
    assert np.array_equal(idx, want)


@pytest.mark.parametrize("n_pages", [8192, 20000])
@pytest.mark.parametrize("kind,k_pages", [("equal", 256), ("many_ties", 50), ("many_ties", 256)])
def test_topk_ties_at_large_page_counts(da, kind, k_pages, n_pages):
    """The same tie cases at 8192 pages (32 items per thread) and at 20000
    (the streaming select): every page tied, and 100 tied pages over the
    rest straddling the K-th place."""
    idx, want = _topk_case(da, kind, n_pages=n_pages, k_pages=k_pages, seed=710)
    if kind == "equal":
        assert list(want[0, 0]) == list(range(k_pages))
    assert np.array_equal(idx, want)
