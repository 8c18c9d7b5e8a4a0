"""Pins for the CPU oracle: facts fixed by the pages or by mathematics, checked
without reference to the oracle's own formulas.

Each pin is chosen so that a plausible mistake (a wrong head map, a dropped
scale, a wrong sign in the page score, an off-by-one in the page range, a
tie broken the wrong way) fails at least one of them; the mutation tests at the
end plant such mistakes in the oracle and check that a pin catches each.
"""

import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import dense as odense
from oracle import quest as oquest
from decode_attention_folded_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _fold_attention(q, k, v, seqlens, scale):
    """The fold written as on the Core ML page (section 3 "Implementation"):
    reshape Q to [B, Hkv, G, D], multiply against K/V at their stored width,
    softmax over context, reshape back.  Independent of repeat_kv."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        lb = int(seqlens[b])
        qf = q[b].reshape(hkv, g, d)
        kb = np.asarray(k[b, :, :lb], dtype=np.float64)
        vb = np.asarray(v[b, :, :lb], dtype=np.float64)
        s = np.einsum("kgd,ktd->kgt", qf, kb) * scale
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        out[b] = np.einsum("kgt,ktd->kgd", p, vb).reshape(hq, d)
    return out


# ----------------------------------------------------------------- dense


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_fold_equals_repeat_kv(group):
    """[CoreML-GQA] section 3 "Why the Computation Is Equivalent": the fold
    gives the repeat_kv result row for row (the page reports exactly matching
    outputs on its tested inputs)."""
    hkv, d, cap = 3, 16, 40
    case = workloads.dense_case(7, 2, hkv * group, hkv, d, cap, [37, 5])
    ref = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    fold = _fold_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    np.testing.assert_allclose(ref, fold, rtol=0, atol=1e-12)


@pytest.mark.parametrize("group,seqlens", [(4, [33, 1, 17]), (1, [8, 9, 2]), (8, [64, 63, 5])])
def test_matches_torch_sdpa_fp64(group, seqlens):
    """Library special case: torch's scaled_dot_product_attention in float64
    on the CPU with its native GQA broadcast and a boolean length mask."""
    hkv, d, cap = 2, 32, 64
    case = workloads.dense_case(11, 3, hkv * group, hkv, d, cap, seqlens, poison=False)
    ref = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    q = torch.from_numpy(case.q.astype(np.float64))[:, :, None, :]
    k = torch.from_numpy(case.k.astype(np.float64))
    v = torch.from_numpy(case.v.astype(np.float64))
    mask = torch.arange(cap)[None, None, None, :] < torch.tensor(seqlens)[:, None, None, None]
    lib = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=case.scale,
                                         enable_gqa=True)[:, :, 0, :].numpy()
    np.testing.assert_allclose(ref, lib, rtol=0, atol=1e-12)


# ----------------------------------------------------------- q_len > 1


def _causal_mask(seqlens, lq, cap):
    """Boolean [B, 1, Lq, cap]: query i of sequence b (position L_b - Lq + i)
    sees key t iff t <= L_b - Lq + i."""
    pos = torch.tensor(seqlens)[:, None, None, None] - lq + torch.arange(lq)[None, None, :, None]
    return torch.arange(cap)[None, None, None, :] <= pos


@pytest.mark.parametrize("group,lq,seqlens", [(4, 2, [33, 2, 17]), (1, 8, [8, 9, 40]),
                                              (2, 4, [64, 5, 4])])
def test_multi_query_matches_torch_sdpa_fp64(group, lq, seqlens):
    """Library special case for the q_len > 1 reading: torch's
    scaled_dot_product_attention in float64 on the CPU, native GQA broadcast,
    with an explicit position mask (query i of a sequence of length L sits at
    L - q_len + i and sees keys up to its own position)."""
    hkv, d, cap = 2, 32, 64
    case = workloads.dense_case(13, 3, hkv * group, hkv, d, cap, seqlens, poison=False)
    rng = np.random.default_rng(14)
    q = rng.standard_normal((3, hkv * group, lq, d), dtype=np.float32).astype(np.float16)
    ref = oracle.multi_query_attention(q, case.k, case.v, case.seqlens, case.scale)
    lib = F.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)), torch.from_numpy(case.k.astype(np.float64)),
        torch.from_numpy(case.v.astype(np.float64)), attn_mask=_causal_mask(seqlens, lq, cap),
        scale=case.scale, enable_gqa=True).numpy()
    np.testing.assert_allclose(ref, lib, rtol=0, atol=1e-12)


def test_multi_query_special_cases():
    """q_len = 1 is single-token decode; with L = q_len the first query sees
    only key 0 (o = v_0 exactly) and the last sees every key; a query before
    the start of the sequence (L < q_len) gets zeros."""
    hkv, g, d, cap = 2, 4, 64, 32
    case = workloads.dense_case(15, 2, hkv * g, hkv, d, cap, [20, 5])
    q1 = case.q[:, :, None, :]
    np.testing.assert_array_equal(
        oracle.multi_query_attention(q1, case.k, case.v, case.seqlens, case.scale)[:, :, 0],
        oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale))
    rng = np.random.default_rng(16)
    lq = 5
    q = rng.standard_normal((2, hkv * g, lq, d), dtype=np.float32).astype(np.float16)
    out = oracle.multi_query_attention(q, case.k, case.v, [20, 5], case.scale)
    for h in range(hkv * g):
        np.testing.assert_array_equal(out[1, h, 0], case.v[1, h // g, 0].astype(np.float64))
    last = oracle.decode_attention(q[:, :, lq - 1], case.k, case.v, [20, 5], case.scale)
    np.testing.assert_allclose(out[:, :, lq - 1], last, rtol=0, atol=1e-12)
    short = oracle.multi_query_attention(q, case.k, case.v, [3, 5], case.scale)
    assert np.all(short[0, :, :2] == 0.0) and np.all(short[0, :, 2:] != 0.0)


def test_mutation_multi_query_off_by_one_is_caught(monkeypatch):
    real = odense.multi_query_attention

    def one_key_short(q, k, v, seqlens, scale):
        # each query sees one key fewer than its own position
        out = real(q, k, v, [int(l) - 1 for l in seqlens], scale)
        return out
    monkeypatch.setattr(oracle, "multi_query_attention", one_key_short)
    with pytest.raises(AssertionError):
        test_multi_query_matches_torch_sdpa_fp64(4, 2, [33, 2, 17])


def test_single_key_returns_its_value():
    """With one valid key the softmax is exactly 1: o = v_0 for every query
    head of the group."""
    case = workloads.dense_case(3, 2, 8, 2, 64, 16, [1, 1])
    out = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    for b in range(2):
        for h in range(8):
            np.testing.assert_array_equal(out[b, h], case.v[b, h // 4, 0].astype(np.float64))


def test_identical_keys_average_values():
    """Equal keys give equal weights: o = mean of the valid values."""
    case = workloads.dense_case(4, 1, 4, 1, 64, 32, [20])
    case.k[:, :, :20, :] = case.k[:, :, :1, :]
    out = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    want = case.v[0, 0, :20].astype(np.float64).mean(axis=0)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], want, rtol=0, atol=1e-12)


def test_dominant_key_and_head_map():
    """A key aligned with only query head h*G+g's query dominates that head's
    softmax: that head returns (almost) that key's value, which checks the head
    map h = G*kv + g ([CoreML-GQA] "Why Reshape Replaces Integer Division")."""
    hkv, group, d, cap = 4, 4, 64, 64
    case = workloads.dense_case(5, 1, hkv * group, hkv, d, cap, [cap], poison=False)
    kv, g, t = 2, 3, 41
    h = kv * group + g
    q = np.zeros_like(case.q)
    q[0, h, :] = 1.0
    case.k[0, kv, t, :] = 8.0
    case.q[:] = q
    out = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, 1.0)
    np.testing.assert_allclose(out[0, h], case.v[0, kv, t].astype(np.float64), atol=1e-12)
    # every other head has an all-zero query: uniform weights, mean of its KV head
    for hh in range(hkv * group):
        if hh == h:
            continue
        want = case.v[0, hh // group].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(out[0, hh], want, atol=1e-12)


def test_mask_equals_truncation_and_ignores_poison():
    """Length L_b < capacity is the same as a cache cut to [0, L_b); the NaN
    written past L_b never reaches the output."""
    case = workloads.dense_case(6, 2, 8, 2, 64, 48, [30, 48])
    out = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    assert np.all(np.isfinite(out))
    cut = oracle.decode_attention(case.q[:1], case.k[:1, :, :30], case.v[:1, :, :30],
                                  [30], case.scale)
    np.testing.assert_array_equal(out[:1], cut)


def test_append_then_attend():
    """Appending the new row at slot L_b - 1 then attending equals attending
    on a cache that already held the row ([CoreML-GQA] section 1)."""
    case = workloads.dense_case(8, 2, 8, 2, 64, 40, [25, 40], with_new=True)
    k2, v2 = oracle.append_kv(case.k, case.v, case.seqlens, case.k_new, case.v_new)
    prefilled_k = case.k.copy()
    prefilled_v = case.v.copy()
    prefilled_k[0, :, 24] = case.k_new[0]
    prefilled_v[0, :, 24] = case.v_new[0]
    prefilled_k[1, :, 39] = case.k_new[1]
    prefilled_v[1, :, 39] = case.v_new[1]
    np.testing.assert_array_equal(k2, prefilled_k)
    np.testing.assert_array_equal(
        oracle.decode_attention(case.q, k2, v2, case.seqlens, case.scale),
        oracle.decode_attention(case.q, prefilled_k, prefilled_v, case.seqlens, case.scale))
    # the untouched original differs in exactly those rows
    assert not np.array_equal(k2, case.k)


@pytest.mark.parametrize("page_size", [8, 16, 32])
def test_paged_gather_round_trip(page_size):
    """Scatter a contiguous cache into a pool by a random page permutation
    (written here, independently of the oracle's gather), gather it back with
    the oracle's paged addressing, and attention must not change."""
    bsz, hkv, d, max_pages = 3, 2, 16, 6
    cap = max_pages * page_size
    lens = [cap, page_size * 2 + 3, 1]
    case = workloads.dense_case(9, bsz, 4, hkv, d, cap, lens, poison=False)
    rng = np.random.default_rng(0)
    n_pool = bsz * max_pages + 2
    perm = rng.permutation(n_pool)
    pool_k = np.full((n_pool, hkv, page_size, d), np.nan, np.float16)
    pool_v = np.full((n_pool, hkv, page_size, d), np.nan, np.float16)
    table = np.full((bsz, max_pages), -1, np.int32)
    nxt = 0
    for b in range(bsz):
        for p in range((lens[b] + page_size - 1) // page_size):
            phys = perm[nxt]
            nxt += 1
            table[b, p] = phys
            for r in range(page_size):
                pool_k[phys, :, r] = case.k[b, :, p * page_size + r]
                pool_v[phys, :, r] = case.v[b, :, p * page_size + r]
    gk = oracle.gather_paged(pool_k, table, page_size, cap)
    gv = oracle.gather_paged(pool_v, table, page_size, cap)
    for b in range(bsz):
        n = ((lens[b] + page_size - 1) // page_size) * page_size
        np.testing.assert_array_equal(gk[b, :, :n], case.k[b, :, :n])
        np.testing.assert_array_equal(gv[b, :, :n], case.v[b, :, :n])
    np.testing.assert_array_equal(
        oracle.decode_attention(case.q, gk, gv, lens, case.scale),
        oracle.decode_attention(case.q, case.k, case.v, lens, case.scale))


def test_empty_sequence_returns_zero():
    case = workloads.dense_case(10, 2, 4, 1, 64, 16, [0, 3])
    out = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    assert np.all(out[0] == 0.0) and np.all(np.isfinite(out[1]))


# ----------------------------------------------------------------- quest


def test_worked_example_page_scores():
    """[Quest-review] worked example: U(A, q) = 0.7 + 0.6 + 0.06 = 1.36 with true
    dots -0.49 and 1.12; page B = {(1.2, 0, 0)} scores 1.2 = its dot; U ranks A
    above B although B holds the larger true dot."""
    ex = _golden("quest_worked_example.json")
    q = np.array(ex["q"], dtype=np.float64)
    keys = np.zeros((1, 1, 4, 3), dtype=np.float64)
    keys[0, 0, 0:2] = ex["page_A_keys"]
    keys[0, 0, 2:3] = ex["page_B_keys"]
    # page size 2: page 0 = A (2 keys), page 1 = B (1 key, partial page)
    meta = oquest.build_metadata(keys, [3], 2, 2)
    u = oquest.page_scores(q[None, None, :], meta, [3], 2)[0, 0]
    assert abs(u[0] - ex["U_A"]) < 1e-12
    assert abs(u[1] - ex["U_B"]) < 1e-12
    terms = np.maximum(q * meta[0, 0, 0, 0], q * meta[0, 0, 0, 1])
    np.testing.assert_allclose(terms, ex["U_A_channel_terms"], atol=1e-12)
    np.testing.assert_allclose(keys[0, 0, 0:2] @ q, ex["true_dots_A"], atol=1e-12)
    assert abs(keys[0, 0, 2] @ q - ex["true_dot_B"]) < 1e-12
    # U ranks A first; the true maximum dot ranks B first
    sel = oquest.select_pages(u[None, None, :], [3], 2, 1)
    assert sel[0, 0, 0] == 0
    assert max(keys[0, 0, 0:2] @ q) < keys[0, 0, 2] @ q


@pytest.mark.parametrize("page_size,seqlen", [(16, 100), (8, 64), (1, 20), (32, 31)])
def test_score_is_upper_bound_and_closed_form(page_size, seqlen):
    """[Quest-review] (paper section 3.4): q.k <= U(p, q) for every key in the
    page.  Closed form: U = sum_i q_i c_i + |q_i| r_i with c = (M + m)/2 and
    r = (M - m)/2 (the maximum of q.k over the box [m, M]).  S = 1 gives
    U = q.k exactly."""
    hkv, group, d = 2, 4, 32
    case = workloads.dense_case(12, 2, hkv * group, hkv, d, seqlen + 8, [seqlen, seqlen - 3])
    n_pages = (seqlen + page_size - 1) // page_size
    meta = oquest.build_metadata(case.k, case.seqlens, page_size, n_pages)
    u = oquest.page_scores(case.q, meta, case.seqlens, page_size)
    q64 = case.q.astype(np.float64)
    for b in range(2):
        lb = int(case.seqlens[b])
        for kv in range(hkv):
            qg = q64[b, kv * group:(kv + 1) * group]
            for p in range(oquest.page_count(lb, page_size)):
                keys = case.k[b, kv, p * page_size:min(p * page_size + page_size, lb)]
                keys = keys.astype(np.float64)
                dots = (keys @ qg.T).sum(axis=1)     # summed over the group
                assert np.all(dots <= u[b, kv, p] + 1e-9)
                lo, hi = keys.min(axis=0), keys.max(axis=0)
                c, r = (hi + lo) / 2, (hi - lo) / 2
                closed = sum(float(qh @ c + np.abs(qh) @ r) for qh in qg)
                assert abs(closed - u[b, kv, p]) < 1e-9
                if page_size == 1:
                    assert abs(dots[0] - u[b, kv, p]) < 1e-9
            # pages past the end do not exist
            assert np.all(np.isneginf(u[b, kv, oquest.page_count(lb, page_size):]))


def test_ranking_invariant_under_positive_scale():
    case = workloads.dense_case(13, 1, 8, 2, 64, 256, [250])
    meta = oquest.build_metadata(case.k, case.seqlens, 16, 16)
    u1 = oquest.page_scores(case.q, meta, case.seqlens, 16)
    u2 = oquest.page_scores(case.q.astype(np.float64) * 3.0, meta, case.seqlens, 16)
    np.testing.assert_array_equal(oquest.select_pages(u1, case.seqlens, 16, 5),
                                  oquest.select_pages(u2, case.seqlens, 16, 5))


@pytest.mark.parametrize("page_size", [8, 16])
def test_metadata_bulk_equals_incremental_equals_brute(page_size):
    """Metadata built in one pass, built key by key as new keys arrive, and
    computed by brute force over explicit token lists all agree bit for bit."""
    hkv, d, cap = 2, 64, 90
    lens = [90, 37, 1, 16]
    case = workloads.dense_case(14, 4, 4, hkv, d, cap, lens)
    max_pages = (cap + page_size - 1) // page_size
    bulk = oquest.build_metadata(case.k, case.seqlens, page_size, max_pages)
    inc = np.zeros_like(bulk)
    for step in range(1, cap + 1):
        cur = np.minimum(case.seqlens, step)
        inc = oquest.append_metadata(inc, case.k, cur, 1, page_size)
    for b, lb in enumerate(lens):
        for p in range(oquest.page_count(lb, page_size)):
            toks = [t for t in range(lb) if t // page_size == p]
            brute_min = np.array([[min(case.k[b, kv, t, i] for t in toks) for i in range(d)]
                                  for kv in range(hkv)], dtype=np.float16)
            np.testing.assert_array_equal(bulk[b, :, p, 0], brute_min)
            np.testing.assert_array_equal(bulk[b, :, p, 1], case.k[b][:, toks].max(axis=1))
            np.testing.assert_array_equal(inc[b, :, p], bulk[b, :, p])
    # a bulk append over [0, L) equals the bulk build
    inc2 = oquest.append_metadata(np.zeros_like(bulk), case.k, case.seqlens, cap, page_size)
    for b, lb in enumerate(lens):
        n = oquest.page_count(lb, page_size)
        np.testing.assert_array_equal(inc2[b, :, :n], bulk[b, :, :n])


def _valid_selection(scores, chosen):
    """The defining property of top-K with ties to the lower index: every
    chosen page beats every unchosen page under (higher U, then lower index)."""
    others = [p for p in range(len(scores)) if p not in chosen]
    for s in chosen:
        for u in others:
            if not (scores[s] > scores[u] or (scores[s] == scores[u] and s < u)):
                return False
    return True


@pytest.mark.parametrize("seed", range(6))
def test_topk_exhaustive_tiny(seed):
    rng = np.random.default_rng(seed)
    n_pages = 7
    scores = np.round(rng.standard_normal(n_pages), 1)   # rounding plants ties
    for k in range(1, n_pages + 2):
        sel = oquest.select_pages(scores[None, None, :], [n_pages * 4], 4, k)[0, 0]
        chosen = [int(p) for p in sel if p >= 0]
        assert chosen == sorted(chosen)
        assert len(chosen) == min(k, n_pages)
        if k > n_pages:
            assert list(sel[n_pages:]) == [-1] * (k - n_pages)
        valid = [set(c) for c in itertools.combinations(range(n_pages), min(k, n_pages))
                 if _valid_selection(scores, set(c))]
        assert valid == [set(chosen)]


def test_topk_planted_exact_ties_pick_lower_index():
    """Pages with identical keys score identically; the lower index wins.

    Every key of pages 5, 9 and 12 is 8 * sign(w) per channel, w = the sum of
    the group's queries, so those pages score 8 * sum_i |w_i| > 0, far above
    any page of N(0,1) keys (whose min/max box spans about +-2): they are the
    top three, tied, and a budget of two pages must take 5 and 9."""
    hkv, d, s = 1, 64, 16
    case = workloads.dense_case(15, 1, 4, hkv, d, 16 * s, [16 * s])
    w = case.q[0].astype(np.float64).sum(0)
    planted = np.where(w >= 0, 8.0, -8.0).astype(np.float16)
    for p in (5, 9, 12):
        case.k[0, 0, p * s:(p + 1) * s] = planted
    meta = oquest.build_metadata(case.k, case.seqlens, s, 16)
    u = oquest.page_scores(case.q, meta, case.seqlens, s)
    assert u[0, 0, 5] == u[0, 0, 9] == u[0, 0, 12]
    assert u[0, 0, 5] == pytest.approx(8.0 * np.abs(w).sum(), rel=1e-12)
    others = np.delete(u[0, 0], [5, 9, 12])
    assert u[0, 0, 5] > others.max()
    assert list(oquest.select_pages(u, case.seqlens, s, 2)[0, 0]) == [5, 9]
    assert list(oquest.select_pages(u, case.seqlens, s, 1)[0, 0]) == [5]
    assert list(oquest.select_pages(u, case.seqlens, s, 3)[0, 0]) == [5, 9, 12]


def test_sparse_all_pages_equals_dense():
    """With every page chosen, Quest's attention is dense attention."""
    case = workloads.dense_case(16, 2, 8, 2, 64, 200, [200, 77])
    k_pages = 13
    idx = np.full((2, 2, k_pages), -1, np.int32)
    for b, lb in enumerate([200, 77]):
        n = oquest.page_count(lb, 16)
        idx[b, :, :n] = np.arange(n)
    sparse = oquest.sparse_decode_attention(case.q, case.k, case.v, case.seqlens, idx, 16,
                                            case.scale)
    dense = oracle.decode_attention(case.q, case.k, case.v, case.seqlens, case.scale)
    np.testing.assert_allclose(sparse, dense, rtol=0, atol=1e-12)


def test_sparse_equals_attention_on_gathered_pages():
    """Second construction: copy the chosen pages' tokens into a compact cache
    and run plain attention on it; it must equal the masked oracle."""
    s, hkv, group, d = 16, 2, 4, 64
    lens = [300, 129]
    case = workloads.dense_case(17, 2, hkv * group, hkv, d, 320, lens)
    meta = oquest.build_metadata(case.k, case.seqlens, s, 20)
    u = oquest.page_scores(case.q, meta, case.seqlens, s)
    idx = oquest.select_pages(u, case.seqlens, s, 4)
    sparse = oquest.sparse_decode_attention(case.q, case.k, case.v, case.seqlens, idx, s,
                                            case.scale)
    for b in range(2):
        for kv in range(hkv):
            toks = [t for p in idx[b, kv] if p >= 0
                    for t in range(p * s, min(p * s + s, lens[b]))]
            kk = case.k[b:b + 1, kv:kv + 1, toks]
            vv = case.v[b:b + 1, kv:kv + 1, toks]
            qq = case.q[b:b + 1, kv * group:(kv + 1) * group]
            want = oracle.decode_attention(qq, kk, vv, [len(toks)], case.scale)
            np.testing.assert_allclose(sparse[b, kv * group:(kv + 1) * group], want[0],
                                       rtol=0, atol=1e-12)


def test_planted_pages_are_found():
    """Sanity of the planted workload: shifted pages rank at the top (a
    statistic of the synthetic recipe, reported rather than a property of the
    method)."""
    case = workloads.dense_case(18, 1, 4, 1, 128, 4096, [4096], plant_pages=8)
    meta = oquest.build_metadata(case.k, case.seqlens, 16, 256)
    u = oquest.page_scores(case.q, meta, case.seqlens, 16)
    sel = set(int(p) for p in oquest.select_pages(u, case.seqlens, 16, 32)[0, 0])
    recall = len(set(case.planted[(0, 0)]) & sel) / 8
    # chance level for 32 of 256 pages is 1/8; the shift is about 1.8 noise
    # standard deviations of U at G = 4, D = 128, so recall is high but not 1
    assert recall >= 0.5


# ------------------------------------------------------------- byte model


def test_byte_model_examples():
    ex = _golden("quest_byte_model.json")
    e = ex["example"]
    assert e["K"] * e["S"] == e["budget_tokens"]
    assert oracle.quest_read_ratio(e["L"], e["S"], e["K"]) == e["ratio"]
    t = ex["token_budget_example"]
    assert t["K"] * t["S"] == t["budget_tokens"]
    # the two Quest workloads: L=32768, K=128 -> 1/8; L=131072, K=256 -> 3/32
    assert oracle.quest_read_ratio(32768, 16, 128) == 0.125
    assert oracle.quest_read_ratio(131072, 16, 256) == 3 / 32
    # accounted by counting: one min and one max vector per page, K and V of
    # each chosen full page
    L, S, K, M = 32768, 16, 128, 128 * 2
    d_meta, d_sel, d_full = oracle.quest_read_bytes(L, S, K, M)
    assert d_meta == (L // S) * 2 * M
    assert d_sel == K * S * 2 * M
    assert (d_meta + d_sel) / d_full == 0.125


def test_core_ml_sizes():
    g = _golden("coreml_sizes.json")
    layers, (hkv, ctx, d) = g["layers"], g["kv_cache_shape_per_layer"]
    assert hkv * ctx * d * 2 == g["bytes_per_kv_tensor"]
    assert layers * oracle.dense_kv_bytes([ctx], hkv, d) == g["bytes_all_layers_k_plus_v"]
    assert layers * 2 * hkv * d * 2 == g["bytes_new_per_token_all_layers"]
    rep = odense.repeat_kv(np.zeros((1, hkv, ctx, d), np.float16), g["group"])
    assert rep.nbytes == g["repeat_kv_output_bytes_per_tensor"]
    assert g["tile_ops"] * rep.nbytes == g["tile_output_bytes_total"]
    assert 2 * g["tile_output_bytes_total"] == g["tile_write_plus_read_bytes"]
    q = np.zeros(g["decode_q_shape"], np.float16)
    assert q.nbytes == g["decode_q_bytes"]
    assert q.reshape(g["fold_shape"]).nbytes == q.nbytes


# -------------------------------------------------- planted oracle mistakes


def _wrong_repeat_kv(x, n_rep):
    # head h reads kv head h % Hkv (interleaved) instead of h // G
    return np.tile(x, (1, n_rep, 1, 1))


def test_mutation_wrong_head_map_is_caught(monkeypatch):
    monkeypatch.setattr(odense, "repeat_kv", _wrong_repeat_kv)
    with pytest.raises(AssertionError):
        test_matches_torch_sdpa_fp64(4, [33, 1, 17])


def test_mutation_wrong_score_sign_is_caught(monkeypatch):
    def wrong_scores(q, meta, seqlens, page_size):
        # uses the max vector for every channel regardless of the sign of q_i
        q64 = np.asarray(q, dtype=np.float64)
        bsz, hq, d = q64.shape
        hkv, mp = meta.shape[1], meta.shape[2]
        g = hq // hkv
        out = np.full((bsz, hkv, mp), -np.inf)
        for b in range(bsz):
            n = oquest.page_count(seqlens[b], page_size)
            for kv in range(hkv):
                maxs = np.asarray(meta[b, kv, :n, 1], dtype=np.float64)
                out[b, kv, :n] = sum((maxs * q64[b, kv * g + j]).sum(axis=1) for j in range(g))
        return out
    monkeypatch.setattr(oquest, "page_scores", wrong_scores)
    with pytest.raises(AssertionError):
        test_worked_example_page_scores()


def test_mutation_tie_to_higher_index_is_caught(monkeypatch):
    def wrong_select(scores, seqlens, page_size, k_pages):
        bsz, hkv, _ = scores.shape
        out = np.full((bsz, hkv, k_pages), -1, np.int32)
        for b in range(bsz):
            n = oquest.page_count(seqlens[b], page_size)
            for kv in range(hkv):
                order = sorted(range(n), key=lambda p: (-scores[b, kv, p], -p))
                ch = sorted(order[:k_pages])
                out[b, kv, :len(ch)] = ch
        return out
    monkeypatch.setattr(oquest, "select_pages", wrong_select)
    with pytest.raises(AssertionError):
        for seed in range(6):
            test_topk_exhaustive_tiny(seed)


def test_mutation_missing_scale_is_caught(monkeypatch):
    real = odense.decode_attention

    def no_scale(q, k, v, seqlens, scale, token_mask=None):
        return real(q, k, v, seqlens, 1.0, token_mask)
    monkeypatch.setattr(oracle, "decode_attention", no_scale)
    with pytest.raises(AssertionError):
        test_matches_torch_sdpa_fp64(4, [33, 1, 17])


def test_mutation_page_off_by_one_is_caught(monkeypatch):
    real = oquest.build_metadata

    def shifted(k_cache, seqlens, page_size, max_pages):
        # pages start one token late
        k2 = np.concatenate([k_cache[:, :, :1], k_cache[:, :, :-1]], axis=2)
        return real(k2, seqlens, page_size, max_pages)
    monkeypatch.setattr(oquest, "build_metadata", shifted)
    with pytest.raises(AssertionError):
        test_metadata_bulk_equals_incremental_equals_brute(16)


def test_generators_are_deterministic():
    a = workloads.dense_case(21, 2, 8, 2, 64, 40, [40, 3], with_new=True, plant_pages=1)
    b = workloads.dense_case(21, 2, 8, 2, 64, 40, [40, 3], with_new=True, plant_pages=1)
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.k_new, b.k_new)]:
        assert x.tobytes() == y.tobytes()
    p1 = workloads.paged_case(22, 3, 8, 2, 64, 16, 8, [100, 16, 7])
    p2 = workloads.paged_case(22, 3, 8, 2, 64, 16, 8, [100, 16, 7])
    assert p1.k.tobytes() == p2.k.tobytes()
    assert np.array_equal(p1.page_table, p2.page_table)
