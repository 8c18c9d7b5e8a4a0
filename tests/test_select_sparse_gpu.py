"""GPU checks of quest_select_sparse_decode_attn, the top-K selection fused
into the attention over the chosen pages, and of the scores-only mode of the
scoring calls that feeds it.

The fused call must make exactly the choice of quest_page_score_topk's top-K
launch and produce bit-identical output to quest_sparse_decode_attn over that
choice (same arithmetic, same split plan): both are compared element by
element, on every items-per-thread width of the in-kernel top-K (up to 16384
pages) and beyond it (where the call runs the streaming top-K launch first),
with ragged and empty sequences, K >= P_b, explicit split counts and a paged
cache.  Two cases are also compared with the fp64 oracle directly.
"""

import numpy as np
import pytest
import torch

from oracle import quest as oquest
from decode_attention_folded_amd import workloads
from test_parity_gpu import ATOL, check_selection, dev, host, max_err, run_meta_bulk

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def da():
    import decode_attention_folded_amd as pkg
    pkg.load_library()
    return pkg


def _two_ways(da, case, page_size, budget, meta_pages, splits=0):
    """Scores, then (top-K launch + selected-page attention) and the fused
    call on the same scores.  Returns (idx_ref, out_ref, idx_fused, out_fused)."""
    pt = dev(case.page_table) if case.page_table is not None else None
    meta = run_meta_bulk(da, case, page_size, meta_pages)
    q, k, v, lens = dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens)
    scores = torch.full((case.batch, case.num_kv_heads, meta_pages), float("nan"),
                        dtype=torch.float32, device=DEV)
    idx_ref = da.quest_page_score_topk(q, meta, lens, page_size=page_size, budget_tokens=budget,
                                       page_scores=scores)
    out_ref = da.quest_sparse_decode_attn(q, k, v, lens, idx_ref, budget_tokens=budget,
                                          page_size=page_size, page_table=pt, num_splits=splits)
    idx_fused = torch.full_like(idx_ref, -7)
    out_fused = da.quest_select_sparse_decode_attn(q, k, v, lens, scores, budget_tokens=budget,
                                                   page_size=page_size, page_table=pt,
                                                   page_idx=idx_fused, num_splits=splits)
    torch.cuda.synchronize()
    return host(idx_ref), host(out_ref), host(idx_fused), host(out_fused)


# page_size, budget, g, d, lens, cap (tokens), splits; the score row is cap / S pages
SELECT_CASES = [
    (16, 256, 4, 128, [4096, 1000, 200, 17], 4096, 0),      # 256 pages: 8 per thread
    (16, 2048, 1, 128, [2048, 2047], 2048, 0),              # K >= P_b: every page
    (8, 64, 2, 64, [1024, 900, 0], 1024, 0),                # an empty sequence
    (32, 512, 8, 128, [3000, 64, 33], 3008, 0),
    (64, 128, 4, 64, [4096, 100], 4096, 3),                 # explicit split count
    (16, 512, 4, 64, [16384 * 4 - 5, 70], 16384 * 4, 0),    # 4096 pages: 16 per thread
    (16, 1024, 2, 64, [8192 * 16, 8192 * 16 - 100], 8192 * 16, 0),  # 8192: 32 per thread
    (8, 4096, 1, 64, [16384 * 8 - 1], 16384 * 8, 1),        # 16384: 64 per thread, 1 split
    (8, 2048, 1, 64, [20000 * 8 - 3, 5000], 20000 * 8, 0),  # 20000: streaming top-K first
]


@pytest.mark.parametrize("page_size,budget,g,d,lens,cap,splits", SELECT_CASES)
def test_select_matches_topk_then_sparse(da, page_size, budget, g, d, lens, cap, splits):
    hkv = 2 if cap <= 16384 else 1
    case = workloads.dense_case(900 + page_size + g, len(lens), hkv * g, hkv, d, cap, lens,
                                plant_pages=4 if cap <= 16384 else 0,
                                plant_page_size=page_size)
    idx_ref, out_ref, idx_fused, out_fused = _two_ways(da, case, page_size, budget,
                                                       cap // page_size, splits)
    assert np.array_equal(idx_fused, idx_ref)
    assert np.array_equal(out_fused.view(np.uint16), out_ref.view(np.uint16))


def test_select_over_paged_cache(da):
    page_size, lens = 16, [1500, 200, 1]
    case = workloads.paged_case(910, 3, 32, 8, 128, page_size, 100, lens)
    idx_ref, out_ref, idx_fused, out_fused = _two_ways(da, case, page_size, 256, 100)
    assert np.array_equal(idx_fused, idx_ref)
    assert np.array_equal(out_fused.view(np.uint16), out_ref.view(np.uint16))


def test_select_without_page_idx_output(da):
    """page_idx is optional: the output is the same without it."""
    page_size, budget, lens = 16, 512, [3000, 1200]
    case = workloads.dense_case(920, 2, 16, 4, 128, 3008, lens)
    meta = run_meta_bulk(da, case, page_size, 188)
    q, k, v, ln = dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens)
    scores = torch.empty((2, 4, 188), dtype=torch.float32, device=DEV)
    da.quest_page_score_topk(q, meta, ln, page_size=page_size, budget_tokens=budget,
                             page_scores=scores, select=False)
    idx = torch.empty((2, 4, budget // page_size), dtype=torch.int32, device=DEV)
    a = da.quest_select_sparse_decode_attn(q, k, v, ln, scores, budget_tokens=budget,
                                           page_size=page_size, page_idx=idx)
    b = da.quest_select_sparse_decode_attn(q, k, v, ln, scores, budget_tokens=budget,
                                           page_size=page_size)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_select_sparse_parity_with_oracle(da):
    """Metadata, scores only, then the fused call, against the oracle running
    the same steps: the choice agrees under the near-tie rule, and the output
    is within the attention tolerance of the oracle's attention over the pages
    the GPU chose."""
    page_size, budget, lens = 16, 512, [8192, 3000, 5]
    case = workloads.dense_case(930, 3, 32, 8, 128, 8192, lens, plant_pages=8)
    meta = run_meta_bulk(da, case, page_size, 512)
    q, k, v, ln = dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens)
    scores = torch.empty((3, 8, 512), dtype=torch.float32, device=DEV)
    da.quest_page_score_topk(q, meta, ln, page_size=page_size, budget_tokens=budget,
                             page_scores=scores, select=False)
    idx = torch.empty((3, 8, budget // page_size), dtype=torch.int32, device=DEV)
    out = da.quest_select_sparse_decode_attn(q, k, v, ln, scores, budget_tokens=budget,
                                             page_size=page_size, page_idx=idx)
    torch.cuda.synchronize()
    want_meta = oquest.build_metadata(case.k, case.seqlens, page_size, 512)
    want_scores = oquest.page_scores(case.q, want_meta, case.seqlens, page_size)
    want_idx = oquest.select_pages(want_scores, case.seqlens, page_size, budget // page_size)
    check_selection(host(idx), host(scores).astype(np.float64), want_idx, want_scores,
                    case.seqlens, page_size, budget // page_size)
    want = oquest.sparse_decode_attention(case.q, case.k, case.v, case.seqlens, host(idx),
                                          page_size, case.scale)
    assert max_err(host(out), want) <= ATOL


def test_select_beyond_register_held_top_k(da):
    """More than 16384 pages per unit: the call runs the streaming top-K, then
    the attention over its choice, written to page_idx or (without it) to the
    workspace.  Both give the same output, the choice agrees with the oracle's
    under the near-tie rule, and the output with the oracle's attention over
    the GPU's choice."""
    page_size, budget, g = 16, 1024, 4
    cap = 16384 * 16 + 1600                 # 16484 pages
    lens = [cap, cap - 700]
    case = workloads.dense_case(940, 2, g, 1, 64, cap, lens, plant_pages=6,
                                plant_page_size=page_size)
    n_meta = cap // page_size
    meta = run_meta_bulk(da, case, page_size, n_meta)
    q, k, v, ln = dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens)
    scores = torch.empty((2, 1, n_meta), dtype=torch.float32, device=DEV)
    da.quest_page_score_topk(q, meta, ln, page_size=page_size, budget_tokens=budget,
                             page_scores=scores, select=False)
    idx = torch.full((2, 1, budget // page_size), -7, dtype=torch.int32, device=DEV)
    a = da.quest_select_sparse_decode_attn(q, k, v, ln, scores, budget_tokens=budget,
                                           page_size=page_size, page_idx=idx)
    b = da.quest_select_sparse_decode_attn(q, k, v, ln, scores, budget_tokens=budget,
                                           page_size=page_size)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    want_meta = oquest.build_metadata(case.k, case.seqlens, page_size, n_meta)
    want_scores = oquest.page_scores(case.q, want_meta, case.seqlens, page_size)
    want_idx = oquest.select_pages(want_scores, case.seqlens, page_size, budget // page_size)
    check_selection(host(idx), host(scores).astype(np.float64), want_idx, want_scores,
                    case.seqlens, page_size, budget // page_size)
    want = oquest.sparse_decode_attention(case.q, case.k, case.v, case.seqlens, host(idx),
                                          page_size, case.scale)
    assert max_err(host(a), want) <= ATOL


def test_scores_only_mode(da):
    """select=False writes the same scores and, with the append, the same
    cache and metadata as the full call, and launches no top-K."""
    page_size, budget, lens = 16, 256, [1000, 17]
    case = workloads.dense_case(940, 2, 16, 4, 64, 1024, lens, with_new=True)
    q, ln = dev(case.q), dev(case.seqlens)
    meta0 = run_meta_bulk(da, case, page_size, 64)
    outs = []
    for select in (True, False):
        k, v, meta = dev(case.k), dev(case.v), meta0.clone()
        scores = torch.full((2, 4, 64), float("nan"), dtype=torch.float32, device=DEV)
        r = da.quest_append_score_topk(q, k, v, meta, ln, dev(case.k_new), dev(case.v_new),
                                       page_size=page_size, budget_tokens=budget,
                                       page_scores=scores, select=select)
        torch.cuda.synchronize()
        assert (r is None) == (not select)
        outs.append((host(k), host(v), host(meta), host(scores)))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    with pytest.raises(ValueError):
        da.quest_page_score_topk(q, meta0, ln, page_size=page_size, budget_tokens=budget,
                                 select=False)
