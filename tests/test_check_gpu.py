"""GPU check of da_check_cache, the debugging aid that reports the inputs the
other calls clamp or mask on the device: lengths outside [0, capacity] and
page-table entries of valid pages outside the pool.  The expected reports are
counted on the host from the same arrays."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def da():
    import decode_attention_folded_amd as pkg
    pkg.load_library()
    return pkg


def expected(lens, cap, table=None, num_pages=0, page_size=16):
    bad_len = [b for b, L in enumerate(lens) if L < 0 or L > cap]
    bad_page = 0
    firsts = list(bad_len)
    if table is not None:
        for b, L in enumerate(lens):
            L = min(max(L, 0), cap)
            pages = -(-L // page_size)
            n = sum(1 for e in table[b, :pages] if e < 0 or e >= num_pages)
            bad_page += n
            if n:
                firsts.append(b)
    return [len(bad_len), bad_page, min(firsts) if firsts else -1, 0]


def test_clean_contiguous_cache_reports_nothing(da):
    k = torch.zeros((3, 2, 256, 64), dtype=torch.float16, device=DEV)
    lens = torch.tensor([256, 0, 17], dtype=torch.int32, device=DEV)
    rep = da.check_cache(k, k, lens).cpu().tolist()
    assert rep == [0, 0, -1, 0]


def test_lengths_outside_the_capacity_are_counted(da):
    k = torch.zeros((5, 2, 256, 64), dtype=torch.float16, device=DEV)
    lens_h = [256, -3, 257, 0, 100000]
    lens = torch.tensor(lens_h, dtype=torch.int32, device=DEV)
    rep = da.check_cache(k, k, lens).cpu().tolist()
    assert rep == expected(lens_h, 256) == [3, 0, 1, 0]


@pytest.mark.parametrize("batch", [4, 300])
def test_page_table_entries_outside_the_pool_are_counted(da, batch):
    rng = np.random.default_rng(41 + batch)
    page_size, max_pages, num_pages = 16, 40, 500
    pool = torch.zeros((num_pages, 2, page_size, 64), dtype=torch.float16, device=DEV)
    lens_h = rng.integers(0, max_pages * page_size + 1, size=batch).tolist()
    lens_h[0] = max_pages * page_size + 9   # beyond the capacity: clamped, counted
    table = rng.integers(0, num_pages, size=(batch, max_pages)).astype(np.int32)
    # plant bad entries, some inside the valid pages, some past them (ignored)
    for b in range(batch):
        for _ in range(3):
            p = int(rng.integers(0, max_pages))
            table[b, p] = int(rng.choice([-1, num_pages, num_pages + 7, -100]))
    rep = da.check_cache(pool, pool, torch.tensor(lens_h, dtype=torch.int32, device=DEV),
                         page_table=torch.from_numpy(table).to(DEV),
                         page_size=page_size).cpu().tolist()
    want = expected(lens_h, max_pages * page_size, table, num_pages, page_size)
    assert rep == want
    assert want[1] > 0 and want[0] >= 1 and want[2] == 0
