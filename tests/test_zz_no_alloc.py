"""GPU test of gqa_decode_attn_noalloc, the entry point that allocates
nothing: its split partials live in the library's static per-device scratch.
Its outputs must equal gqa_decode_attn's (the same kernels and split plan, so
bit for bit) and the oracle's within the attention tolerance, on two calls in
a row, the second with a smaller input."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from decode_attention_folded_amd import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL = 2e-3


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


@pytest.fixture(scope="module")
def da():
    import decode_attention_folded_amd as pkg
    pkg.load_library()
    return pkg


def _noalloc_c(da, q, k, v, seqlens, out, k_new=None, v_new=None, page_table=None,
               page_size=0, num_splits=0):
    """Call the C ABI directly (ctypes), no binding logic in between."""
    from decode_attention_folded_amd import _binding
    lib = da.load_library()
    desc = _binding._kv_desc(k, v, q.shape[0], page_table, page_size)
    P = ctypes.c_void_p
    st = lib.gqa_decode_attn_noalloc(
        P(q.data_ptr()), ctypes.byref(desc), P(seqlens.data_ptr()), q.shape[1],
        1.0 / np.sqrt(q.shape[2]), P(k_new.data_ptr()) if k_new is not None else None,
        P(v_new.data_ptr()) if v_new is not None else None, P(out.data_ptr()), num_splits,
        P(torch.cuda.current_stream().cuda_stream))
    return st


def _both(da, case, with_new, paged=False):
    """(noalloc output, gqa_decode_attn output) on the same inputs; each call
    gets its own copy of the cache (the append writes it)."""
    outs = []
    for use_noalloc in (True, False):
        q, k, v, ln = dev(case.q), dev(case.k), dev(case.v), dev(case.seqlens)
        kn = dev(case.k_new) if with_new else None
        vn = dev(case.v_new) if with_new else None
        pt = dev(case.page_table) if paged else None
        ps = case.page_size if paged else 0
        out = torch.full_like(q, float("nan"))
        if use_noalloc:
            assert _noalloc_c(da, q, k, v, ln, out, kn, vn, pt, ps) == 0
        else:
            da.gqa_decode_attn(q, k, v, ln, k_new=kn, v_new=vn, page_table=pt, page_size=ps,
                               out=out)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()))
    return outs


def test_noalloc_matches_workspace_entry_point_twice_then_smaller(da):
    # first call: 4 sequences, 8 KV heads, G = 4, D = 128, up to 6000 keys
    # (several splits per unit, ragged last tile), with the step's append
    big = workloads.dense_case(1701, 4, 32, 8, 128, 6000, [6000, 4097, 1, 2500], with_new=True)
    (a, ka, va), (b, kb, vb) = _both(da, big, with_new=True)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(ka.view(np.uint16), kb.view(np.uint16))
    k2, v2 = oracle.append_kv(big.k, big.v, big.seqlens, big.k_new, big.v_new)
    want = oracle.decode_attention(big.q, k2, v2, big.seqlens, big.scale)
    assert np.max(np.abs(a.astype(np.float64) - want)) <= ATOL
    # second call right after, smaller: 1 sequence, 2 KV heads, D = 64, 300
    # keys; the scratch still holds the first call's partials
    small = workloads.dense_case(1702, 1, 8, 2, 64, 300, [300])
    (a, _, _), (b, _, _) = _both(da, small, with_new=False)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    want = oracle.decode_attention(small.q, small.k, small.v, small.seqlens, small.scale)
    assert np.max(np.abs(a.astype(np.float64) - want)) <= ATOL


def test_noalloc_paged_cache(da):
    case = workloads.paged_case(1703, 3, 16, 4, 128, 16, 160, [2500, 17, 900])
    (a, _, _), (b, _, _) = _both(da, case, with_new=False, paged=True)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    kc = oracle.gather_paged(case.k, case.page_table, 16, case.capacity)
    vc = oracle.gather_paged(case.v, case.page_table, 16, case.capacity)
    want = oracle.decode_attention(case.q, kc, vc, case.seqlens, case.scale)
    assert np.max(np.abs(a.astype(np.float64) - want)) <= ATOL


def test_noalloc_rejects_a_call_too_large_for_the_scratch(da):
    """A request whose partials exceed the scratch fails before anything is
    enqueued (the output is left untouched)."""
    from decode_attention_folded_amd._binding import DecodeAttnError
    q = torch.zeros((64, 32, 128), dtype=torch.float16, device=DEV)
    # a cache view that is never read: 64 x 8 KV heads x 2^20 slots would be
    # 256 GiB, so use a one-slot cache and ask for 2^20 slots through the
    # C ABI's capacity alone
    from decode_attention_folded_amd import _binding
    lib = da.load_library()
    k = torch.zeros((64, 8, 16, 128), dtype=torch.float16, device=DEV)
    desc = _binding._kv_desc(k, k, 64, None, 0)
    desc.capacity = 1 << 20
    out = torch.full_like(q, 7.0)
    ln = torch.ones(64, dtype=torch.int32, device=DEV)
    P = ctypes.c_void_p
    st = lib.gqa_decode_attn_noalloc(P(q.data_ptr()), ctypes.byref(desc), P(ln.data_ptr()), 32,
                                     0.1, None, None, P(out.data_ptr()), 0, None)
    torch.cuda.synchronize()
    assert st == -7
    assert torch.all(out == 7.0)
    with pytest.raises(DecodeAttnError, match="DA_ERR_TOO_LARGE"):
        _binding._check(st, "gqa_decode_attn_noalloc")
