"""CPU tests of the C ABI boundary: the library loads, exports every function
include/decode_attn.h declares, and rejects bad arguments with the documented
status codes before touching the GPU.  No computation runs here."""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attn.h")


@pytest.fixture(scope="module")
def lib():
    from decode_attention_folded_amd import _binding
    if not os.path.exists(_binding.library_path()):
        from decode_attention_folded_amd import build
        build.build(verbose=False)
    return _binding.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_entry_points():
    names = _declared_functions()
    for n in ("gqa_decode_attn", "quest_meta_append", "quest_page_score_topk",
              "quest_sparse_decode_attn"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from decode_attention_folded_amd import _binding
    names = _declared_functions()
    assert set(names) == set(_binding.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_every_entry_point_has_declared_argument_types(lib):
    """ctypes must know every argument type (size_t and float arguments are
    passed wrongly without them)."""
    from decode_attention_folded_amd import _binding
    for n in _binding.EXPORTED_SYMBOLS:
        assert getattr(lib, n).argtypes is not None, n


def test_multi_query_validation_codes(lib):
    P = ctypes.c_void_p
    d = _desc()

    def call(hq=32, q_len=2, desc=d, q=FAKE, out=FAKE, ws_bytes=1 << 30):
        return lib.gqa_decode_attn_multi(P(q), ctypes.byref(desc), P(FAKE), hq, q_len, 0.125,
                                         P(out), P(FAKE), ws_bytes, 0, None)
    assert call(q_len=0) == -2
    assert call(hq=30) == -2
    assert call(q_len=3) == -3          # G * q_len = 12
    assert call(hq=64, q_len=2) == -3   # G * q_len = 16
    assert call(q=0) == -1
    assert call(ws_bytes=16) == -5
    assert call(desc=_desc(batch=0), q=0, out=0) == 0


def test_read_calibration_validation_codes(lib):
    P = ctypes.c_void_p
    assert lib.da_read_calibration(P(0), 1 << 20, P(FAKE), None) == -1
    assert lib.da_read_calibration(P(FAKE), 1 << 20, P(0), None) == -1
    assert lib.da_read_calibration(P(FAKE), 0, P(FAKE), None) == -2
    assert lib.da_read_calibration(P(FAKE), 1000, P(FAKE), None) == -2
    assert lib.da_read_calibration(P(FAKE + 8), 1 << 20, P(FAKE), None) == -2


def test_select_sparse_validation_codes(lib):
    P = ctypes.c_void_p

    def call(desc=None, scores=FAKE, meta_pages=256, budget=256, hq=32, idx=None, out=FAKE,
             ws_bytes=1 << 30):
        desc = desc if desc is not None else _desc()
        return lib.quest_select_sparse_decode_attn(P(FAKE), ctypes.byref(desc), P(FAKE),
                                                   P(scores) if scores else None, meta_pages,
                                                   budget, hq, 0.125, P(idx) if idx else None,
                                                   P(out) if out else None, P(FAKE), ws_bytes, 0,
                                                   None)
    assert call(scores=0) == -1                                # page scores required
    assert call(out=0) == -1
    assert call(budget=100) == -4                              # not a multiple of S
    assert call(budget=0) == -4
    assert call(meta_pages=255) == -2                          # 255 * 16 < capacity 4096
    assert call(meta_pages=0) == -2
    # > 16384 pages per unit: streaming top-K, then attention (no device here)
    assert call(desc=_desc(capacity=1 << 20), meta_pages=1 << 16) == -6
    assert call(desc=_desc(page_size=12)) == -3
    assert call(hq=30) == -2
    assert call(ws_bytes=16) == -5
    assert call(desc=_desc(batch=0), scores=0, out=0) == 0     # nothing to do


def test_status_strings(lib):
    for code in range(0, -8, -1):
        s = lib.da_status_string(code).decode()
        assert s.startswith("DA_")
    assert lib.da_status_string(-99) == b"unknown status"


FAKE = 1 << 20  # an aligned, never-dereferenced address: every call below fails validation


def _desc(**kw):
    from decode_attention_folded_amd._binding import KVCacheDesc
    d = KVCacheDesc()
    d.k, d.v, d.page_table = FAKE, FAKE, None
    d.batch, d.num_kv_heads, d.head_dim, d.capacity = 2, 8, 128, 4096
    d.page_size, d.max_pages, d.num_pages = 16, 0, 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _attn(lib, desc, hq=32, ws_bytes=1 << 30, q=FAKE, seqlens=FAKE, out=FAKE, ws=FAKE,
          k_new=None, v_new=None, splits=0, scale=0.125):
    P = ctypes.c_void_p
    return lib.gqa_decode_attn(P(q), ctypes.byref(desc), P(seqlens), hq, scale,
                               P(k_new) if k_new else None, P(v_new) if v_new else None,
                               P(out), P(ws), ws_bytes, splits, None)


def test_validation_codes(lib):
    assert _attn(lib, _desc(), q=0) == -1
    assert _attn(lib, _desc(), out=0) == -1
    assert _attn(lib, _desc(k=0)) == -1
    assert _attn(lib, _desc(), k_new=FAKE) == -1             # k_new without v_new
    assert _attn(lib, _desc(), hq=30) == -2                  # Hq % Hkv != 0
    assert _attn(lib, _desc(), hq=8 * 16) == -3              # G = 16
    assert _attn(lib, _desc(head_dim=96)) == -3
    assert _attn(lib, _desc(capacity=0)) == -2
    assert _attn(lib, _desc(), q=FAKE + 2) == -2              # misaligned
    assert _attn(lib, _desc(), scale=float("nan")) == -2
    assert _attn(lib, _desc(), ws_bytes=16) == -5
    assert _attn(lib, _desc(page_table=FAKE, page_size=12, max_pages=4, num_pages=8)) == -3
    assert _attn(lib, _desc(page_table=FAKE, page_size=16, max_pages=0, num_pages=8)) == -2
    assert lib.gqa_decode_attn(None, None, None, 32, 1.0, None, None, None, None, 0, 0,
                               None) == -1


def test_quest_validation_codes(lib):
    P = ctypes.c_void_p
    # budget not a multiple of S, K < 1
    for budget, want in ((100, -4), (0, -4), (-16, -4)):
        st = lib.quest_page_score_topk(P(FAKE), P(FAKE), 256, P(FAKE), 1, 32, 8, 128, 16,
                                       budget, P(FAKE), P(FAKE), None, 0, None)
        assert st == want
    st = lib.quest_page_score_topk(P(FAKE), P(FAKE), 256, P(FAKE), 1, 32, 8, 128, 12, 48,
                                   P(FAKE), P(FAKE), None, 0, None)
    assert st == -3                                            # S = 12
    st = lib.quest_page_score_topk(P(FAKE), P(FAKE), 1 << 15, P(FAKE), 1, 32, 8, 128, 16, 256,
                                   P(FAKE), P(FAKE), None, 0, None)
    assert st == -6                    # 32768 pages: streaming top-K, no device here
    st = lib.quest_page_score_topk(P(FAKE), P(FAKE), 256, P(FAKE), 1, 32, 8, 128, 16, 256,
                                   P(FAKE), None, P(FAKE), 16, None)
    assert st == -5                                            # score workspace too small
    d = _desc()
    st = lib.quest_sparse_decode_attn(P(FAKE), ctypes.byref(d), P(FAKE), P(FAKE), 100, 32,
                                      0.1, P(FAKE), P(FAKE), 1 << 30, 0, None)
    assert st == -4
    st = lib.quest_sparse_decode_attn(P(FAKE), ctypes.byref(d), P(FAKE), None, 256, 32,
                                      0.1, P(FAKE), P(FAKE), 1 << 30, 0, None)
    assert st == -1
    # metadata: k_new requires n_new == 1; too few metadata pages
    st = lib.quest_meta_append(ctypes.byref(d), P(FAKE), 256, P(FAKE), 2, P(FAKE), P(FAKE),
                               None)
    assert st == -2
    st = lib.quest_meta_append(ctypes.byref(d), P(FAKE), 255, P(FAKE), 1, None, None, None)
    assert st == -2
    st = lib.quest_meta_append(ctypes.byref(_desc(page_size=24)), P(FAKE), 256, P(FAKE), 1,
                               None, None, None)
    assert st == -3


def test_repeat_kv_validation_codes(lib):
    P = ctypes.c_void_p
    d = _desc()
    assert lib.gqa_repeat_kv(ctypes.byref(d), 32, P(FAKE), None, P(FAKE), None) == -1
    assert lib.gqa_repeat_kv(ctypes.byref(d), 32, None, P(FAKE), P(FAKE), None) == -1
    assert lib.gqa_repeat_kv(ctypes.byref(d), 8 * 16, P(FAKE), P(FAKE), P(FAKE), None) == -3
    assert lib.gqa_repeat_kv(ctypes.byref(d), 30, P(FAKE), P(FAKE), P(FAKE), None) == -2
    assert lib.gqa_repeat_kv(ctypes.byref(d), 32, P(FAKE), P(FAKE + 4), P(FAKE), None) == -2
    assert lib.gqa_repeat_kv(ctypes.byref(_desc(batch=0)), 32, None, None, None, None) == 0
    assert lib.gqa_repeat_kv(None, 32, P(FAKE), P(FAKE), P(FAKE), None) == -1


def test_workspace_sizes(lib):
    def size(desc, hq=32, budget=0, splits=0):
        out = ctypes.c_size_t()
        st = lib.da_workspace_size(ctypes.byref(desc), hq, budget, splits, ctypes.byref(out))
        assert st == 0
        return out.value
    small = size(_desc(batch=1))
    big = size(_desc(batch=8))
    assert 0 < small <= big
    # the selected-page stream: fewer partials, plus room for the choice
    d = _desc()
    choice = d.batch * d.num_kv_heads * (2048 // d.page_size) * 4
    assert size(_desc(), budget=2048) <= size(_desc()) + choice
    assert size(_desc(), splits=1) < size(_desc(), splits=64)
    out = ctypes.c_size_t()
    assert lib.da_quest_workspace_size(8, 8, 8192, ctypes.byref(out)) == 0
    assert out.value >= 8 * 8 * 8192 * 4


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_no_device_reports_hip_error(lib):
    # arguments pass validation; the launch itself finds no device
    assert _attn(lib, _desc(batch=1)) == -6


def test_zero_batch_is_a_no_op(lib):
    assert _attn(lib, _desc(batch=0)) == 0


def test_binding_rejects_host_tensors():
    import decode_attention_folded_amd as da
    q = torch.zeros(1, 32, 64, dtype=torch.float16)
    k = torch.zeros(1, 8, 16, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        da.gqa_decode_attn(q, k, k, torch.ones(1, dtype=torch.int32))


def test_product_path_never_uses_the_oracle():
    pkg = os.path.join(ROOT, "decode_attention_folded_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle." not in text, f


def _planned_splits(units, max_keys, page_list, num_splits=0):
    """The split plan as documented: 16-key tiles; without an explicit count,
    chunks of at least 8 tiles sized for about 256 workgroups, at most 160
    tiles when the chunk reads a page list and 512 otherwise."""
    tiles = max(1, -(-max_keys // 16))
    if num_splits > 0:
        tps = -(-tiles // num_splits)
    else:
        tps = max(-(-(units * tiles) // 256), 8)
    tps = min(max(tps, 1), 160 if page_list else 512, tiles)
    return -(-tiles // tps)


def _plan_bytes(units, splits, rows, d, k_sel=0):
    """The work counter's 256 bytes, then the partials (m, l) and o; with a
    page budget also the choice, K int32 per unit, after the 256-byte aligned
    partials."""
    ml = -(-(units * splits * rows * 2 * 4) // 256) * 256
    o = units * splits * rows * d * 4
    if k_sel == 0:
        return 256 + ml + o
    return 256 + ml + -(-o // 256) * 256 + units * k_sel * 4


# (desc fields, Hq, budget tokens, explicit splits, page list, longest key stream, splits)
PLAN_CASES = [
    (dict(batch=1, num_kv_heads=8, head_dim=64, capacity=4096), 32, 0, 0, False, 4096, 32),
    (dict(batch=8, num_kv_heads=8, head_dim=128, capacity=131072), 32, 0, 0, False, 131072, 16),
    (dict(batch=64, num_kv_heads=8, head_dim=128, page_table=FAKE, page_size=16, max_pages=2048,
          num_pages=70000), 32, 0, 0, True, 32768, 13),
    (dict(batch=8, num_kv_heads=8, head_dim=128, capacity=131072), 32, 4096, 0, True, 4096, 4),
    (dict(batch=1, num_kv_heads=32, head_dim=128, capacity=32768), 32, 2048, 0, True, 2048, 8),
    (dict(batch=2, num_kv_heads=8, head_dim=128, capacity=4096), 32, 0, 7, False, 4096, 7),
    (dict(batch=2, num_kv_heads=8, head_dim=64, capacity=1000, page_size=16), 32, 4096, 0, True,
     1008, 8),
]


@pytest.mark.parametrize("fields,hq,budget,splits,page_list,max_keys,want_splits", PLAN_CASES)
def test_workspace_follows_the_split_plan(lib, fields, hq, budget, splits, page_list, max_keys,
                                          want_splits):
    desc = _desc(**fields)
    units = desc.batch * desc.num_kv_heads
    got_splits = _planned_splits(units, max_keys, page_list, splits)
    assert got_splits == want_splits  # the rule itself, on the workloads' shapes
    out = ctypes.c_size_t()
    assert lib.da_workspace_size(ctypes.byref(desc), hq, budget, splits, ctypes.byref(out)) == 0
    k_sel = budget // desc.page_size if budget else 0
    assert out.value == _plan_bytes(units, want_splits, hq // desc.num_kv_heads, desc.head_dim,
                                    k_sel)


def _noalloc(lib, desc, hq=32, q=FAKE, seqlens=FAKE, out=FAKE, splits=0):
    P = ctypes.c_void_p
    return lib.gqa_decode_attn_noalloc(P(q), ctypes.byref(desc), P(seqlens), hq, 0.125, None,
                                       None, P(out), splits, None)


def test_noalloc_validation_codes(lib):
    """The entry point without a workspace checks its arguments, then the size
    of its split partials against the library's static scratch, before any
    HIP call."""
    assert _noalloc(lib, _desc(), q=0) == -1
    assert _noalloc(lib, _desc(), out=0) == -1
    assert _noalloc(lib, _desc(), hq=30) == -2
    assert _noalloc(lib, _desc(batch=0), q=0, out=0) == 0
    # 64 sequences x 8 KV heads x 2^20 keys: 128 splits of fp32 partials per
    # unit, far beyond 32 MiB
    huge = _desc(batch=64, capacity=1 << 20)
    size = ctypes.c_size_t()
    assert lib.da_workspace_size(ctypes.byref(huge), 32, 0, 0, ctypes.byref(size)) == 0
    assert size.value > (32 << 20)
    assert _noalloc(lib, huge) == -7
    assert b"DA_ERR_TOO_LARGE" in lib.da_status_string(-7)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_noalloc_without_a_device_reports_hip_error(lib):
    assert _noalloc(lib, _desc(batch=1)) == -6
