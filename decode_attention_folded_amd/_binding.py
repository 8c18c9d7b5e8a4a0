"""ctypes binding of libdecode_attn.so: argument marshalling only.

Every computation happens in the library's HIP kernels.  This module turns
torch tensors (device memory and the current stream are the only things torch
provides here) into the pointers and sizes of the C ABI in
``include/decode_attn.h`` and raises :class:`DecodeAttnError` on a non-zero
status.  If the shared library has not been built, loading it raises
``ImportError``; there is no fallback implementation.
"""

import ctypes
import math
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_LOCK = threading.Lock()

DA_OK = 0
STATUS_NAMES = {
    0: "DA_OK", -1: "DA_ERR_NULL", -2: "DA_ERR_SHAPE", -3: "DA_ERR_UNSUPPORTED",
    -4: "DA_ERR_BUDGET", -5: "DA_ERR_WORKSPACE", -6: "DA_ERR_HIP", -7: "DA_ERR_TOO_LARGE",
}

# bytes of the library's static per-device scratch (DA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTED_SYMBOLS = (
    "da_status_string", "da_workspace_size", "gqa_decode_attn", "quest_meta_append",
    "da_quest_workspace_size", "quest_page_score_topk", "quest_sparse_decode_attn",
    "gqa_repeat_kv", "quest_append_score_topk", "gqa_decode_attn_multi", "da_read_calibration",
    "quest_select_sparse_decode_attn", "gqa_decode_attn_noalloc", "da_check_cache",
)


class DecodeAttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = load_library().da_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


class KVCacheDesc(ctypes.Structure):
    """Mirror of ``da_kv_cache``."""
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
    ]


def library_path():
    return os.environ.get("DECODE_ATTN_LIB", os.path.join(_PKG, "libdecode_attn.so"))


def load_library():
    """Load (once) and return the ctypes handle of libdecode_attn.so."""
    global _LIB
    if _LIB is not None:
        return _LIB
    with _LOCK:
        if _LIB is not None:
            return _LIB
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is not built; run `python -m decode_attention_folded_amd.build` "
                "(there is no CPU fallback for the decode-attention kernels)")
        lib = ctypes.CDLL(path)
        P, I32, I64, SZ, F32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_size_t, ctypes.c_float)
        KVP = ctypes.POINTER(KVCacheDesc)
        SZP = ctypes.POINTER(ctypes.c_size_t)
        lib.da_status_string.argtypes = [ctypes.c_int]
        lib.da_status_string.restype = ctypes.c_char_p
        lib.da_workspace_size.argtypes = [KVP, I32, I32, I32, SZP]
        lib.gqa_decode_attn.argtypes = [P, KVP, P, I32, F32, P, P, P, P, SZ, I32, P]
        lib.gqa_decode_attn_noalloc.argtypes = [P, KVP, P, I32, F32, P, P, P, I32, P]
        lib.quest_meta_append.argtypes = [KVP, P, I32, P, I32, P, P, P]
        lib.da_quest_workspace_size.argtypes = [I32, I32, I32, SZP]
        lib.quest_page_score_topk.argtypes = [P, P, I32, P, I32, I32, I32, I32, I32, I32, P, P,
                                              P, SZ, P]
        lib.quest_sparse_decode_attn.argtypes = [P, KVP, P, P, I32, I32, F32, P, P, SZ, I32, P]
        lib.gqa_decode_attn_multi.argtypes = [P, KVP, P, I32, I32, F32, P, P, SZ, I32, P]
        lib.gqa_repeat_kv.argtypes = [KVP, I32, P, P, P, P]
        lib.quest_append_score_topk.argtypes = [P, KVP, P, I32, P, I32, I32, P, P, P, P, P, SZ,
                                                P]
        lib.da_read_calibration.argtypes = [P, SZ, P, P]
        lib.da_check_cache.argtypes = [KVP, P, P, P]
        lib.quest_select_sparse_decode_attn.argtypes = [P, KVP, P, P, I32, I32, I32, F32, P, P,
                                                        P, SZ, I32, P]
        for name in EXPORTED_SYMBOLS[1:]:
            getattr(lib, name).restype = ctypes.c_int
        _LIB = lib
        return lib


def _check(status, where):
    if status != DA_OK:
        raise DecodeAttnError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def _kv_desc(k_cache, v_cache, batch, page_table, page_size):
    _need(k_cache, "k_cache", torch.float16, 4)
    _need(v_cache, "v_cache", torch.float16, 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    desc = KVCacheDesc()
    desc.k = k_cache.data_ptr()
    desc.v = v_cache.data_ptr()
    desc.batch = batch
    desc.head_dim = k_cache.shape[3]
    desc.page_size = int(page_size)
    if page_table is None:
        if k_cache.shape[0] != batch:
            raise ValueError("contiguous cache batch does not match q")
        desc.page_table = None
        desc.num_kv_heads = k_cache.shape[1]
        desc.capacity = k_cache.shape[2]
        desc.max_pages = 0
        desc.num_pages = 0
    else:
        _need(page_table, "page_table", torch.int32, 2)
        if page_table.shape[0] != batch:
            raise ValueError("page_table batch does not match q")
        if k_cache.shape[2] != page_size:
            raise ValueError("paged pool is [num_pages, Hkv, page_size, D]")
        desc.page_table = page_table.data_ptr()
        desc.num_kv_heads = k_cache.shape[1]
        desc.capacity = page_table.shape[1] * page_size
        desc.max_pages = page_table.shape[1]
        desc.num_pages = k_cache.shape[0]
    return desc


def _check_common(q, seqlens, desc):
    if seqlens.shape[0] != q.shape[0]:
        raise ValueError("seqlens must be [B]")
    if q.shape[2] != desc.head_dim:
        raise ValueError("q and the cache disagree on head_dim")
    if q.device != seqlens.device:
        raise ValueError("q and seqlens are on different devices")


def _out_like(q, out):
    if out is None:
        return torch.empty_like(q)
    _need(out, "out", torch.float16, 3)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape [B, Hq, D]")
    return out


class Workspace:
    """A device scratch buffer that grows on demand.  It holds only per-call
    partial results, so one workspace serves any number of calls issued in
    order on one stream.  Calls that may run concurrently (on different
    streams) need different workspaces; the default workspaces below are kept
    per stream for that reason."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes, device, stream=None):
        """A buffer of at least `nbytes`.  A new buffer is allocated on
        `stream` (default: the current stream), so the caching allocator
        recycles a replaced buffer only in that stream's order."""
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = None
            if stream is None:
                self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
            else:
                with torch.cuda.stream(stream):
                    self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


_DEFAULT_WS = {}


def _workspace(ws, device, kind="attn", stream=None):
    # The attention calls share one default workspace per device and stream;
    # page scores get their own, so a score buffer is never overwritten by a
    # later attention call.  A caller-supplied workspace is used as given.
    if ws is None:
        s = stream if stream is not None else torch.cuda.current_stream(device)
        key = (kind, device.type, device.index, s.cuda_stream)
        ws = _DEFAULT_WS.setdefault(key, Workspace(device))
    return ws


def workspace_bytes(k_cache, v_cache, batch, num_q_heads, *, page_table=None, page_size=0,
                    budget_tokens=0, num_splits=0):
    lib = load_library()
    desc = _kv_desc(k_cache, v_cache, batch, page_table, page_size)
    out = ctypes.c_size_t()
    _check(lib.da_workspace_size(ctypes.byref(desc), num_q_heads, budget_tokens, num_splits,
                                 ctypes.byref(out)), "da_workspace_size")
    return out.value


def quest_workspace_bytes(batch, num_kv_heads, meta_max_pages):
    out = ctypes.c_size_t()
    _check(load_library().da_quest_workspace_size(batch, num_kv_heads, meta_max_pages,
                                                  ctypes.byref(out)), "da_quest_workspace_size")
    return out.value


def gqa_decode_attn(q, k_cache, v_cache, seqlens, *, scale=None, k_new=None, v_new=None,
                    page_table=None, page_size=0, out=None, workspace=None, num_splits=0,
                    stream=None):
    """Folded GQA decode attention (see ``gqa_decode_attn`` in decode_attn.h).

    q [B, Hq, D] fp16; k_cache/v_cache [B, Hkv, cap, D] fp16 (or a paged pool
    [NP, Hkv, S, D] with page_table [B, max_pages] int32); seqlens [B] int32
    on the device.  Returns out [B, Hq, D] fp16."""
    lib = load_library()
    _need(q, "q", torch.float16, 3)
    _need(seqlens, "seqlens", torch.int32, 1)
    batch, hq, d = q.shape
    desc = _kv_desc(k_cache, v_cache, batch, page_table, page_size)
    _check_common(q, seqlens, desc)
    if k_new is not None or v_new is not None:
        _need(k_new, "k_new", torch.float16, 3)
        _need(v_new, "v_new", torch.float16, 3)
        for t, name in ((k_new, "k_new"), (v_new, "v_new")):
            if tuple(t.shape) != (batch, desc.num_kv_heads, d):
                raise ValueError(f"{name} must be [B, Hkv, D]")
    out = _out_like(q, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = ctypes.c_size_t()
    _check(lib.da_workspace_size(ctypes.byref(desc), hq, 0, num_splits, ctypes.byref(nbytes)),
           "da_workspace_size")
    ws = _workspace(workspace, q.device, stream=stream).get(nbytes.value, q.device, stream)
    _check(lib.gqa_decode_attn(_ptr(q), ctypes.byref(desc), _ptr(seqlens), hq, scale,
                               _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(ws), ws.numel(),
                               num_splits, _stream_handle(q.device, stream)),
           "gqa_decode_attn")
    return out


def gqa_decode_attn_noalloc(q, k_cache, v_cache, seqlens, out, *, scale=None, k_new=None,
                            v_new=None, page_table=None, page_size=0, num_splits=0, stream=None):
    """gqa_decode_attn without a workspace (see ``gqa_decode_attn_noalloc`` in
    decode_attn.h): the library call allocates nothing, its split partials
    live in the library's static per-device scratch.  ``out`` [B, Hq, D] fp16
    must be given (nothing is allocated here either).  Calls that may overlap
    on one GPU race on that scratch.  Returns ``out``."""
    lib = load_library()
    _need(q, "q", torch.float16, 3)
    _need(seqlens, "seqlens", torch.int32, 1)
    batch, hq, d = q.shape
    desc = _kv_desc(k_cache, v_cache, batch, page_table, page_size)
    _check_common(q, seqlens, desc)
    if k_new is not None or v_new is not None:
        _need(k_new, "k_new", torch.float16, 3)
        _need(v_new, "v_new", torch.float16, 3)
        for t, name in ((k_new, "k_new"), (v_new, "v_new")):
            if tuple(t.shape) != (batch, desc.num_kv_heads, d):
                raise ValueError(f"{name} must be [B, Hkv, D]")
    _need(out, "out", torch.float16, 3)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape [B, Hq, D]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib.gqa_decode_attn_noalloc(_ptr(q), ctypes.byref(desc), _ptr(seqlens), hq, scale,
                                       _ptr(k_new), _ptr(v_new), _ptr(out), num_splits,
                                       _stream_handle(q.device, stream)),
           "gqa_decode_attn_noalloc")
    return out


def gqa_decode_attn_multi(q, k_cache, v_cache, seqlens, *, scale=None, page_table=None,
                          page_size=0, out=None, workspace=None, num_splits=0, stream=None):
    """Folded GQA attention for q_len > 1 queries per head (see
    ``gqa_decode_attn_multi`` in decode_attn.h): q [B, Hq, q_len, D] fp16, the
    last q_len positions of each sequence, causally aligned.  Returns out
    [B, Hq, q_len, D] fp16."""
    lib = load_library()
    _need(q, "q", torch.float16, 4)
    _need(seqlens, "seqlens", torch.int32, 1)
    batch, hq, q_len, d = q.shape
    desc = _kv_desc(k_cache, v_cache, batch, page_table, page_size)
    if seqlens.shape[0] != batch:
        raise ValueError("seqlens must be [B]")
    if desc.head_dim != d:
        raise ValueError("q and the cache disagree on head_dim")
    if hq % desc.num_kv_heads != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.float16, 4)
    if out.shape != q.shape:
        raise ValueError("out must be [B, Hq, q_len, D]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = ctypes.c_size_t()
    _check(lib.da_workspace_size(ctypes.byref(desc), hq * q_len, 0, num_splits,
                                 ctypes.byref(nbytes)), "da_workspace_size")
    ws = _workspace(workspace, q.device, stream=stream).get(nbytes.value, q.device, stream)
    _check(lib.gqa_decode_attn_multi(_ptr(q), ctypes.byref(desc), _ptr(seqlens), hq, q_len,
                                     scale, _ptr(out), _ptr(ws), ws.numel(), num_splits,
                                     _stream_handle(q.device, stream)),
           "gqa_decode_attn_multi")
    return out


def gqa_repeat_kv(k_cache, v_cache, seqlens, num_q_heads, *, page_table=None, page_size=0,
                  k_out=None, v_out=None, stream=None):
    """Materialised repeat_kv (see ``gqa_repeat_kv`` in decode_attn.h): returns
    k_out, v_out [B, Hq, cap, D] fp16 whose rows t < L_b of head h are the rows
    of KV head h // G (other rows are left as allocated)."""
    lib = load_library()
    _need(seqlens, "seqlens", torch.int32, 1)
    batch = seqlens.shape[0]
    desc = _kv_desc(k_cache, v_cache, batch, page_table, page_size)
    shape = (batch, int(num_q_heads), desc.capacity, desc.head_dim)
    outs = []
    for t, name in ((k_out, "k_out"), (v_out, "v_out")):
        if t is None:
            t = torch.empty(shape, dtype=torch.float16, device=k_cache.device)
        _need(t, name, torch.float16, 4)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be [B, Hq, cap, D] = {shape}")
        outs.append(t)
    _check(lib.gqa_repeat_kv(ctypes.byref(desc), int(num_q_heads), _ptr(seqlens), _ptr(outs[0]),
                             _ptr(outs[1]), _stream_handle(k_cache.device, stream)),
           "gqa_repeat_kv")
    return outs[0], outs[1]


def read_calibration(buf, sink, stream=None):
    """Streaming-read calibration (``da_read_calibration``): reads every byte
    of the contiguous device tensor ``buf`` once; ``sink`` is a device tensor
    of at least 4 bytes.  A measurement helper: time it with events."""
    lib = load_library()
    for t, name in ((buf, "buf"), (sink, "sink")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    _check(lib.da_read_calibration(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                   _stream_handle(buf.device, stream)),
           "da_read_calibration")


def quest_meta_append(k_cache, v_cache, meta, seqlens, n_new=1, *, page_size, k_new=None,
                      v_new=None, page_table=None, stream=None):
    """Update Quest page metadata meta [B, Hkv, P, 2, D] fp16 in place."""
    lib = load_library()
    _need(meta, "meta", torch.float16, 5)
    _need(seqlens, "seqlens", torch.int32, 1)
    batch = seqlens.shape[0]
    desc = _kv_desc(k_cache, v_cache, batch, page_table, page_size)
    if tuple(meta.shape) != (batch, desc.num_kv_heads, meta.shape[2], 2, desc.head_dim):
        raise ValueError("meta must be [B, Hkv, P, 2, D]")
    if k_new is not None or v_new is not None:
        _need(k_new, "k_new", torch.float16, 3)
        _need(v_new, "v_new", torch.float16, 3)
        for t, name in ((k_new, "k_new"), (v_new, "v_new")):
            if tuple(t.shape) != (batch, desc.num_kv_heads, desc.head_dim):
                raise ValueError(f"{name} must be [B, Hkv, D]")
    _check(lib.quest_meta_append(ctypes.byref(desc), _ptr(meta), meta.shape[2], _ptr(seqlens),
                                 int(n_new), _ptr(k_new), _ptr(v_new),
                                 _stream_handle(meta.device, stream)),
           "quest_meta_append")
    return meta


def _page_idx_out(select, page_idx, page_scores, batch, hkv, budget_tokens, page_size, device):
    """The chosen-page output of a scoring call: a tensor (allocated if not
    given), or None for scores only (select=False)."""
    if not select:
        if page_scores is None:
            raise ValueError("select=False needs page_scores (the scores are the only output)")
        if page_idx is not None:
            raise ValueError("select=False writes no page_idx")
        return None
    k_pages = budget_tokens // page_size if page_size > 0 else 0
    if page_idx is None:
        return torch.empty((batch, hkv, max(k_pages, 1)), dtype=torch.int32, device=device)
    _need(page_idx, "page_idx", torch.int32, 3)
    if tuple(page_idx.shape) != (batch, hkv, k_pages):
        raise ValueError("page_idx must be [B, Hkv, budget_tokens / page_size]")
    return page_idx


def quest_page_score_topk(q, meta, seqlens, *, page_size, budget_tokens, page_idx=None,
                          page_scores=None, workspace=None, select=True, stream=None):
    """Page scores and top-K chosen pages.  Returns page_idx [B, Hkv, K]
    int32 (ascending, -1 padded); fills page_scores [B, Hkv, P] fp32 if
    given.  select=False: the scores only (page_scores required, returns
    None), for quest_select_sparse_decode_attn."""
    lib = load_library()
    _need(q, "q", torch.float16, 3)
    _need(meta, "meta", torch.float16, 5)
    _need(seqlens, "seqlens", torch.int32, 1)
    batch, hq, d = q.shape
    hkv, max_pages = meta.shape[1], meta.shape[2]
    if tuple(meta.shape) != (batch, hkv, max_pages, 2, d):
        raise ValueError("meta must be [B, Hkv, P, 2, D] matching q")
    if seqlens.shape[0] != batch:
        raise ValueError("seqlens must be [B]")
    page_idx = _page_idx_out(select, page_idx, page_scores, batch, hkv, budget_tokens,
                             page_size, q.device)
    ws = None
    if page_scores is None:
        ws = _workspace(workspace, q.device, "scores", stream).get(
            quest_workspace_bytes(batch, hkv, max_pages), q.device, stream)
    else:
        _need(page_scores, "page_scores", torch.float32, 3)
        if tuple(page_scores.shape) != (batch, hkv, max_pages):
            raise ValueError("page_scores must be [B, Hkv, P]")
    _check(lib.quest_page_score_topk(_ptr(q), _ptr(meta), max_pages, _ptr(seqlens), batch, hq,
                                     hkv, d, page_size, budget_tokens, _ptr(page_idx),
                                     _ptr(page_scores), _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream_handle(q.device, stream)),
           "quest_page_score_topk")
    return page_idx


def quest_append_score_topk(q, k_cache, v_cache, meta, seqlens, k_new, v_new, *, page_size,
                            budget_tokens, page_table=None, page_idx=None, page_scores=None,
                            workspace=None, select=True, stream=None):
    """One decode step's K/V row append and metadata update fused into page
    scoring and top-K (see ``quest_append_score_topk`` in decode_attn.h).
    Updates the cache and meta in place; returns page_idx [B, Hkv, K] int32
    (select=False: the append and the scores only; page_scores required,
    returns None)."""
    lib = load_library()
    _need(q, "q", torch.float16, 3)
    _need(meta, "meta", torch.float16, 5)
    _need(seqlens, "seqlens", torch.int32, 1)
    batch, hq, d = q.shape
    desc = _kv_desc(k_cache, v_cache, batch, page_table, page_size)
    _check_common(q, seqlens, desc)
    if tuple(meta.shape) != (batch, desc.num_kv_heads, meta.shape[2], 2, d):
        raise ValueError("meta must be [B, Hkv, P, 2, D]")
    _need(k_new, "k_new", torch.float16, 3)
    _need(v_new, "v_new", torch.float16, 3)
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if tuple(t.shape) != (batch, desc.num_kv_heads, d):
            raise ValueError(f"{name} must be [B, Hkv, D]")
    hkv, max_pages = desc.num_kv_heads, meta.shape[2]
    page_idx = _page_idx_out(select, page_idx, page_scores, batch, hkv, budget_tokens,
                             page_size, q.device)
    ws = None
    if page_scores is None:
        ws = _workspace(workspace, q.device, "scores", stream).get(
            quest_workspace_bytes(batch, hkv, max_pages), q.device, stream)
    else:
        _need(page_scores, "page_scores", torch.float32, 3)
        if tuple(page_scores.shape) != (batch, hkv, max_pages):
            raise ValueError("page_scores must be [B, Hkv, P]")
    _check(lib.quest_append_score_topk(_ptr(q), ctypes.byref(desc), _ptr(meta), max_pages,
                                       _ptr(seqlens), hq, int(budget_tokens), _ptr(k_new),
                                       _ptr(v_new), _ptr(page_idx), _ptr(page_scores), _ptr(ws),
                                       0 if ws is None else ws.numel(),
                                       _stream_handle(q.device, stream)),
           "quest_append_score_topk")
    return page_idx


def quest_sparse_decode_attn(q, k_cache, v_cache, seqlens, page_idx, *, budget_tokens,
                             page_size, scale=None, page_table=None, out=None, workspace=None,
                             num_splits=0, stream=None):
    """Attention over the chosen pages only.  Returns out [B, Hq, D] fp16."""
    lib = load_library()
    _need(q, "q", torch.float16, 3)
    _need(seqlens, "seqlens", torch.int32, 1)
    _need(page_idx, "page_idx", torch.int32, 3)
    batch, hq, d = q.shape
    desc = _kv_desc(k_cache, v_cache, batch, page_table, page_size)
    _check_common(q, seqlens, desc)
    if page_size > 0 and tuple(page_idx.shape) != (batch, desc.num_kv_heads,
                                                   budget_tokens // page_size):
        raise ValueError("page_idx must be [B, Hkv, budget_tokens / page_size]")
    out = _out_like(q, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = ctypes.c_size_t()
    _check(lib.da_workspace_size(ctypes.byref(desc), hq, budget_tokens, num_splits,
                                 ctypes.byref(nbytes)), "da_workspace_size")
    ws = _workspace(workspace, q.device, stream=stream).get(nbytes.value, q.device, stream)
    _check(lib.quest_sparse_decode_attn(_ptr(q), ctypes.byref(desc), _ptr(seqlens),
                                        _ptr(page_idx), budget_tokens, hq, scale, _ptr(out),
                                        _ptr(ws), ws.numel(), num_splits,
                                        _stream_handle(q.device, stream)),
           "quest_sparse_decode_attn")
    return out


def quest_select_sparse_decode_attn(q, k_cache, v_cache, seqlens, page_scores, *, budget_tokens,
                                    page_size, scale=None, page_table=None, page_idx=None,
                                    out=None, workspace=None, num_splits=0, stream=None):
    """Top-K page selection from page_scores [B, Hkv, P] fp32 fused into the
    attention over the chosen pages (see ``quest_select_sparse_decode_attn`` in
    decode_attn.h).  Returns out [B, Hq, D] fp16; fills page_idx [B, Hkv, K]
    int32 with the choice if given."""
    lib = load_library()
    _need(q, "q", torch.float16, 3)
    _need(seqlens, "seqlens", torch.int32, 1)
    _need(page_scores, "page_scores", torch.float32, 3)
    batch, hq, d = q.shape
    desc = _kv_desc(k_cache, v_cache, batch, page_table, page_size)
    _check_common(q, seqlens, desc)
    if tuple(page_scores.shape[:2]) != (batch, desc.num_kv_heads):
        raise ValueError("page_scores must be [B, Hkv, P]")
    if page_idx is not None:
        _need(page_idx, "page_idx", torch.int32, 3)
        if page_size > 0 and tuple(page_idx.shape) != (batch, desc.num_kv_heads,
                                                       budget_tokens // page_size):
            raise ValueError("page_idx must be [B, Hkv, budget_tokens / page_size]")
    out = _out_like(q, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = ctypes.c_size_t()
    _check(lib.da_workspace_size(ctypes.byref(desc), hq, budget_tokens, num_splits,
                                 ctypes.byref(nbytes)), "da_workspace_size")
    ws = _workspace(workspace, q.device, stream=stream).get(nbytes.value, q.device, stream)
    _check(lib.quest_select_sparse_decode_attn(_ptr(q), ctypes.byref(desc), _ptr(seqlens),
                                               _ptr(page_scores), page_scores.shape[2],
                                               budget_tokens, hq, scale, _ptr(page_idx),
                                               _ptr(out), _ptr(ws), ws.numel(), num_splits,
                                               _stream_handle(q.device, stream)),
           "quest_select_sparse_decode_attn")
    return out


def check_cache(k_cache, v_cache, seqlens, *, page_table=None, page_size=0, report=None,
                stream=None):
    """Device-side precondition check (see ``da_check_cache`` in decode_attn.h):
    returns report [4] int32 on the device -- sequences with a length outside
    [0, capacity], page-table entries of valid pages outside the pool, the
    lowest offending sequence index (-1 if none), 0."""
    lib = load_library()
    _need(seqlens, "seqlens", torch.int32, 1)
    desc = _kv_desc(k_cache, v_cache, seqlens.shape[0], page_table, page_size)
    if report is None:
        # no fill: the kernel writes all four entries (a fill on another
        # stream than the check's could land after it)
        report = torch.empty(4, dtype=torch.int32, device=seqlens.device)
    _need(report, "report", torch.int32, 1)
    if report.numel() < 4:
        raise ValueError("report must hold 4 int32")
    if seqlens.numel() == 0:  # nothing to check; the library writes nothing
        report.copy_(torch.tensor([0, 0, -1, 0], dtype=torch.int32))
        return report
    _check(lib.da_check_cache(ctypes.byref(desc), _ptr(seqlens), _ptr(report),
                              _stream_handle(seqlens.device, stream)), "da_check_cache")
    return report
