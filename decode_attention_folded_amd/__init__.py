"""Folded-GQA decode attention and Quest sparse decode for AMD MI355X (gfx950).

The compute lives in ``libdecode_attn.so`` (hand-written HIP kernels behind a
C ABI declared in ``include/decode_attn.h``).  This package is the thin Python
binding over it: argument marshalling only.  Importing the package is cheap;
the first use of an entry point loads the shared library and raises
``ImportError`` if it has not been built (there is no CPU fallback).

Entry points (same names as the C ABI):

* :func:`gqa_decode_attn`          -- folded decode attention, dense or paged
* :func:`gqa_decode_attn_noalloc`  -- the same with no workspace (library scratch)
* :func:`gqa_decode_attn_multi`    -- the fold for q_len > 1 queries (causal alignment)
* :func:`quest_meta_append`        -- per-page Key min/max metadata update
* :func:`quest_page_score_topk`    -- page scores and top-K page selection
* :func:`quest_append_score_topk`  -- the step's append fused into scoring + top-K
* :func:`quest_sparse_decode_attn` -- attention over the selected pages
* :func:`quest_select_sparse_decode_attn` -- top-K fused into that attention
* :func:`gqa_repeat_kv`            -- the materialised repeat_kv copy (A/B baseline)
* :func:`read_calibration`         -- streaming-read calibration (measurement helper)
* :func:`check_cache`              -- reports lengths and page-table entries the calls
                                      would clamp or mask (debugging aid)
"""

_EXPORTS = (
    "gqa_decode_attn",
    "gqa_decode_attn_noalloc",
    "gqa_decode_attn_multi",
    "quest_meta_append",
    "quest_page_score_topk",
    "quest_append_score_topk",
    "quest_sparse_decode_attn",
    "quest_select_sparse_decode_attn",
    "gqa_repeat_kv",
    "read_calibration",
    "check_cache",
    "workspace_bytes",
    "quest_workspace_bytes",
    "Workspace",
    "DecodeAttnError",
    "library_path",
    "load_library",
)


def __getattr__(name):
    if name in _EXPORTS:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)


__all__ = list(_EXPORTS)
