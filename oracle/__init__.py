"""CPU fp64 oracle for folded-GQA decode attention and Quest sparse decode.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path: it shares
no kernels, headers, helpers, tables or constants with it. Inputs arrive as the
same fp16 arrays the GPU sees and are widened exactly to float64.

Sources (cited by page title and section only):

* [CoreML-GQA] "Core ML Decode Optimization: Removing the 1.9 GiB Per-Token
  Copy Caused by GQA repeat_kv" (OptAI engineering blog).
* [Quest-review] jaehun.me review of "Quest: Query-Aware Sparsity for
  Efficient Long-Context LLM Inference", which cites the paper's own sections
  (section 3.4, Algorithm 1, section 3.5).

Modules:

* ``oracle.dense``  -- repeat_kv decode attention (the plain definition), its
  q_len > 1 form with the causal alignment, the paged-address gather, the KV
  append.
* ``oracle.quest``  -- page min/max metadata, the page score U(p, q), top-K
  selection and attention restricted to the selected pages.
* ``oracle.bytes_model`` -- algorithmic byte counts and the Quest read-bytes
  model.

Every function is pinned by ``tests/test_oracle_pins.py`` against facts the
pages or mathematics fix (worked examples, closed forms, library special cases,
brute force).  The only part without such a pin is the *quality* of Quest's
approximation relative to dense attention (the pages measure it on datasets
that are not available here): parity unpinned for quality; the oracle only
defines the approximation itself.
"""

from .dense import (  # noqa: F401
    repeat_kv,
    append_kv,
    gather_paged,
    decode_attention,
    multi_query_attention,
)
from .quest import (  # noqa: F401
    page_count,
    build_metadata,
    append_metadata,
    page_scores,
    select_pages,
    selected_token_mask,
    sparse_decode_attention,
)
from .bytes_model import (  # noqa: F401
    dense_kv_bytes,
    quest_read_bytes,
    quest_read_ratio,
)
