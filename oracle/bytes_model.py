"""Algorithmic byte counts: what each step must move, and the Quest model.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).
"""


def dense_kv_bytes(seqlens, num_kv_heads, head_dim, elem_bytes=2):
    """K plus V bytes a folded decode step reads: every valid token of every KV
    head once (the fold reads K/V at their stored width; [CoreML-GQA]
    section 3, "Implementation")."""
    tokens = sum(max(0, int(l)) for l in seqlens)
    return 2 * tokens * num_kv_heads * head_dim * elem_bytes


def quest_read_bytes(seq_len, page_size, k_pages, key_bytes):
    """Quest's simple read model, [Quest-review] "how read bytes shrink"
    (paper section 3.5): with M bytes per Key (or Value),
        D_metadata ~ 2 M L / S   (a min and a max vector per page),
        D_selected ~ 2 M K S     (K and V of the chosen full pages),
        D_full      = 2 M L.
    Returns (d_meta, d_sel, d_full).  Top-K, sorting and buffers are outside
    the model."""
    d_meta = 2 * key_bytes * seq_len // page_size
    d_sel = 2 * key_bytes * k_pages * page_size
    d_full = 2 * key_bytes * seq_len
    return d_meta, d_sel, d_full


def quest_read_ratio(seq_len, page_size, k_pages):
    """D_Quest / D_full = 1/S + K S / L = 1/S + B/L with B = K S tokens."""
    return 1.0 / page_size + (k_pages * page_size) / seq_len
