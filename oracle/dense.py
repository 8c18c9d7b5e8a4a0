"""Dense decode attention, written the plain way: materialise repeat_kv, then
ordinary per-head attention in float64.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): never imported by the
product path.

The folded kernel must give exactly this result (up to rounding order):
[CoreML-GQA] section 3 "Why the Computation Is Equivalent" argues that
splitting the query heads into [Hkv, G] groups changes no row of the
computation, so the definition to check against is the unfolded one.
"""

import numpy as np


def repeat_kv(x, n_rep):
    """Replicate KV heads so that query head h reads KV head h // n_rep.

    [CoreML-GQA] section 2, "expand Is a View, but reshape Introduces a Copy":
    insert a repetition axis after the KV-head axis, expand it n_rep times and
    merge (kv, rep) into one head axis in that order.  ``x``: [B, Hkv, T, D].
    Returns a new [B, Hkv * n_rep, T, D] array (a real copy, like the eager
    reshape the page describes).
    """
    b, hkv, t, d = x.shape
    expanded = np.broadcast_to(x[:, :, None, :, :], (b, hkv, n_rep, t, d))
    return np.array(expanded.reshape(b, hkv * n_rep, t, d))


def append_kv(k_cache, v_cache, seqlens, k_new, v_new):
    """Write this step's K/V row into slot L_b - 1 of a copy of the cache.

    [CoreML-GQA] section 1: adding a token updates one position along the
    sequence axis of every layer's cache.  The valid length L_b counts the new
    token, so the row lands at index L_b - 1.  ``k_new``/``v_new``: [B, Hkv, D].
    Sequences with L_b < 1 are left untouched.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for b in range(k_cache.shape[0]):
        lb = int(seqlens[b])
        if lb >= 1:
            k_out[b, :, lb - 1, :] = k_new[b]
            v_out[b, :, lb - 1, :] = v_new[b]
    return k_out, v_out


def gather_paged(pool, page_table, page_size, capacity):
    """Rebuild a contiguous [B, Hkv, capacity, D] cache from a paged pool.

    Paged addressing as the problem statement gives it: token t of sequence b
    lives in row (t mod S) of physical page page_table[b][t // S]; the pool is
    [num_pages, Hkv, S, D].  Logical slots whose page-table entry is negative
    are filled with NaN so that any read of them is visible.
    """
    num_b = page_table.shape[0]
    _, hkv, s, d = pool.shape
    assert s == page_size
    out = np.full((num_b, hkv, capacity, d), np.nan, dtype=pool.dtype)
    for b in range(num_b):
        for t in range(capacity):
            phys = int(page_table[b, t // page_size])
            if phys >= 0:
                out[b, :, t, :] = pool[phys, :, t % page_size, :]
    return out


def decode_attention(q, k_cache, v_cache, seqlens, scale, token_mask=None):
    """Single-token decode attention over a GQA cache, in float64.

    [CoreML-GQA] section 3 "Implementation" lists the decode path: scores
    q.k^T, multiply by the scale, add the (sliced) additive mask, softmax over
    the context axis, then prob.V, and reshape back to [B, Hq, 1, D].  Here the
    KV heads are first replicated with :func:`repeat_kv` (section 2), which is
    the reference form the fold must reproduce.

    * ``q``: [B, Hq, D]; ``k_cache``/``v_cache``: [B, Hkv, cap, D].
    * ``seqlens[b]``: valid length L_b; the mask is -inf at positions >= L_b
      (the decode-time meaning of the sliced mask).  The cache is sliced to
      [0, L_b) before any arithmetic, so values stored past L_b never matter.
    * ``scale``: plain multiplier on the scores (1/sqrt(D) in the workloads).
    * ``token_mask``: optional bool [B, Hkv, cap]; False also masks a token
      (used by the Quest oracle).  It is replicated across the G query heads of
      a group exactly like K and V.
    * A row with no unmasked token returns zeros (an empty softmax has no
      value; zero is this library's documented convention).

    Returns float64 [B, Hq, D].
    """
    q64 = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q64.shape
    hkv = k_cache.shape[1]
    assert hq % hkv == 0
    n_rep = hq // hkv
    out = np.zeros((bsz, hq, d), dtype=np.float64)
    for b in range(bsz):
        lb = int(seqlens[b])
        lb = max(0, min(lb, k_cache.shape[2]))
        if lb == 0:
            continue
        k_rep = repeat_kv(np.asarray(k_cache[b:b + 1, :, :lb, :], dtype=np.float64), n_rep)[0]
        v_rep = repeat_kv(np.asarray(v_cache[b:b + 1, :, :lb, :], dtype=np.float64), n_rep)[0]
        scores = np.einsum("hd,htd->ht", q64[b], k_rep) * scale
        if token_mask is not None:
            keep = np.repeat(np.asarray(token_mask[b, :, :lb], dtype=bool), n_rep, axis=0)
            scores = np.where(keep, scores, -np.inf)
        for h in range(hq):
            row = scores[h]
            if not np.any(np.isfinite(row)):
                continue
            row_max = np.max(row)
            e = np.exp(row - row_max)
            prob = e / np.sum(e)
            out[b, h] = prob @ v_rep[h]
    return out


def multi_query_attention(q, k_cache, v_cache, seqlens, scale):
    """Attention for q_len > 1 new tokens per sequence over a GQA cache, float64.

    [CoreML-GQA] section 5 "Limitations and Next Steps" ("Prefill Needs
    Separate Design"): with more than one query position per head, the grouped
    path must also align the causal mask.  Reading used here (chunked prefill,
    speculative verify): the q_len queries of sequence b sit at its last q_len
    positions L_b - q_len .. L_b - 1 (their keys are already in the cache), and
    query i attends to the keys t <= L_b - q_len + i.  Written the plain way:
    repeat_kv, then per head and per query a softmax over that key prefix.

    * ``q``: [B, Hq, Lq, D]; ``k_cache``/``v_cache``: [B, Hkv, cap, D];
      ``seqlens[b]`` = L_b (clamped to [0, cap]).
    * A query with no key (L_b - q_len + i < 0) returns zeros.

    Returns float64 [B, Hq, Lq, D].
    """
    q64 = np.asarray(q, dtype=np.float64)
    bsz, hq, lq, d = q64.shape
    hkv = k_cache.shape[1]
    assert hq % hkv == 0
    n_rep = hq // hkv
    out = np.zeros((bsz, hq, lq, d), dtype=np.float64)
    for b in range(bsz):
        lb = max(0, min(int(seqlens[b]), k_cache.shape[2]))
        if lb == 0:
            continue
        k_rep = repeat_kv(np.asarray(k_cache[b:b + 1, :, :lb, :], dtype=np.float64), n_rep)[0]
        v_rep = repeat_kv(np.asarray(v_cache[b:b + 1, :, :lb, :], dtype=np.float64), n_rep)[0]
        for i in range(lq):
            visible = lb - lq + 1 + i          # keys 0 .. L_b - q_len + i
            if visible <= 0:
                continue
            for h in range(hq):
                scores = (k_rep[h, :visible] @ q64[b, h, i]) * scale
                e = np.exp(scores - np.max(scores))
                out[b, h, i] = (e / np.sum(e)) @ v_rep[h, :visible]
    return out
