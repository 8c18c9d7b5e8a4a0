"""Quest query-aware page selection, by brute force, in the order the method
takes its steps.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): never imported by the
product path.

[Quest-review] flowchart in "keep the cache, read what is needed now"
(paper sections 2.2, 3.3-3.5): the current query and every page's Key min/max
metadata give a score per page; the highest-scoring pages are chosen; only the
chosen pages' K and V are read; attention runs over those tokens.  The full
cache is kept, so a page left out now can be chosen at the next step.

Readings of points the review leaves open (each also listed in the design
notes):

* GQA: the review describes one query per KV head.  With G query heads per KV
  head, the page score is the sum of U over the G heads of the group, and one
  selection per (batch, KV head) serves all G heads.
* The last, partly filled page is scored from its valid keys only; pages with
  no valid key do not exist and are never chosen; if a sequence has at most K
  pages, all of them are chosen.
* Ties in U go to the lower page index; the chosen pages are reported in
  ascending page order, padded with -1.
* The budget is given in tokens and K = budget / S pages (the review's
  page/token distinction, paper section 3.4).
"""

import numpy as np

from .dense import decode_attention


def page_count(seqlen, page_size):
    """Number of pages holding at least one valid key: ceil(L / S)."""
    seqlen = max(0, int(seqlen))
    return (seqlen + page_size - 1) // page_size


def build_metadata(k_cache, seqlens, page_size, max_pages):
    """Per-page, per-channel Key minimum and maximum over the valid keys.

    [Quest-review] "the page score is not an exact attention probability"
    (paper section 3.4): for page p and channel i the method keeps m_{p,i} and
    M_{p,i}, the smallest and largest value of channel i over the Keys stored
    in the page.

    ``k_cache``: [B, Hkv, cap, D] (fp16 for the library; any float dtype is
    kept).  Returns [B, Hkv, max_pages, 2, D] of the same dtype, where
    [..., 0, :] is the minimum and [..., 1, :] the maximum.  Min and max of
    fp16 values are fp16 values, so this result is exact.  Entries for pages
    at or beyond ceil(L_b / S) are left at zero and carry no meaning.
    """
    bsz, hkv, _, d = k_cache.shape
    meta = np.zeros((bsz, hkv, max_pages, 2, d), dtype=k_cache.dtype)
    for b in range(bsz):
        lb = int(seqlens[b])
        for p in range(page_count(lb, page_size)):
            lo = p * page_size
            hi = min(lo + page_size, lb)
            keys = k_cache[b, :, lo:hi, :]
            meta[b, :, p, 0, :] = keys.min(axis=1)
            meta[b, :, p, 1, :] = keys.max(axis=1)
    return meta


def append_metadata(meta, k_cache, seqlens, n_new, page_size):
    """Update page metadata key by key, the way the method maintains it.

    [Quest-review] (paper section 3.4): the metadata is updated whenever a new
    Key enters the cache.  For the key at position t, page p = t // S: a key
    that starts a page (t mod S == 0) sets m = M = k; any other key lowers m
    and raises M channel by channel.  The keys handled are positions
    [L_b - n_new, L_b), taken in increasing order from ``k_cache`` (which must
    already hold them).  Returns an updated copy of ``meta``.
    """
    out = np.array(meta, copy=True)
    for b in range(k_cache.shape[0]):
        lb = int(seqlens[b])
        for t in range(max(0, lb - n_new), lb):
            p = t // page_size
            key = k_cache[b, :, t, :]
            if t % page_size == 0:
                out[b, :, p, 0, :] = key
                out[b, :, p, 1, :] = key
            else:
                out[b, :, p, 0, :] = np.minimum(out[b, :, p, 0, :], key)
                out[b, :, p, 1, :] = np.maximum(out[b, :, p, 1, :], key)
    return out


def page_scores(q, meta, seqlens, page_size):
    """Upper-bound page score U(p, q), summed over the query heads of a group.

    [Quest-review] "the page score is not an exact attention probability"
    (paper section 3.4, Algorithm 1):
        U(p, q) = sum_i max(q_i * m_{p,i}, q_i * M_{p,i}).
    Both extremes are needed because a negative q_i pairs best with the
    minimum.  No softmax scale is applied; a common positive scale would not
    change the ranking.

    ``q``: [B, Hq, D]; ``meta``: [B, Hkv, P, 2, D].  Returns float64
    [B, Hkv, P]; pages at or beyond ceil(L_b / S) score -inf.
    """
    q64 = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q64.shape
    hkv, max_pages = meta.shape[1], meta.shape[2]
    group = hq // hkv
    out = np.full((bsz, hkv, max_pages), -np.inf, dtype=np.float64)
    for b in range(bsz):
        n_pages = page_count(seqlens[b], page_size)
        for kv in range(hkv):
            mins = np.asarray(meta[b, kv, :n_pages, 0, :], dtype=np.float64)
            maxs = np.asarray(meta[b, kv, :n_pages, 1, :], dtype=np.float64)
            total = np.zeros(n_pages, dtype=np.float64)
            for g in range(group):
                qh = q64[b, kv * group + g]
                total += np.maximum(mins * qh, maxs * qh).sum(axis=1)
            out[b, kv, :n_pages] = total
    return out


def select_pages(scores, seqlens, page_size, k_pages):
    """Top-K pages by score, ties to the lower page index, ascending output.

    [Quest-review] (paper section 3.4): keep the K pages with the highest U.
    A full sort by (-U, page index) is used, then the first min(K, P_b) are
    kept and reported in increasing page order, padded with -1.  Returns int32
    [B, Hkv, K].
    """
    bsz, hkv, _ = scores.shape
    out = np.full((bsz, hkv, k_pages), -1, dtype=np.int32)
    for b in range(bsz):
        n_pages = page_count(seqlens[b], page_size)
        for kv in range(hkv):
            order = sorted(range(n_pages), key=lambda p: (-scores[b, kv, p], p))
            chosen = sorted(order[:k_pages])
            out[b, kv, :len(chosen)] = chosen
    return out


def selected_token_mask(page_idx, seqlens, page_size, capacity):
    """Token positions covered by the chosen pages: the union over chosen p of
    [p*S, min(p*S + S, L_b)).  Returns bool [B, Hkv, capacity]."""
    bsz, hkv, _ = page_idx.shape
    mask = np.zeros((bsz, hkv, capacity), dtype=bool)
    for b in range(bsz):
        lb = int(seqlens[b])
        for kv in range(hkv):
            for p in page_idx[b, kv]:
                if p < 0:
                    continue
                lo = int(p) * page_size
                mask[b, kv, lo:min(lo + page_size, lb)] = True
    return mask


def sparse_decode_attention(q, k_cache, v_cache, seqlens, page_idx, page_size, scale):
    """Exact attention over the chosen pages' real K and V.

    [Quest-review] worked example and flowchart (paper sections 3.3-3.5):
    inside the chosen pages attention uses the true Keys and Values; tokens
    outside them are left out, and the softmax renormalises over what remains.
    Built as the dense oracle with every unchosen token masked to -inf.
    """
    mask = selected_token_mask(page_idx, seqlens, page_size, k_cache.shape[2])
    return decode_attention(q, k_cache, v_cache, seqlens, scale, token_mask=mask)
