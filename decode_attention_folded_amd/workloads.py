"""Seeded synthetic inputs for the decode-attention library and its tests.

This module only *draws inputs*: shapes, N(0, 1) values rounded to fp16,
valid lengths, page permutations and planted pages.  It holds none of the
attention or Quest arithmetic, so both the HIP path and the CPU oracle can be
fed from it without sharing any of the computation.

Recipe (the design notes restate it):

* Values are N(0, 1), drawn as float32 and rounded to fp16 (round to nearest
  even).  NumPy generators are ``np.random.default_rng([seed, stream])`` with
  streams 0 = Q, 1 = K, 2 = V, 3 = lengths, 4 = page permutation,
  5 = planted pages, 6 = new K/V row.
* Cache slots at or past a sequence's valid length are filled with NaN when
  ``poison=True``, so any read of them shows up in the output.
* Planted pages (to give Quest something to find): for each (batch, KV head)
  a set of pages is drawn uniformly without replacement, and every Key in them
  gets +1.5 * q_hat added in float32 before the fp16 rounding, where q_hat is
  the unit vector along the sum of the group's fp16 queries.
* Large configurations are drawn on the GPU with ``torch.Generator`` by
  :func:`device_case` (same recipe, different random stream); the oracle then
  reads back exactly the fp16 bytes the GPU holds.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_LEN, STREAM_PERM, STREAM_PLANT, STREAM_NEW = range(7)


def _rng(seed, stream):
    return np.random.default_rng([int(seed), int(stream)])


def normal_fp16(seed, stream, shape):
    return _rng(seed, stream).standard_normal(size=shape, dtype=np.float32).astype(np.float16)


@dataclass
class Case:
    """One decode step's inputs, as host NumPy arrays (fp16 unless noted)."""
    q: np.ndarray                      # [B, Hq, D]
    k: np.ndarray                      # contiguous [B, Hkv, cap, D] or pool [NP, Hkv, S, D]
    v: np.ndarray
    seqlens: np.ndarray                # int32 [B]
    num_kv_heads: int
    head_dim: int
    capacity: int                      # per-sequence logical slots
    page_size: int = 0                 # paged pool page size (0 = contiguous)
    page_table: Optional[np.ndarray] = None   # int32 [B, max_pages], -1 = unused
    k_new: Optional[np.ndarray] = None        # [B, Hkv, D]
    v_new: Optional[np.ndarray] = None
    planted: dict = field(default_factory=dict)  # (b, kv) -> sorted planted pages

    @property
    def batch(self):
        return self.q.shape[0]

    @property
    def num_q_heads(self):
        return self.q.shape[1]

    @property
    def scale(self):
        return 1.0 / float(np.sqrt(self.head_dim))


def draw_seqlens(seed, batch, lo, hi):
    """Integer lengths uniform on [lo, hi] inclusive."""
    return _rng(seed, STREAM_LEN).integers(lo, hi + 1, size=batch).astype(np.int32)


def dense_case(seed, batch, num_q_heads, num_kv_heads, head_dim, capacity, seqlens,
               with_new=False, poison=True, plant_pages=0, plant_page_size=16,
               plant_shift=1.5):
    """A contiguous-cache case: K/V [B, Hkv, capacity, D]."""
    seqlens = np.asarray(seqlens, dtype=np.int32).reshape(batch)
    q = normal_fp16(seed, STREAM_Q, (batch, num_q_heads, head_dim))
    k32 = _rng(seed, STREAM_K).standard_normal(
        size=(batch, num_kv_heads, capacity, head_dim), dtype=np.float32)
    planted = {}
    if plant_pages:
        planted = _plant(seed, q, k32, seqlens, num_kv_heads, plant_pages,
                         plant_page_size, plant_shift)
    k = k32.astype(np.float16)
    del k32
    v = normal_fp16(seed, STREAM_V, (batch, num_kv_heads, capacity, head_dim))
    k_new = v_new = None
    if with_new:
        kv_new = normal_fp16(seed, STREAM_NEW, (2, batch, num_kv_heads, head_dim))
        k_new, v_new = np.ascontiguousarray(kv_new[0]), np.ascontiguousarray(kv_new[1])
    if poison:
        for b in range(batch):
            k[b, :, max(0, int(seqlens[b])):, :] = np.nan
            v[b, :, max(0, int(seqlens[b])):, :] = np.nan
    return Case(q=q, k=k, v=v, seqlens=seqlens, num_kv_heads=num_kv_heads,
                head_dim=head_dim, capacity=capacity, k_new=k_new, v_new=v_new,
                planted=planted)


def _plant(seed, q, k32, seqlens, num_kv_heads, n_plant, page_size, shift):
    """Add shift * q_hat to every Key of n_plant random pages per (b, kv)."""
    rng = _rng(seed, STREAM_PLANT)
    batch, num_q_heads, _ = q.shape
    group = num_q_heads // num_kv_heads
    planted = {}
    for b in range(batch):
        n_pages = (int(seqlens[b]) + page_size - 1) // page_size
        for kv in range(num_kv_heads):
            qsum = q[b, kv * group:(kv + 1) * group].astype(np.float32).sum(axis=0)
            qhat = qsum / np.float32(np.linalg.norm(qsum))
            count = min(n_plant, n_pages)
            pages = np.sort(rng.choice(n_pages, size=count, replace=False))
            for p in pages:
                lo = int(p) * page_size
                hi = min(lo + page_size, int(seqlens[b]))
                k32[b, kv, lo:hi, :] += np.float32(shift) * qhat
            planted[(b, kv)] = [int(p) for p in pages]
    return planted


def paged_case(seed, batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages,
               seqlens, poison=True, spare_pages=0):
    """A paged case: pool [NP, Hkv, S, D] with pages assigned by a random
    permutation; page_table [B, max_pages] with -1 for unused entries."""
    seqlens = np.asarray(seqlens, dtype=np.int32).reshape(batch)
    pages_per_seq = [(int(l) + page_size - 1) // page_size for l in seqlens]
    total = sum(pages_per_seq) + spare_pages
    perm = _rng(seed, STREAM_PERM).permutation(max(total, 1)).astype(np.int32)
    q = normal_fp16(seed, STREAM_Q, (batch, num_q_heads, head_dim))
    pool_k = normal_fp16(seed, STREAM_K, (max(total, 1), num_kv_heads, page_size, head_dim))
    pool_v = normal_fp16(seed, STREAM_V, (max(total, 1), num_kv_heads, page_size, head_dim))
    table = np.full((batch, max_pages), -1, dtype=np.int32)
    nxt = 0
    for b in range(batch):
        for p in range(pages_per_seq[b]):
            table[b, p] = perm[nxt]
            nxt += 1
    if poison:
        for b in range(batch):
            lb = int(seqlens[b])
            if lb % page_size:
                last = table[b, lb // page_size]
                pool_k[last, :, lb % page_size:, :] = np.nan
                pool_v[last, :, lb % page_size:, :] = np.nan
        used = set(int(x) for x in table[table >= 0])
        for p in range(pool_k.shape[0]):
            if p not in used:
                pool_k[p] = np.nan
                pool_v[p] = np.nan
    return Case(q=q, k=pool_k, v=pool_v, seqlens=seqlens, num_kv_heads=num_kv_heads,
                head_dim=head_dim, capacity=max_pages * page_size, page_size=page_size,
                page_table=table)


# --------------------------------------------------------------------------
# The five benchmark workloads (shapes and value recipes).
# --------------------------------------------------------------------------

WORKLOADS = {
    1: dict(name="gqa_decode_b1_hq32_hkv8_d64_ctx4096",
            batch=1, num_q_heads=32, num_kv_heads=8, head_dim=64, capacity=4096,
            seqlen=4096),
    2: dict(name="exaone1.2b_30layer_decode_hq32_hkv8_d64_cap4096_len3000_append",
            layers=30, batch=1, num_q_heads=32, num_kv_heads=8, head_dim=64,
            capacity=4096, seqlen=3000),
    3: dict(name="paged_gqa_decode_b64_hq32_hkv8_d128_s16_len1k-32k",
            batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
            max_pages=2048, len_lo=1024, len_hi=32768),
    4: dict(name="quest_llama2-7b_b1_h32_d128_L32768_s16_budget2048",
            batch=1, num_q_heads=32, num_kv_heads=32, head_dim=128, capacity=32768,
            seqlen=32768, page_size=16, budget=2048, plant=8),
    5: dict(name="quest_gqa_b8_hq32_hkv8_d128_L131072_s16_budget4096_append",
            batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128, capacity=131072,
            seqlen=131072, page_size=16, budget=4096, plant=16),
}


def device_normal_fp16(gen, shape, device):
    import torch
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.float16)


def device_generator(seed, stream, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(stream))
    return g


def device_dense(seed, batch, num_q_heads, num_kv_heads, head_dim, capacity, seqlen,
                 device, plant_pages=0, plant_page_size=16, plant_shift=1.5,
                 with_new=False):
    """Draw a contiguous-cache case directly on ``device`` (torch tensors).

    Same recipe as :func:`dense_case`; all slots of the cache hold N(0, 1)
    values (positions past the valid length are masked by the kernels, never
    read).  Planting is done in float32 before the fp16 rounding, one
    (batch, KV head) slab at a time to bound the float32 footprint.
    """
    import torch
    q = device_normal_fp16(device_generator(seed, STREAM_Q, device),
                           (batch, num_q_heads, head_dim), device)
    gk = device_generator(seed, STREAM_K, device)
    gv = device_generator(seed, STREAM_V, device)
    k = torch.empty((batch, num_kv_heads, capacity, head_dim), dtype=torch.float16, device=device)
    v = torch.empty_like(k)
    group = num_q_heads // num_kv_heads
    rng = _rng(seed, STREAM_PLANT)
    n_pages = (seqlen + plant_page_size - 1) // plant_page_size
    planted = {}
    for b in range(batch):
        for kv in range(num_kv_heads):
            slab = torch.randn((capacity, head_dim), generator=gk, device=device,
                               dtype=torch.float32)
            if plant_pages:
                qsum = q[b, kv * group:(kv + 1) * group].float().sum(dim=0)
                qhat = qsum / qsum.norm()
                pages = np.sort(rng.choice(n_pages, size=min(plant_pages, n_pages),
                                           replace=False))
                for p in pages:
                    lo = int(p) * plant_page_size
                    hi = min(lo + plant_page_size, seqlen)
                    slab[lo:hi] += plant_shift * qhat
                planted[(b, kv)] = [int(p) for p in pages]
            k[b, kv] = slab.to(torch.float16)
            v[b, kv] = torch.randn((capacity, head_dim), generator=gv, device=device,
                                   dtype=torch.float32).to(torch.float16)
    seqlens = torch.full((batch,), seqlen, dtype=torch.int32, device=device)
    out = dict(q=q, k=k, v=v, seqlens=seqlens, planted=planted)
    if with_new:
        gn = device_generator(seed, STREAM_NEW, device)
        out["k_new"] = device_normal_fp16(gn, (batch, num_kv_heads, head_dim), device)
        out["v_new"] = device_normal_fp16(gn, (batch, num_kv_heads, head_dim), device)
    return out


def device_paged(seed, batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages,
                 seqlens, device):
    """Draw a paged case on ``device``: lengths given on the host, pages of the
    pool assigned to sequences by a seeded random permutation."""
    import torch
    seqlens = np.asarray(seqlens, dtype=np.int32)
    pages_per_seq = [(int(l) + page_size - 1) // page_size for l in seqlens]
    total = sum(pages_per_seq)
    perm = _rng(seed, STREAM_PERM).permutation(total).astype(np.int32)
    table = np.full((batch, max_pages), -1, dtype=np.int32)
    nxt = 0
    for b in range(batch):
        table[b, :pages_per_seq[b]] = perm[nxt:nxt + pages_per_seq[b]]
        nxt += pages_per_seq[b]
    q = device_normal_fp16(device_generator(seed, STREAM_Q, device),
                           (batch, num_q_heads, head_dim), device)
    shape = (total, num_kv_heads, page_size, head_dim)
    k = device_normal_fp16(device_generator(seed, STREAM_K, device), shape, device)
    v = device_normal_fp16(device_generator(seed, STREAM_V, device), shape, device)
    return dict(q=q, k=k, v=v,
                seqlens=torch.from_numpy(seqlens).to(device),
                page_table=torch.from_numpy(table).to(device),
                seqlens_host=seqlens, page_table_host=table)
