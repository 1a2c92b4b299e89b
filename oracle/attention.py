"""Tag-masked attention over the flattened verification batch.

TEST INFRASTRUCTURE (see the package docstring).

What the pages fix: dynamic, variable-length verification ruins the
utilisation of padded decode kernels, so every token is flattened into an
independent element and the dependencies inside a sequence travel in a tag
tensor ([P1] engineering table, row "内核利用率暴跌": 物理解耦稀疏注意力).

Readings where the pages are silent (each listed with its reason in the design
notes):
  query rows    the flattened batch of the verification forward: row (r, j) is
                the token at position ctx_r + j of request r (j = 0 is the last
                committed token, j = 1 .. L_r the drafts; the bonus row of the
                verification batch is the row after the last verified draft).
  keys          request r's KV cache, positions 0 .. ctx_r + j inclusive: the
                draft tokens' keys and values are already in the cache, and the
                tag's position j masks the ones after the row (causal inside the
                block); other requests are never visible.
  cache         paged: position p of request r lives in page
                page_table[r, p // page_size], slot p % page_size; the pool is
                [pages, page_size, H_kv, D] (position-major) or
                [pages, H_kv, page_size, D] (head-major): two storage orders of
                the same cache.
  heads         grouped-query attention: query head h reads KV head
                h // (H_q / H_kv).
  scale         1 / sqrt(D); softmax over the visible keys.

The computation is the definition, in float64: for every row and query head,
scores s_p = q . k_p * scale for the visible positions p, weights
softmax(s), output sum_p w_p v_p.

Pins (tests/test_oracle_attention.py): against torch's scaled_dot_product_
attention on a dense padded copy with an explicit mask (a library routine for
the dense special case); all-equal keys give the mean of the visible values
(exact mask length); a single visible key returns its value; permuting the
page pool with the page table leaves the output unchanged; a shifted key
(k + c q direction) changes nothing when the shift is common to all keys.
"""
from __future__ import annotations

import numpy as np

from .numerics import decode


def gather_keys(cache: np.ndarray, page_table: np.ndarray, r: int, n: int, page_size: int, hk: int,
                head_major: bool = False) -> np.ndarray:
    """Positions 0 .. n-1 of request r, KV head hk: float64 [n, D]."""
    p = np.arange(n)
    pages = page_table[r, p // page_size]
    if head_major:
        return cache[pages, hk, p % page_size, :].astype(np.float64)
    return cache[pages, p % page_size, hk, :].astype(np.float64)


def flat_attention(q, k_cache, v_cache, page_table, ctx_len, tags, n_rows, page_size, dtype="bf16",
                   head_major=False):
    """Output [n_rows, H_q, D] float64 for the flattened rows 0 .. n_rows-1.

    q [B, H_q, D], caches [pages, page_size, H_kv, D] (bf16 bit patterns or
    fp32), page_table [R, max_pages], ctx_len [R], tags [B, 2] (request,
    position). head_major: the caches are [pages, H_kv, page_size, D]."""
    Q = decode(q, dtype)
    K = decode(k_cache, dtype)
    Vc = decode(v_cache, dtype)
    Hq, D = Q.shape[1], Q.shape[2]
    Hkv = K.shape[1] if head_major else K.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(float(D))
    out = np.zeros((n_rows, Hq, D), dtype=np.float64)
    for t in range(n_rows):
        r, j = int(tags[t, 0]), int(tags[t, 1])
        n = int(ctx_len[r]) + j + 1                   # visible positions
        for hk in range(Hkv):
            Kr = gather_keys(K, page_table, r, n, page_size, hk, head_major)
            Vr = gather_keys(Vc, page_table, r, n, page_size, hk, head_major)
            for h in range(hk * G, (hk + 1) * G):
                s = (Kr @ Q[t, h]) * scale
                w = np.exp(s - s.max())
                w /= w.sum()
                out[t, h] = w @ Vr
    return out
