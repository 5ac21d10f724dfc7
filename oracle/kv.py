"""KV commit after acceptance (oracle).

Source: "Support Eagle-3 Speculative Decoding in llama.cpp", the reply on how
large the draft's context grows: the target model keeps KV entries only for
accepted tokens, while the draft keeps them for every candidate and so needs
an eviction step.  Read with "EAGLE-2: Feature-Level Speculative Decoding
Guide", Key Architectural Mechanics 3 (the accepted tokens are the longest
verified root path), this gives the step after acceptance: the K/V rows of
the accepted path, root first, become the next cache positions L, L + 1, ...;
every other candidate's rows are dropped.

Readings (the pages give no layout): the tree's K/V are ``[layers][Hkv][rows]
[hd]`` with row r holding tree node (or draft slot) r; ``rows`` lists the
source rows in order, and ``count`` of them are appended.  The copy reads
every source row before it writes, so source and cache may be the same
buffer (tree rows stored right after the prefix).
"""
from __future__ import annotations

import numpy as np


def kv_commit(src_k, src_v, rows, count, cache_k, cache_v, L):
    """Return ``(cache_k, cache_v)`` with positions ``L .. L + count - 1`` of
    every layer and head replaced by source rows ``rows[0 .. count - 1]``.

    ``src_*``: ``[layers][Hkv][S][hd]``; ``cache_*``: ``[layers][Hkv][C][hd]``
    (any dtype; values are copied, never converted).  The inputs are not
    modified.
    """
    src_k = np.asarray(src_k)
    src_v = np.asarray(src_v)
    rows = [int(r) for r in np.asarray(rows).reshape(-1)[:count]]
    S = src_k.shape[2]
    if count < 0 or L < 0 or L + count > np.asarray(cache_k).shape[2]:
        raise ValueError("commit past the end of the cache")
    for r in rows:
        if not 0 <= r < S:
            raise ValueError(f"source row {r} outside [0, {S})")
    gathered_k = [src_k[:, :, r, :].copy() for r in rows]     # every read before any write
    gathered_v = [src_v[:, :, r, :].copy() for r in rows]
    out_k = np.array(cache_k, copy=True)
    out_v = np.array(cache_v, copy=True)
    for j in range(count):
        out_k[:, :, L + j, :] = gathered_k[j]
        out_v[:, :, L + j, :] = gathered_v[j]
    return out_k, out_v


def kv_commit_in_place(cache_k, cache_v, L, path, count):
    """The in-place layout: tree row r is cache position L + r.  Returns the
    caches after moving tree rows ``path[j]`` to positions ``L + j``."""
    cache_k = np.asarray(cache_k)
    cache_v = np.asarray(cache_v)
    rows = [L + int(r) for r in np.asarray(path).reshape(-1)[:count]]
    return kv_commit(cache_k, cache_v, rows, count, cache_k, cache_v, L)
