"""Dynamic draft tree: expansion by cumulative confidence, then rerank (oracle).

Sources:
  * "Support Eagle-3 Speculative Decoding in llama.cpp" (reply on PR #3624 vs
    dynamic trees): the draft's confidence approximates the acceptance rate,
    the tree is grown from it, and it is pruned at the end of drafting.
  * "EAGLE-2: Feature-Level Speculative Decoding Guide", section 2: the tree
    spends its token budget where confidence is high, so verification is not
    spent on unlikely paths.

Readings (the pages defer the details to the EAGLE-2 paper): a node's value
is its cumulative log-probability along the path from the root, each step one
fp32 addition ``value[parent] + logp``; the root's value is 0.  Every child
proposed in a round stays in the candidate pool; the next frontier is chosen
among the current round's new entries only.  Ranking is by value descending,
lower pool index first among equal values.  Outputs list pool entries in
ascending pool index, which is a topological order.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class Pool:
    token: list
    parent: list
    depth: list
    value: list     # numpy float32 scalars

    @classmethod
    def root(cls, token: int) -> "Pool":
        return cls([int(token)], [-1], [0], [np.float32(0.0)])

    def __len__(self):
        return len(self.token)

    def arrays(self):
        return (np.array(self.token, np.int32), np.array(self.parent, np.int32),
                np.array(self.depth, np.int32), np.array(self.value, np.float32))


def _better(a_val, a_idx, b_val, b_idx) -> bool:
    """Strict order: larger value first, then lower index."""
    return a_val > b_val or (a_val == b_val and a_idx < b_idx)


def _top(indices, values, n):
    """The n best of ``indices`` under (value desc, index asc)."""
    ranked = sorted(indices, key=lambda i: (-float(values[i]), i))
    return ranked[:n]


def expand(pool: Pool, frontier, child_id, child_logp, k_select: int):
    """Append every child of every frontier node; return the new frontier.

    For frontier slot s and child rank j (s-major, j-minor) the new entry gets
    token ``child_id[s][j]``, parent ``frontier[s]``, depth + 1 and value
    ``fp32(value[frontier[s]] + child_logp[s][j])``.  The new frontier is the
    ``k_select`` best new entries, listed by ascending pool index.
    """
    child_id = np.asarray(child_id)
    child_logp = np.asarray(child_logp, dtype=np.float32)
    kf, k = child_id.shape
    if len(frontier) != kf:
        raise ValueError("frontier and child rows disagree")
    start = len(pool)
    for s in range(kf):
        u = int(frontier[s])
        for j in range(k):
            pool.token.append(int(child_id[s, j]))
            pool.parent.append(u)
            pool.depth.append(pool.depth[u] + 1)
            pool.value.append(np.float32(pool.value[u]) + np.float32(child_logp[s, j]))
    new = list(range(start, len(pool)))
    chosen = _top(new, pool.value, min(k_select, len(new)))
    return sorted(chosen)


def rerank(pool: Pool, T: int):
    """Keep the root plus the T-1 best non-root entries; re-index parents.

    Returns ``(token, parent, depth, pool_idx)`` as int32 arrays of length T
    in ascending pool index, ``parent`` given as positions in that list.
    """
    n = len(pool)
    if not (1 <= T <= n):
        raise ValueError("T must be between 1 and the pool size")
    keep = sorted([0] + _top(range(1, n), pool.value, T - 1))
    pos = {p: i for i, p in enumerate(keep)}
    token = np.array([pool.token[p] for p in keep], np.int32)
    depth = np.array([pool.depth[p] for p in keep], np.int32)
    parent = np.empty(T, np.int32)
    for i, p in enumerate(keep):
        pp = pool.parent[p]
        if pp == -1:
            parent[i] = -1
        elif pp in pos:
            parent[i] = pos[pp]
        else:
            raise ValueError(f"pool entry {p} kept without its parent {pp}")
    return token, parent, depth, np.array(keep, np.int32)


def selection_margin(values, chosen, candidates) -> float:
    """Smallest gap between a chosen and an unchosen value (inf if none).

    A cut with a wide margin is robust to small perturbations of the values;
    used by end-to-end tests to tell near-ties from real disagreements.
    """
    chosen = set(chosen)
    cv = [float(values[i]) for i in candidates if i in chosen]
    uv = [float(values[i]) for i in candidates if i not in chosen]
    if not cv or not uv:
        return float("inf")
    return min(cv) - max(uv)
