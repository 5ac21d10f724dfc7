"""Tree attention mask (oracle).

Source: "EAGLE-2: Feature-Level Speculative Decoding Guide", Key Architectural
Mechanics section 3 (Single-Pass Tree Verification): a draft token attends to
the tokens on its own branch (its ancestors) and never to tokens on another
branch.  Read with the chain case of section 1 (causal self-attention), a node
also sees itself, so a chain tree gives the ordinary causal mask.

Representation (the pages give none): ``parents[i]`` is the parent of node i,
-1 for a root, and a parent always precedes its child (``parents[i] < i``).
The mask is packed as ``uint64 mask[T][W]`` with ``W = ceil(T / 64)``; bit
``j % 64`` of word ``j // 64`` of row i is set exactly when node j is visible
to node i.  ``depth[i]`` counts the edges from i up to its root.
"""
from __future__ import annotations

import numpy as np


def validate_parents(parents: np.ndarray) -> None:
    T = parents.shape[0]
    for i in range(T):
        p = int(parents[i])
        if p != -1 and not (0 <= p < i):
            raise ValueError(f"parents[{i}] = {p}: a parent must be -1 or an earlier node")


def build_tree_mask(parents, words: int | None = None):
    """Return ``(mask uint64[T][W], depth int32[T])``.

    For every node i, walk up through its parents to the root, marking each
    node met, and mark i itself; the number of steps is the depth.
    """
    parents = np.asarray(parents, dtype=np.int64)
    validate_parents(parents)
    T = parents.shape[0]
    W = (T + 63) // 64 if words is None else words
    if W * 64 < T:
        raise ValueError("too few mask words for T nodes")
    mask = np.zeros((T, W), dtype=np.uint64)
    depth = np.zeros(T, dtype=np.int32)
    for i in range(T):
        seen = [i]
        j = int(parents[i])
        steps = 0
        while j != -1:
            seen.append(j)
            j = int(parents[j])
            steps += 1
        depth[i] = steps
        for b in seen:
            mask[i, b // 64] |= np.uint64(1) << np.uint64(b % 64)
    return mask, depth


def mask_bits(mask: np.ndarray, T: int) -> np.ndarray:
    """Unpack a packed mask into a bool matrix ``[rows][T]``."""
    rows = mask.shape[0]
    out = np.zeros((rows, T), dtype=bool)
    for i in range(rows):
        for j in range(T):
            out[i, j] = bool((int(mask[i, j // 64]) >> (j % 64)) & 1)
    return out


def mask_popcount(mask: np.ndarray) -> np.ndarray:
    return np.array([sum(bin(int(w)).count("1") for w in row) for row in mask], dtype=np.int64)
