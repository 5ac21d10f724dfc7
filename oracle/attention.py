"""Tree-masked attention of draft-tree nodes against a KV prefix (oracle).

Sources:
  * "EAGLE-2: Feature-Level Speculative Decoding Guide", Key Architectural
    Mechanics section 3: the target scores every tree node in one batched
    pass; a node attends to its ancestors only.
  * same page, section 1: the draft layer uses causal self-attention.
  * "Support Eagle-3 Speculative Decoding in llama.cpp", the
    LlamaAttention printout: q_proj 4096 -> 4096 and k_proj/v_proj
    4096 -> 1024, i.e. grouped-query attention with 32 query and 8 KV heads
    of 128 dims.

Readings where the pages are silent: scores are scaled by ``scale`` (by
default 1/sqrt(head_dim)); query head h reads KV head ``h // G`` with
``G = Hq / Hkv``; the visible set of a tree node is every prefix position plus
the tree nodes its mask row marks; masked positions are left out of the
softmax (they are not given -inf scores, they are simply absent).

Everything is computed in fp64 from the (exactly upcast) inputs.
"""
from __future__ import annotations

import numpy as np

from ._util import f64 as _f64
from .mask import mask_bits


def tree_attention(q, k_cache, v_cache, L: int, k_tree, v_tree, mask, q_mask_row=None,
                   scale: float | None = None, Tk: int | None = None) -> np.ndarray:
    """out[i][h] = sum_j softmax_j(scale * q[i][h] . k_j) v_j over the visible set.

    q: [Tq][Hq][hd]; k_cache/v_cache: [Hkv][>=L][hd]; k_tree/v_tree:
    [Hkv][>=Tk][hd]; mask: uint64 [rows][W]; q_mask_row: optional [Tq] map
    from query row to mask row (identity when None).  Returns fp64
    [Tq][Hq][hd].
    """
    q = _f64(q)
    kc, vc = _f64(k_cache), _f64(v_cache)
    kt, vt = _f64(k_tree), _f64(v_tree)
    Tq, Hq, hd = q.shape
    Hkv = kc.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if Tk is None:
        Tk = kt.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    vis_all = mask_bits(np.asarray(mask, dtype=np.uint64), Tk)
    out = np.zeros((Tq, Hq, hd), dtype=np.float64)
    for i in range(Tq):
        r = i if q_mask_row is None else int(q_mask_row[i])
        vis = np.nonzero(vis_all[r])[0]
        if L + vis.shape[0] == 0:
            raise ValueError(f"query row {i} sees nothing")
        for g in range(Hkv):
            # the G query heads h = g*G .. g*G+G-1 read KV head g: one column each
            heads = slice(g * G, (g + 1) * G)
            qg = q[i, heads].T                                        # [hd][G]
            s = np.concatenate([kc[g, :L] @ qg, kt[g, vis] @ qg], axis=0) * scale   # [L+|vis|][G]
            s = s - s.max(axis=0)
            p = np.exp(s)
            p = p / p.sum(axis=0)
            # sum over the visible set = sum over the prefix + sum over the visible tree nodes
            out[i, heads] = p[:L].T @ vc[g, :L] + p[L:].T @ vt[g, vis]
    return out
