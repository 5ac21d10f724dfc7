"""One full draft-and-verify cycle (oracle), composed from the pinned steps.

Sources:
  * "EAGLE-2: Feature-Level Speculative Decoding Guide", section 1 (the draft
    step h = W_fuse [f ; Emb(y)], f' = TransformerLayer(h),
    P = softmax(W_LM f')), and the Reference Implementation listing's loop,
    which pairs each drafted feature with the token it predicted before the
    next step;
  * same page, sections 2-3 (dynamic tree, single-pass tree verification);
  * "Support Eagle-3 Speculative Decoding in llama.cpp": the draft shares the
    target's embedding; confidence-driven expansion with pruning at the end of
    drafting; the target caches accepted tokens only while the draft keeps
    K/V for every candidate it expands.

Readings: the draft's feature is the layer output before the final RMSNorm,
and the LM head reads the normed feature (the printout's final ``norm``); the
root row pairs the target's feature with the root token; the fused vector
enters the decoder layer directly (no extra norm); the verify pass is stood in
for by one decoder layer with the target's own weights over the embedded tree
tokens, followed by the final norm and the shared LM head.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from ._util import f64 as _f64
from .accept import accept_sample
from .layer import LayerWeights, decoder_layer, rms_norm
from .lmhead import lm_head_logits, lm_head_topk
from .mask import build_tree_mask
from .tree import Pool, expand, rerank, selection_margin


@dataclasses.dataclass
class CycleWeights:
    w_fuse: object          # [d][2d]
    draft: LayerWeights
    draft_norm: object      # [d]
    embed: object           # [V][d]
    w_lm: object            # [V][d]
    target: LayerWeights
    target_norm: object     # [d]
    draft_k_cache: object   # [Hkv][L][hd]
    draft_v_cache: object
    target_k_cache: object
    target_v_cache: object


def draft_and_verify_cycle(cw: CycleWeights, root_token: int, root_feature, *, hq: int, hkv: int,
                           hd: int, L: int, rounds: int, k: int, k_select: int, T: int,
                           temperature: float, uniforms, theta: float = 500000.0,
                           eps: float = 1e-5):
    """Run ``rounds`` draft rounds from the root, rerank to T nodes, verify
    them in one pass and accept a path by speculative sampling.

    Returns a dict with the pool, each round's rows/top-k/frontier, the
    reranked tree, the verify logits, the accepted path and the smallest
    decision margins (top-k cut, frontier cut, rerank cut, acceptance).
    """
    embed = cw.embed
    pool = Pool.root(root_token)
    frontier = [0]
    slot_of = {0: 0}
    slot_parent = [-1]
    cap = 1 + (rounds - 1) * k_select
    d_kt = np.zeros((hkv, cap, hd))
    d_vt = np.zeros((hkv, cap, hd))
    feat = {}
    rounds_out = []
    topk_margin = np.inf
    frontier_margin = np.inf
    for r in range(rounds):
        rows = list(frontier)
        tok = [pool.token[p] for p in rows]
        fin = np.stack([_f64(root_feature) if p == 0 else feat[pool.parent[p]] for p in rows])
        emb = _f64(embed[np.asarray(tok, np.int64)])
        x = np.concatenate([fin, emb], axis=1) @ _f64(cw.w_fuse).T
        pos = np.array([L + pool.depth[p] for p in rows], np.int64)
        slots = [slot_of[p] for p in rows]
        smask, _ = build_tree_mask(np.array(slot_parent, np.int32))
        out, d_kt, d_vt = decoder_layer(x, cw.draft, pos, hq, hkv, hd, cw.draft_k_cache,
                                        cw.draft_v_cache, L, d_kt, d_vt, slots, smask, slots,
                                        theta, eps)
        for p, o in zip(rows, out):
            feat[p] = o
        z = rms_norm(out, cw.draft_norm, eps)
        lm = lm_head_topk(z, cw.w_lm, k)
        srt = -np.sort(-lm["logits"], axis=1)
        # smallest gap between consecutive logits among the top k + 1 of each row:
        # the order of the chosen ids (and the cut after k) is robust to logit
        # errors below half this gap
        row_margin = np.min(srt[:, :k] - srt[:, 1:k + 1], axis=1) if srt.shape[1] > k else \
            np.full(len(rows), np.inf)
        topk_margin = min(topk_margin, float(np.min(row_margin)))
        logp32 = lm["logp"].astype(np.float32)
        start = len(pool)
        new_frontier = expand(pool, rows, lm["ids"], logp32, k_select)
        fr_margin = selection_margin(pool.value, new_frontier, range(start, len(pool)))
        frontier_margin = min(frontier_margin, fr_margin)
        rounds_out.append({"rows": rows, "ids": lm["ids"], "logp": logp32, "lse": lm["lse"],
                           "frontier": new_frontier, "x": x, "out": out,
                           "topk_margin": row_margin, "frontier_margin": fr_margin})
        if r < rounds - 1:
            for p in new_frontier:
                slot_of[p] = len(slot_parent)
                slot_parent.append(slot_of[pool.parent[p]])
        frontier = new_frontier
    tok, par, dep, pidx = rerank(pool, T)
    rerank_margin = selection_margin(pool.value, list(pidx[1:]), range(1, len(pool)))
    mask, _ = build_tree_mask(par)
    x = _f64(embed[tok.astype(np.int64)])
    zeros = np.zeros((hkv, T, hd))
    out, _, _ = decoder_layer(x, cw.target, L + dep.astype(np.int64), hq, hkv, hd,
                              cw.target_k_cache, cw.target_v_cache, L, zeros, zeros,
                              list(range(T)), mask, list(range(T)), theta, eps)
    z = rms_norm(out, cw.target_norm, eps)
    logits = lm_head_logits(z, cw.w_lm)
    logits32 = logits.astype(np.float32)
    path, nacc, bonus, acc_margin = accept_sample(tok, par, logits32, temperature, uniforms,
                                                  return_margin=True)
    return {
        "pool": pool, "rounds": rounds_out, "node_token": tok, "node_parent": par,
        "node_depth": dep, "node_pool_idx": pidx, "mask": mask, "verify_out": out,
        "verify_logits": logits, "path": path, "n_accepted": nacc, "bonus": bonus,
        "margins": {"topk": topk_margin, "frontier": frontier_margin,
                    "rerank": rerank_margin, "accept": acc_margin},
    }
