"""Mixed-sampling logits processor: temperature, top-k, top-p (oracle).

Source: "EAGLE-2 Speculative Decoding Support for llama.cpp - Phase 1": the
acceleration is measured with mixed sampling (temperature + top_k + top_p);
"EAGLE-2: Feature-Level Speculative Decoding Guide", Key Architectural
Mechanics 3: a greedy or nucleus-sampling verifier walks the tree.  The
verifier's target distribution is then the processed one.

Readings (the pages name the three controls only):
  * top-k keeps the k tokens with the largest logits, ranked by (logit
    descending, token index ascending) - the order every selection here uses;
    k = 0 keeps all V tokens;
  * top-p works on those k tokens in that order with probabilities
    p_j = exp((l_j - l_max) / temperature) (fp64) and keeps the shortest
    prefix whose mass reaches top_p times the mass of all k: token j stays
    while the mass before it is below that; top_p = 1 keeps all k;
  * the output is the logits with every removed token set to -inf, so the
    sampling verifier (which applies the temperature itself) sees exactly
    the renormalised processed distribution.
"""
from __future__ import annotations

import numpy as np


def process_logits(logits, temperature: float, top_k: int, top_p: float):
    """``logits`` float32 [T][V] -> (processed float32 [T][V], kept int32 [T],
    margin float64 [T]).  ``margin`` is, for rows where top-p cut the list,
    the distance |mass before the cut - top_p * total| relative to the total
    (how close the decision was), else +inf."""
    lg = np.asarray(logits, dtype=np.float32)
    T, V = lg.shape
    k = V if top_k <= 0 or top_k >= V else int(top_k)
    out = np.full_like(lg, -np.inf)
    kept = np.zeros(T, np.int32)
    margin = np.full(T, np.inf)
    for t in range(T):
        row = lg[t]
        order = np.lexsort((np.arange(V), -row.astype(np.float64)))[:k]   # logit desc, index asc
        keep = k
        if top_p < 1.0:
            lv = row[order].astype(np.float64)
            p = np.exp((lv - lv[0]) / np.float64(np.float32(temperature)))
            total = p.sum()
            target = np.float64(np.float32(top_p)) * total
            before = 0.0
            keep = 0
            for j in range(k):
                if before >= target:
                    break
                keep += 1
                before += p[j]
            if keep < k:
                cut_before = before                     # mass of the kept prefix
                margin[t] = min(abs(cut_before - target), abs(cut_before - p[keep - 1] - target)) / total
        sel = order[:keep]
        out[t, sel] = row[sel]
        kept[t] = keep
    return out, kept, margin
