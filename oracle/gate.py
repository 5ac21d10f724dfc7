"""Confidence-gated branching of a drafted node (oracle).

Source: "EAGLE-2: Feature-Level Speculative Decoding Guide", Key
Architectural Mechanics 2: the confidence of a drafted node is
C = P(y_(1)) / P(y_(2)); above a threshold tau the draft spends its budget on
depth (a linear chain), at or below it on breadth (2 to 4 branches at that
node); the Reference Implementation listing uses tau = 2.0.

Reading (the pages do not say which 2 to 4): a node keeps the children whose
probability is at least P(y_(1)) / tau, at most ``max_branch`` of them.  Since
the candidates are sorted, that is one child exactly when C > tau (a chain)
and between 2 and ``max_branch`` children otherwise.  In log-probabilities, as
the LM head produces them, child j is kept when logp_j - logp_0 >= -ln(tau),
evaluated in fp32 with ln(tau) rounded once to fp32.  Children that are not
kept get log-probability -inf: the expansion then gives them value -inf, so
they rank below every kept candidate and only fill a budget the kept ones
cannot (verification stays lossless whatever the draft tokens are).
"""
from __future__ import annotations

import numpy as np


def gate_children(logp, tau: float, max_branch: int):
    """``logp`` float32 [rows][k], each row sorted descending (the LM head's
    top-k log-probs).  Returns (gated logp float32 [rows][k], kept int32
    [rows], confidence float32 [rows] = exp(logp_0 - logp_1))."""
    lp = np.asarray(logp, dtype=np.float32)
    rows, k = lp.shape
    neg_ln_tau = np.float32(-np.log(np.float64(tau)))
    out = np.full_like(lp, -np.inf)
    kept = np.zeros(rows, np.int32)
    conf = np.full(rows, np.inf, np.float32)
    for r in range(rows):
        n = 0
        for j in range(k):
            if n < max_branch and np.float32(lp[r, j] - lp[r, 0]) >= neg_ln_tau:
                out[r, j] = lp[r, j]
                n += 1
        kept[r] = n
        if k > 1:
            with np.errstate(over="ignore", invalid="ignore"):
                conf[r] = np.exp(np.float32(lp[r, 0] - lp[r, 1]), dtype=np.float32)
    return out, kept, conf
