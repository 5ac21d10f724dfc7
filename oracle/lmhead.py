"""LM head, softmax statistics and top-k (oracle).

Sources:
  * "EAGLE-2: Feature-Level Speculative Decoding Guide", Key Architectural
    Mechanics section 1: the next-token distribution is the softmax of the
    target's own LM head applied to the drafted feature, P = softmax(W_LM f).
  * same page, section 2: the confidence of a drafted token is the ratio of
    the two largest probabilities, C = P(y_(1)) / P(y_(2)); the Reference
    Implementation listing takes the two largest with a top-k of 2 and
    divides with a 1e-8 guard in the denominator.
  * "Support Eagle-3 Speculative Decoding in llama.cpp", module printout:
    every projection is ``bias=False``, so the LM head has no bias.

Readings: W is stored one row per vocabulary entry ([V][d]); the top-k order
is by logit descending with the lower index first among equal logits (+0.0
and -0.0 compare equal); log-probabilities are at temperature 1; the
confidence ratio is exp(logp_1 - logp_2), which equals P1/P2 without
dividing.  Logits and statistics are fp64.
"""
from __future__ import annotations

import numpy as np

from ._util import f64 as _f64


def lm_head_logits(f, W, row_chunk: int = 8192) -> np.ndarray:
    """logits[t][v] = sum_k f[t][k] * W[v][k], fp64 ([T][V])."""
    f = _f64(f)
    V = W.shape[0]
    out = np.empty((f.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, row_chunk):
        w = _f64(W[v0:v0 + row_chunk])
        out[:, v0:v0 + w.shape[0]] = f @ w.T
    return out


def softmax_stats(logits: np.ndarray):
    """Per row: max m, s = sum exp(l - m), lse = m + ln s (fp64)."""
    l = np.asarray(logits, dtype=np.float64)
    m = l.max(axis=-1)
    s = np.exp(l - m[..., None]).sum(axis=-1)
    return m, s, m + np.log(s)


def topk_ids(logits: np.ndarray, k: int) -> np.ndarray:
    """The k largest entries of each row, larger first, lower index first on
    equal values (a stable sort of the negated row)."""
    l = np.asarray(logits)
    order = np.argsort(-l, axis=-1, kind="stable")
    return order[..., :k].astype(np.int32)


def lm_head_topk(f, W, k: int):
    """Full LM-head step for rows of f: returns dict with ``logits`` (fp64),
    ``ids`` [T][k], ``logp`` [T][k] and ``lse`` [T]."""
    logits = lm_head_logits(f, W)
    _, _, lse = softmax_stats(logits)
    ids = topk_ids(logits, k)
    logp = np.take_along_axis(logits, ids.astype(np.int64), axis=-1) - lse[:, None]
    return {"logits": logits, "ids": ids, "logp": logp, "lse": lse}


def confidence_ratio(logp: np.ndarray) -> np.ndarray:
    """C = P(y_(1)) / P(y_(2)) = exp(logp_1 - logp_2) for each row."""
    logp = np.asarray(logp, dtype=np.float64)
    return np.exp(logp[..., 0] - logp[..., 1])
