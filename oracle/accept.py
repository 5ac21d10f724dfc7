"""Acceptance of the longest verified path through the draft tree (oracle).

Sources:
  * "EAGLE-2: Feature-Level Speculative Decoding Guide", section 3: a greedy
    or sampling verifier walks the tree from the root toward the leaves and
    accepts matching tokens up to the first discrepancy; the output equals
    plain autoregressive decoding.
  * same page, The Problem 1: classical speculative sampling (Leviathan et
    al., Chen et al.) is the accept/reject rule that keeps the target's
    distribution; "Support Eagle-3 Speculative Decoding in llama.cpp", opening
    post: acceptance and rejection of draft tokens (speculative sampling).

Readings: node 0 is the single root; greedy acceptance keeps the longest
matching root path (the lowest end index among equally long ones), which is
the first-discrepancy walk whenever sibling tokens differ; sampling tries
children in ascending node index; the bonus token is the target's choice at
the last accepted node.  For
sampling, the tree's tokens were chosen by top-k, so the draft distribution at
a node is a point mass on each child's token: accepting child token x with
probability min(1, p(x)/q(x)) becomes p_res(x), and the residual max(p - q, 0)
becomes p with the rejected tokens removed (renormalised).  Sampling decisions
are taken in fp64 from fp32 logits, fp32 uniforms and an fp32 temperature.

Uniform layout: ``U[c]`` (c >= 1) is the accept test of node c, ``U[T + u]``
the residual draw at node u; U[0] is unused.
"""
from __future__ import annotations

import numpy as np


def _children(parent):
    T = len(parent)
    kids = [[] for _ in range(T)]
    for i in range(1, T):
        kids[int(parent[i])].append(i)
    return kids


def _validate(token, parent, V=None):
    T = len(parent)
    if T < 1 or int(parent[0]) != -1:
        raise ValueError("node 0 must be the root")
    for i in range(1, T):
        p = int(parent[i])
        if not (0 <= p < i):
            raise ValueError(f"node {i}: parent {p} must be an earlier node (single root)")
    if V is not None:
        for i in range(T):
            if not (0 <= int(token[i]) < V):
                raise ValueError(f"node {i}: token out of range")


def accept_greedy(token, parent, top1):
    """Longest accepted path under the target's greedy choices.

    Node c (with parent p) matches when ``token[c] == top1[p]``; a node is
    accepted when it and every node above it (up to, not including, the root)
    match.  The path ends at the deepest accepted node, the lowest index among
    equally deep ones; with distinct sibling tokens this is the root-to-leaf
    walk that stops at the first discrepancy.  The bonus is the target's
    choice at the end node.

    Returns ``(path, n_accepted, bonus)`` with path[0] = 0 (the root).
    """
    _validate(token, parent)
    T = len(parent)
    ok = [True] + [False] * (T - 1)
    depth = [0] * T
    for c in range(1, T):
        p = int(parent[c])
        depth[c] = depth[p] + 1
        ok[c] = ok[p] and int(token[c]) == int(top1[p])
    end = 0
    for c in range(1, T):
        if ok[c] and depth[c] > depth[end]:
            end = c
    path = []
    u = end
    while u != -1:
        path.append(u)
        u = int(parent[u])
    path = path[::-1]
    return path, len(path) - 1, int(top1[end])


def _node_probs(logits_row, temperature):
    """Unnormalised fp64 probabilities exp((l - max l) / temperature)."""
    l = np.asarray(logits_row, dtype=np.float32).astype(np.float64)
    m = l.max()
    return np.exp((l - m) / np.float64(temperature))


def accept_sample(token, parent, logits, temperature: float, U, return_margin: bool = False):
    """Speculative-sampling walk with a point-mass draft at each node.

    At node u with p = exp((l_u - max) / temperature) (fp64) and
    Z_res = sum(p) minus the mass of tokens already rejected at u: try the
    children of u in ascending index; a child whose token was already
    rejected is rejected; otherwise child c with token x is accepted iff
    U[c] * Z_res < p[x], and the walk moves to c.  A rejected token's mass
    leaves Z_res.  When every child is rejected, or u is a leaf, the bonus is
    the smallest token i whose running sum over non-rejected tokens exceeds
    U[T + u] * Z_res (if rounding leaves none, the last non-rejected token
    with p > 0).

    Returns ``(path, n_accepted, bonus)``, plus the smallest decision margin
    relative to sum(p) when ``return_margin``.
    """
    T = len(parent)
    V = np.asarray(logits).shape[1]
    _validate(token, parent, V)
    if not (temperature > 0 and np.isfinite(temperature)):
        raise ValueError("temperature must be positive and finite")
    U = np.asarray(U, dtype=np.float32).astype(np.float64)
    temperature = np.float64(np.float32(temperature))   # an fp32 argument of the method
    kids = _children(parent)
    u = 0
    path = [0]
    margin = np.inf
    while True:
        p = _node_probs(logits[u], temperature)
        Z = p.sum()
        zres = Z
        rejected = []
        moved = False
        for c in kids[u]:
            x = int(token[c])
            if x in rejected:
                continue
            thr = U[c] * zres
            margin = min(margin, abs(thr - p[x]) / Z)
            if thr < p[x]:
                path.append(c)
                u = c
                moved = True
                break
            rejected.append(x)
            zres = zres - p[x]
        if moved:
            continue
        q = p.copy()
        if rejected:
            q[rejected] = 0.0
        target = U[T + u] * zres
        cdf = np.cumsum(q)
        hit = np.nonzero(cdf > target)[0]
        if hit.size:
            bonus = int(hit[0])
        else:
            bonus = int(np.nonzero(q > 0)[0][-1])
        lo = cdf[bonus - 1] if bonus > 0 else 0.0
        margin = min(margin, abs(target - lo) / Z, abs(cdf[bonus] - target) / Z)
        out = (path, len(path) - 1, bonus)
        return (*out, margin) if return_margin else out


def accept_sample_q(token, parent, target_logits, draft_logits, temperature: float, U,
                    return_margin: bool = False):
    """Speculative sampling over the tree with the draft's own distribution.

    Source: "EAGLE-2: Feature-Level Speculative Decoding Guide", The Problem 1
    (speculative sampling accepts or rejects draft tokens against the target's
    distribution) and Key Architectural Mechanics 3 (the verifier walks the
    tree from the root).  Reading for a sampled draft: the children of node u
    are draws from q_u = softmax(draft_logits[u] / temperature) without
    replacement, and they are verified by recursive rejection sampling:
    with p_1 = p_u = softmax(target_logits[u] / temperature) and q_1 = q_u,
    child i (ascending node index) with token x is accepted iff
    U[c] * q_i(x) < p_i(x), i.e. with probability min(1, p_i(x) / q_i(x)),
    and the walk moves to it; on rejection p_(i+1) = max(p_i - q_i, 0)
    renormalised and q_(i+1) = q_i without x, renormalised.  A child whose
    token was already rejected at u (no draw repeats a token) is skipped.
    When every child is rejected, or u is a leaf, the bonus is the smallest
    token whose running sum of the last residual exceeds U[T + u] times its
    total.  All fp64 from fp32 logits.

    Returns ``(path, n_accepted, bonus)``, plus the smallest decision margin
    (in probability) when ``return_margin``.
    """
    T = len(parent)
    V = np.asarray(target_logits).shape[1]
    _validate(token, parent, V)
    if not (temperature > 0 and np.isfinite(temperature)):
        raise ValueError("temperature must be positive and finite")
    U = np.asarray(U, dtype=np.float32).astype(np.float64)
    temperature = np.float64(np.float32(temperature))
    kids = _children(parent)
    u = 0
    path = [0]
    margin = np.inf
    while True:
        p = _node_probs(target_logits[u], temperature)
        p = p / p.sum()
        q = _node_probs(draft_logits[u], temperature)
        q = q / q.sum()
        rejected = []
        moved = False
        for c in kids[u]:
            x = int(token[c])
            if x in rejected:
                continue
            thr = U[c] * q[x]
            margin = min(margin, abs(thr - p[x]))
            if thr < p[x]:
                path.append(c)
                u = c
                moved = True
                break
            rejected.append(x)
            r = np.maximum(p - q, 0.0)
            p = r / r.sum()
            q = q.copy()
            q[x] = 0.0
            qs = q.sum()
            q = q / qs if qs > 0 else q
        if moved:
            continue
        target = U[T + u] * p.sum()
        cdf = np.cumsum(p)
        hit = np.nonzero(cdf > target)[0]
        bonus = int(hit[0]) if hit.size else int(np.nonzero(p > 0)[0][-1])
        lo = cdf[bonus - 1] if bonus > 0 else 0.0
        margin = min(margin, abs(target - lo), abs(cdf[bonus] - target))
        out = (path, len(path) - 1, bonus)
        return (*out, margin) if return_margin else out
