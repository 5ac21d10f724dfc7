"""Pins of the oracle's speculative sampling with a draft distribution q.

The losslessness that speculative sampling guarantees is checked exactly:
for a node whose children are drawn from q without replacement, the
distribution of the first emitted token, summed over every ordered draw,
equals the target's p.  The oracle's uniform-driven decisions are then
checked against those acceptance probabilities by Monte Carlo, and two
special cases reduce it to closed forms: q = p accepts the first child, and
a point-mass q on a chain gives the point-mass walk (accept_sample)."""
import itertools

import numpy as np
import pytest

from oracle.accept import accept_sample, accept_sample_q
from speculative_decoding_parent_amd import inputs


def softmax(l, t=1.0):
    e = np.exp((np.asarray(l, np.float64) - np.max(l)) / t)
    return e / e.sum()


def emit_distribution(p, q, draw):
    """First-token distribution for one ordered draw (probability domain)."""
    out = np.zeros_like(p)
    reach = 1.0
    p = p.copy()
    q = q.copy()
    for x in draw:
        a = min(1.0, p[x] / q[x])
        out[x] += reach * a
        reach *= 1.0 - a
        r = np.maximum(p - q, 0.0)
        if r.sum() > 0:
            p = r / r.sum()
        q[x] = 0.0
        if q.sum() > 0:
            q = q / q.sum()
    return out + reach * p


@pytest.mark.parametrize("V,m,seed", [(5, 2, 0), (5, 3, 1), (6, 4, 2), (4, 4, 3)])
def test_lossless_by_enumeration(V, m, seed):
    g = inputs.rng(64, seed)
    p = softmax(g.standard_normal(V) * 1.5)
    q = softmax(g.standard_normal(V) * 1.5)
    total = np.zeros(V)
    mass = 0.0
    for draw in itertools.permutations(range(V), m):
        pr = 1.0
        rem = q.copy()
        for x in draw:
            pr *= rem[x] / rem.sum()
            rem[x] = 0.0
        total += pr * emit_distribution(p, q, draw)
        mass += pr
    assert abs(mass - 1.0) < 1e-12
    np.testing.assert_allclose(total, p, rtol=0, atol=1e-12)


def test_oracle_decisions_follow_the_acceptance_probabilities():
    """One root with three leaf children of fixed tokens: the oracle's
    emitted first token over many uniform draws matches emit_distribution."""
    V, T = 6, 4
    g = inputs.rng(65, 0)
    tl = (g.standard_normal((T, V)) * 1.2).astype(np.float32)
    dl = (g.standard_normal((T, V)) * 1.2).astype(np.float32)
    par = np.array([-1, 0, 0, 0], np.int32)
    tok = np.array([0, 4, 1, 3], np.int32)
    want = emit_distribution(softmax(tl[0].astype(np.float64)), softmax(dl[0].astype(np.float64)),
                             [4, 1, 3])
    n = 20000
    counts = np.zeros(V)
    for s in range(n):
        U = inputs.uniforms(inputs.rng(66, s), 2 * T)
        path, nacc, bonus = accept_sample_q(tok, par, tl, dl, 1.0, U)
        counts[int(tok[path[1]]) if nacc else bonus] += 1
    sd = np.sqrt(want * (1 - want) / n)
    assert np.all(np.abs(counts / n - want) <= 5 * sd + 1e-9)


def test_q_equal_p_accepts_the_first_child():
    g = inputs.rng(67, 0)
    T, V = 5, 30
    lg = g.standard_normal((T, V)).astype(np.float32)
    par = np.array([-1, 0, 0, 1, 1], np.int32)
    tok = np.array([0, 3, 4, 5, 6], np.int32)
    for s in range(50):
        U = inputs.uniforms(inputs.rng(68, s), 2 * T)
        path, nacc, _ = accept_sample_q(tok, par, lg, lg, 1.0, U)
        assert path[:3] == [0, 1, 3] and nacc == 2


def test_point_mass_chain_equals_point_mass_walk():
    g = inputs.rng(69, 0)
    T, V = 6, 40
    par = np.arange(-1, T - 1, dtype=np.int32)
    tok = g.integers(0, V, T).astype(np.int32)
    tl = (g.standard_normal((T, V)) * 2).astype(np.float32)
    dl = np.full((T, V), -1.0e4, np.float32)
    for u in range(T - 1):
        dl[u, tok[u + 1]] = 0.0                       # q_u is the point mass on the child's token
    for s in range(200):
        U = inputs.uniforms(inputs.rng(70, s), 2 * T)
        a = accept_sample_q(tok, par, tl, dl, 0.9, U)
        b = accept_sample(tok, par, tl, 0.9, U)
        assert a == b
