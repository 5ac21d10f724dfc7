"""Pins of the oracle's Eagle-3 fusion: the product splits into the three
block products of W's column blocks; selecting one block with an identity
returns that hidden state exactly; swapping two segments together with the
matching column blocks leaves g unchanged; and a brute-force sum."""
import numpy as np

from oracle.fusion import fuse3
from speculative_decoding_parent_amd import inputs


def draw(M, d, N, seed):
    g = inputs.rng(62, seed)
    h = [g.standard_normal((M, d)).astype(np.float32) for _ in range(3)]
    W = (g.standard_normal((N, 3 * d)) / np.sqrt(3 * d)).astype(np.float32)
    return h, W


def test_block_decomposition():
    (lo, mi, hi), W = draw(5, 16, 12, 0)
    d = 16
    want = lo.astype(np.float64) @ W[:, :d].T.astype(np.float64)
    want += mi.astype(np.float64) @ W[:, d:2 * d].T.astype(np.float64)
    want += hi.astype(np.float64) @ W[:, 2 * d:].T.astype(np.float64)
    np.testing.assert_allclose(fuse3(lo, mi, hi, W), want, rtol=0, atol=1e-12)


def test_identity_blocks_select_each_state():
    (lo, mi, hi), _ = draw(4, 8, 8, 1)
    d = 8
    for b, h in enumerate((lo, mi, hi)):
        W = np.zeros((d, 3 * d), np.float32)
        W[:, b * d:(b + 1) * d] = np.eye(d, dtype=np.float32)
        assert np.array_equal(fuse3(lo, mi, hi, W), h.astype(np.float64))


def test_segment_swap_invariance():
    (lo, mi, hi), W = draw(3, 8, 6, 2)
    d = 8
    Wp = np.concatenate([W[:, 2 * d:], W[:, d:2 * d], W[:, :d]], axis=1)
    np.testing.assert_allclose(fuse3(hi, mi, lo, Wp), fuse3(lo, mi, hi, W), rtol=0, atol=1e-12)


def test_brute_force():
    (lo, mi, hi), W = draw(2, 4, 3, 3)
    x = [list(lo[m]) + list(mi[m]) + list(hi[m]) for m in range(2)]
    for m in range(2):
        for n in range(3):
            s = sum(float(x[m][k]) * float(W[n, k]) for k in range(12))
            assert abs(fuse3(lo, mi, hi, W)[m, n] - s) < 1e-12
