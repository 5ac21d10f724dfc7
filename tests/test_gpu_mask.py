"""GPU parity: eagle_build_tree_mask against the oracle (bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decoding_parent_amd import _lib, inputs

pytestmark = pytest.mark.gpu


def run(dev, par, words=None):
    print(f"mask T={len(par)} words={words}", flush=True)
    p = torch.from_numpy(np.asarray(par, np.int32)).to(dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    m, d = _lib.eagle_build_tree_mask(p, words=words, dev_status=st)
    torch.cuda.synchronize()
    return m.cpu().numpy().view(np.uint64), d.cpu().numpy(), int(st.item())


@pytest.mark.parametrize("T", [1, 2, 15, 60, 63, 64, 65, 128, 200, 256])
def test_random_trees(dev, T):
    for seed in range(3):
        par = inputs.random_tree(inputs.rng(100 + seed, 0, T), T, 7, 4)
        m, d, st = run(dev, par)
        rm, rd = oracle.build_tree_mask(par)
        assert st == 0
        assert np.array_equal(m, rm) and np.array_equal(d, rd)


@pytest.mark.parametrize("T", [1, 64, 65, 256])
def test_chain_star_and_extra_words(dev, T):
    for par in (inputs.chain_tree(T), inputs.star_tree(T)):
        m, d, st = run(dev, par, words=4)
        rm, rd = oracle.build_tree_mask(par, words=4)
        assert st == 0 and np.array_equal(m, rm) and np.array_equal(d, rd)


def test_workload_trees(dev):
    for w in inputs.WORKLOADS.values():
        if w.cfg == 3:
            continue
        par = inputs.tree_for(w)
        m, d, _ = run(dev, par)
        rm, rd = oracle.build_tree_mask(par)
        assert np.array_equal(m, rm) and np.array_equal(d, rd)


def test_forest_and_bad_parent(dev):
    par = np.array([-1, 0, -1, 2, 1], np.int32)
    m, d, st = run(dev, par)
    rm, rd = oracle.build_tree_mask(par)
    assert st == 0 and np.array_equal(m, rm)
    m, d, st = run(dev, np.array([-1, 0, 3, 1], np.int32))     # parent after child
    assert st & _lib.DEV_BAD_PARENT
