"""Seeded synthetic inputs for one EAGLE-2 draft-and-verify cycle.

This module only draws random numbers and random tree shapes.  It holds none
of the method's arithmetic (no masks, no attention, no softmax, no selection),
so both the HIP path and the CPU oracle can be fed from it without sharing any
of the computation they are compared on.

Every draw comes from ``numpy.random.Generator(PCG64(SeedSequence([cfg,
stream, layer])))``.  Floating-point tensors are drawn in fp32 and, for bf16
workloads, rounded once to bf16 (round-to-nearest-even); the bf16 tensor is
the canonical value and an fp32 upcast of it is exact.

The pages give no datasets that this path can use (the measurements on the
pages were taken on ShareGPT prompts with trained weights); the shapes below
stand in for them.  Shapes follow the Llama-3-8B printout on the "Support
Eagle-3 Speculative Decoding" page (the yuhuili/EAGLE3-LLaMA3.1-Instruct-8B
module tree), the Qwen2-7B pairing on the llama.cpp "EAGLE-2 Speculative
Decoding Support - Phase 1" page (Demonstrated Performance), and the tree
limits on the "EAGLE-2: Feature-Level Speculative Decoding Guide" page
(Context-Aware Dynamic Tree Construction: chains up to 7 deep, 2 to 4
branches).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

# Stream ids of the seed sequence [cfg, stream, layer].
STREAM_TREE = 0
STREAM_Q = 1
STREAM_KC = 2
STREAM_VC = 3
STREAM_KT = 4
STREAM_VT = 5
STREAM_F = 6
STREAM_W = 7
STREAM_TOK = 8
STREAM_U = 9
STREAM_LOGITS = 10     # synthetic target logits for the acceptance step
STREAM_LOGP = 11       # synthetic child log-probs for expand/rerank
STREAM_WEIGHTS = 20    # 20 + i: the i-th weight matrix of the cycle's layers


def rng(cfg: int, stream: int, layer: int = 0) -> np.random.Generator:
    """The one generator every synthetic tensor is drawn from."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, stream, layer])))


def normal(g: np.random.Generator, shape, std: float = 1.0, dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, std^2) drawn in fp32, then rounded once to ``dtype`` (CPU tensor)."""
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    t = torch.from_numpy(x)
    return t if dtype == torch.float32 else t.to(dtype)


def small_ints(g: np.random.Generator, shape, lo: int, hi: int, scale: float = 1.0,
               dtype=torch.bfloat16) -> torch.Tensor:
    """Integers in [lo, hi] times a power-of-two ``scale``.

    Used for contraction tests whose every partial sum is exactly
    representable in fp32, so that any summation order gives the same bits.
    """
    x = g.integers(lo, hi + 1, size=shape).astype(np.float32) * np.float32(scale)
    t = torch.from_numpy(x)
    return t if dtype == torch.float32 else t.to(dtype)


def uniforms(g: np.random.Generator, n: int) -> np.ndarray:
    """fp32 uniforms in [0, 1)."""
    return g.random(n, dtype=np.float32)


def random_tree(g: np.random.Generator, T: int, max_depth: int, max_branch: int,
                complete_levels: int = 0, complete_branch: int = 0) -> np.ndarray:
    """Random draft tree as a parent array (node 0 is the root, parent -1).

    Node i > 0 picks its parent uniformly among the earlier nodes that are
    shallower than ``max_depth`` and have fewer than ``max_branch`` children,
    so parents precede children, depth <= max_depth and branching is
    1..max_branch.  With ``complete_levels`` > 0 the first levels are built
    complete with ``complete_branch`` children per node first (a wide tree near
    the root).
    """
    parents = np.full(T, -1, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int64)
    children = np.zeros(T, dtype=np.int64)
    n = 1
    if complete_levels > 0:
        level = [0]
        for lv in range(complete_levels):
            nxt = []
            for p in level:
                for _ in range(complete_branch):
                    if n >= T:
                        break
                    parents[n] = p
                    depth[n] = depth[p] + 1
                    children[p] += 1
                    nxt.append(n)
                    n += 1
            level = nxt
    for i in range(n, T):
        ok = np.nonzero((depth[:i] < max_depth) & (children[:i] < max_branch))[0]
        if ok.size == 0:
            raise ValueError("tree generator ran out of open slots")
        p = int(ok[g.integers(0, ok.size)])
        parents[i] = p
        depth[i] = depth[p] + 1
        children[p] += 1
    return parents


def chain_tree(T: int) -> np.ndarray:
    """A chain: node i's parent is i - 1 (linear speculation)."""
    return np.arange(-1, T - 1, dtype=np.int32)


def star_tree(T: int) -> np.ndarray:
    """A star: every node hangs off the root."""
    p = np.zeros(T, dtype=np.int32)
    p[0] = -1
    return p


def sibling_distinct_tokens(g: np.random.Generator, parents: np.ndarray, V: int) -> np.ndarray:
    """Tokens uniform in [0, V), distinct among the children of each node."""
    T = parents.shape[0]
    tok = np.zeros(T, dtype=np.int32)
    tok[0] = g.integers(0, V)
    kids = {}
    for i in range(1, T):
        kids.setdefault(int(parents[i]), []).append(i)
    for p in sorted(kids):
        c = kids[p]
        if len(c) > V:
            raise ValueError("more siblings than vocabulary entries")
        tok[c] = g.choice(V, size=len(c), replace=False)
    return tok


def plant_path(tokens: np.ndarray, parents: np.ndarray, top1: np.ndarray, leaf: int) -> np.ndarray:
    """Rewrite tokens so the root->leaf path follows ``top1`` at every parent.

    ``top1[u]`` is the target's choice at node u (given to this function; it is
    not computed here).  A sibling that already holds the planted token swaps
    tokens with the path node, keeping siblings distinct.
    """
    tok = tokens.copy()
    path = []
    u = leaf
    while u > 0:
        path.append(u)
        u = int(parents[u])
    for c in reversed(path):
        p = int(parents[c])
        want = int(top1[p])
        for s in np.nonzero(parents == p)[0]:
            if s != c and tok[s] == want:
                tok[s] = tok[c]
        tok[c] = want
    return tok


def deepest_leaf(g: np.random.Generator, parents: np.ndarray) -> int:
    """A uniformly chosen node of maximal depth (generator bookkeeping only)."""
    T = parents.shape[0]
    depth = np.zeros(T, dtype=np.int64)
    for i in range(1, T):
        depth[i] = depth[parents[i]] + 1
    cands = np.nonzero(depth == depth.max())[0]
    return int(cands[g.integers(0, cands.size)])


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload."""
    cfg: int
    name: str
    d: int
    hq: int
    hkv: int
    hd: int
    vocab: int
    L: int
    T: int
    max_depth: int
    max_branch: int
    topk: int
    dtype: str                  # "f32" or "bf16"
    sampling: bool = False
    greedy: bool = True
    complete_levels: int = 0
    complete_branch: int = 0
    layers: int = 1             # stacked KV caches run in sequence
    ffn: int = 0                # SwiGLU width of the cycle's decoder layer
    rounds: int = 0             # draft expansion rounds of the cycle
    k_select: int = 0           # frontier width kept per round
    temperature: float = 1.0
    rope_theta: float = 500000.0
    rms_eps: float = 1e-5

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def words(self) -> int:
        return (self.T + 63) // 64


TINY = Workload(cfg=1, name="tiny", d=256, hq=4, hkv=1, hd=64, vocab=1024, L=128, T=15,
                max_depth=4, max_branch=3, topk=4, dtype="f32")
QWEN2_7B_VERIFY = Workload(cfg=2, name="qwen2-7b-verify", d=3584, hq=28, hkv=4, hd=128,
                           vocab=152064, L=2048, T=60, max_depth=7, max_branch=4, topk=10,
                           dtype="bf16")
LLAMA3_8B_CYCLE = Workload(cfg=3, name="llama3-8b-cycle", d=4096, hq=32, hkv=8, hd=128,
                           vocab=128256, L=4096, T=64, max_depth=6, max_branch=10, topk=10,
                           dtype="bf16", sampling=True, greedy=False, ffn=14336, rounds=6,
                           k_select=10)
LONG_CONTEXT = Workload(cfg=4, name="llama3-8b-long-verify", d=4096, hq=32, hkv=8, hd=128,
                        vocab=128256, L=32768, T=64, max_depth=7, max_branch=4, topk=10,
                        dtype="bf16", layers=32)
WIDE_70B = Workload(cfg=5, name="70b-wide-tree", d=8192, hq=64, hkv=8, hd=128, vocab=128256,
                    L=8192, T=128, max_depth=7, max_branch=4, topk=10, dtype="bf16",
                    sampling=True, greedy=True, complete_levels=2, complete_branch=4)

WORKLOADS = {w.cfg: w for w in (TINY, QWEN2_7B_VERIFY, LLAMA3_8B_CYCLE, LONG_CONTEXT, WIDE_70B)}


def tree_for(w: Workload, layer: int = 0) -> np.ndarray:
    g = rng(w.cfg, STREAM_TREE, layer)
    return random_tree(g, w.T, w.max_depth, w.max_branch, w.complete_levels, w.complete_branch)


def torch_dtype(w: Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


@dataclasses.dataclass
class VerifyInputs:
    """Inputs of one verify pass (mask -> attention -> LM head -> accept)."""
    parents: np.ndarray
    tokens: np.ndarray
    q: torch.Tensor        # [T][Hq][hd]
    k_cache: torch.Tensor  # [Hkv][L][hd]
    v_cache: torch.Tensor  # [Hkv][L][hd]
    k_tree: torch.Tensor   # [Hkv][T][hd]
    v_tree: torch.Tensor   # [Hkv][T][hd]
    f: torch.Tensor        # [T][d]
    uniforms: np.ndarray   # [2T]


def verify_inputs(w: Workload, layer: int = 0, T: Optional[int] = None, L: Optional[int] = None,
                  with_lmhead: bool = True) -> VerifyInputs:
    """Draw one verify pass's inputs at workload ``w`` (optionally with a
    smaller T or L for CPU-sized parity cases)."""
    T = w.T if T is None else T
    L = w.L if L is None else L
    dt = torch_dtype(w)
    ww = dataclasses.replace(w, T=T)
    parents = tree_for(ww, layer)
    tokens = sibling_distinct_tokens(rng(w.cfg, STREAM_TOK, layer), parents, w.vocab)
    q = normal(rng(w.cfg, STREAM_Q, layer), (T, w.hq, w.hd), dtype=dt)
    kc = normal(rng(w.cfg, STREAM_KC, layer), (w.hkv, L, w.hd), dtype=dt)
    vc = normal(rng(w.cfg, STREAM_VC, layer), (w.hkv, L, w.hd), dtype=dt)
    kt = normal(rng(w.cfg, STREAM_KT, layer), (w.hkv, T, w.hd), dtype=dt)
    vt = normal(rng(w.cfg, STREAM_VT, layer), (w.hkv, T, w.hd), dtype=dt)
    f = normal(rng(w.cfg, STREAM_F, layer), (T, w.d), dtype=dt) if with_lmhead else None
    u = uniforms(rng(w.cfg, STREAM_U, layer), 2 * T)
    return VerifyInputs(parents, tokens, q, kc, vc, kt, vt, f, u)


def lm_head_weight(w: Workload, vocab: Optional[int] = None, d: Optional[int] = None) -> torch.Tensor:
    """W_LM ~ N(0, 1/d), stored [V][d] (one row per token)."""
    V = w.vocab if vocab is None else vocab
    d = w.d if d is None else d
    return normal(rng(w.cfg, STREAM_W), (V, d), std=float(1.0 / np.sqrt(d)), dtype=torch_dtype(w))


# --------------------------------------------------------------------------
# Synthetic weights of one draft-and-verify cycle
# --------------------------------------------------------------------------

def _w(w: Workload, idx: int, shape, std: float, dtype=torch.bfloat16) -> torch.Tensor:
    return normal(rng(w.cfg, STREAM_WEIGHTS + idx), shape, std=std, dtype=dtype)


def layer_weights(w: Workload, base: int) -> dict:
    """One Llama decoder layer: W ~ N(0, 1/fan_in), RMSNorm gains 1.  q/k/v are
    stored as one [(Hq + 2 Hkv) hd][d] matrix (q rows, then k, then v)."""
    d, hd, F = w.d, w.hd, w.ffn
    nq = (w.hq + 2 * w.hkv) * hd
    return {
        "norm1": torch.ones(d, dtype=torch.float32),
        "wqkv": _w(w, base + 0, (nq, d), float(1 / np.sqrt(d))),
        "wo": _w(w, base + 1, (d, w.hq * hd), float(1 / np.sqrt(w.hq * hd))),
        "norm2": torch.ones(d, dtype=torch.float32),
        "wgate": _w(w, base + 2, (F, d), float(1 / np.sqrt(d))),
        "wup": _w(w, base + 3, (F, d), float(1 / np.sqrt(d))),
        "wdown": _w(w, base + 4, (d, F), float(1 / np.sqrt(F))),
    }


def cycle_inputs(w: Workload) -> dict:
    """Every input of one cycle (CPU tensors): the draft's fuse matrix and
    layer, the target's stand-in layer, the shared embedding and LM head, both
    KV prefixes, the root token and feature, and the acceptance uniforms."""
    d, hd = w.d, w.hd
    g_root = rng(w.cfg, STREAM_F)
    return {
        "w_fuse": _w(w, 0, (d, 2 * d), float(1 / np.sqrt(2 * d))),
        "draft": layer_weights(w, 1),
        "draft_norm": torch.ones(d, dtype=torch.float32),
        "target": layer_weights(w, 10),
        "target_norm": torch.ones(d, dtype=torch.float32),
        "embed": _w(w, 20, (w.vocab, d), 1.0),
        "w_lm": lm_head_weight(w),
        "draft_k_cache": normal(rng(w.cfg, STREAM_KC, 1), (w.hkv, w.L, hd)),
        "draft_v_cache": normal(rng(w.cfg, STREAM_VC, 1), (w.hkv, w.L, hd)),
        "target_k_cache": normal(rng(w.cfg, STREAM_KC, 0), (w.hkv, w.L, hd)),
        "target_v_cache": normal(rng(w.cfg, STREAM_VC, 0), (w.hkv, w.L, hd)),
        "root_feature": normal(g_root, (d,), dtype=torch.float32),
        "root_token": int(rng(w.cfg, STREAM_TOK).integers(0, w.vocab)),
        "uniforms": uniforms(rng(w.cfg, STREAM_U), 2 * w.T),
    }


SMALL_CYCLE = Workload(cfg=13, name="small-cycle", d=256, hq=4, hkv=2, hd=64, vocab=1024, L=64,
                       T=16, max_depth=4, max_branch=4, topk=4, dtype="bf16", sampling=True,
                       greedy=False, ffn=512, rounds=4, k_select=4)


def device_normal(shape, seed: int, device, dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, 1) drawn on the GPU with torch's seeded Philox generator, rounded
    once to ``dtype``.  Used where the host draw would dominate the run time
    (gigabytes of KV cache for throughput measurement); parity cases use the
    host generators above."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, device=device, generator=g, dtype=torch.float32).to(dtype)
