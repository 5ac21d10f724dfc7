"""One Llama decoder layer over draft-tree rows (oracle).

Sources:
  * "Support Eagle-3 Speculative Decoding in llama.cpp", module printout of
    yuhuili/EAGLE3-LLaMA3.1-Instruct-8B: LlamaDecoderLayer with q/k/v/o
    projections 4096 -> 4096/1024/1024/4096, an MLP with gate/up 4096 -> 14336
    and down 14336 -> 4096 under SiLU, input and post-attention RMSNorms with
    eps 1e-5, a final RMSNorm and a rotary embedding; no biases.
  * "EAGLE-2: Feature-Level Speculative Decoding Guide", section 1: the
    draft's single decoder layer uses causal self-attention; with a tree the
    causal order becomes the tree mask (section 3).

Readings: the MLP is SwiGLU, down(silu(gate(x)) * up(x)), which is what
LlamaMLP computes with ``act_fn`` SiLU; the layer is pre-norm with residuals
around attention and MLP; RoPE uses the rotate-half pairing (dims i and
i + hd/2) with base theta 500000 and no frequency scaling; a tree node's
position is L + its depth.  All fp64.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from ._util import f64 as _f64
from .attention import tree_attention


def rms_norm(x, gamma, eps: float = 1e-5) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis."""
    x = _f64(x)
    g = _f64(gamma)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def silu(x) -> np.ndarray:
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def linear(x, W) -> np.ndarray:
    """x W^T for W stored [out][in] (nn.Linear without bias)."""
    return _f64(x) @ _f64(W).T


def swiglu_mlp_hidden(x, w_gate, w_up) -> np.ndarray:
    """LlamaMLP hidden activation silu(x W_gate^T) * (x W_up^T)."""
    return silu(linear(x, w_gate)) * linear(x, w_up)


def rope(x, pos, theta: float = 500000.0) -> np.ndarray:
    """Rotate [rows][H][hd] by position: pair (i, i + hd/2) turns by
    pos * theta^(-2i/hd)."""
    x = _f64(x)
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]     # [rows][half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


@dataclasses.dataclass
class LayerWeights:
    """Weights of one decoder layer, stored [out][in] as nn.Linear does."""
    norm1: object       # [d]
    wq: object          # [Hq*hd][d]
    wk: object          # [Hkv*hd][d]
    wv: object          # [Hkv*hd][d]
    wo: object          # [d][Hq*hd]
    norm2: object       # [d]
    wgate: object       # [F][d]
    wup: object         # [F][d]
    wdown: object       # [d][F]


def decoder_layer(x, w: LayerWeights, pos, hq: int, hkv: int, hd: int,
                  k_cache, v_cache, L: int, k_tree, v_tree, slots, mask, mask_rows,
                  theta: float = 500000.0, eps: float = 1e-5):
    """Run the layer on rows x [n][d].

    Row r's key and value (after RoPE for the key) are written into the tree
    K/V at ``slots[r]`` before attention, so a row sees itself.  Row r
    attends to the prefix and to the tree slots marked in mask row
    ``mask_rows[r]``.  Returns ``(out [n][d], k_tree, v_tree)`` with the tree
    K/V updated (fp64 copies).
    """
    x = _f64(x)
    n = x.shape[0]
    h = rms_norm(x, w.norm1, eps)
    q = (h @ _f64(w.wq).T).reshape(n, hq, hd)
    k = (h @ _f64(w.wk).T).reshape(n, hkv, hd)
    v = (h @ _f64(w.wv).T).reshape(n, hkv, hd)
    q = rope(q, pos, theta)
    k = rope(k, pos, theta)
    kt = _f64(k_tree).copy()
    vt = _f64(v_tree).copy()
    for r in range(n):
        kt[:, slots[r]] = k[r]
        vt[:, slots[r]] = v[r]
    a = tree_attention(q, k_cache, v_cache, L, kt, vt, mask, q_mask_row=mask_rows)
    x2 = x + a.reshape(n, hq * hd) @ _f64(w.wo).T
    h2 = rms_norm(x2, w.norm2, eps)
    m = silu(h2 @ _f64(w.wgate).T) * (h2 @ _f64(w.wup).T)
    out = x2 + m @ _f64(w.wdown).T
    return out, kt, vt
