"""Eagle-3 feature fusion (oracle).

Source: "Support Eagle-3 Speculative Decoding in llama.cpp": the opening post
records the target's hidden states after its first, middle and last decoder
layers (low, middle and high-level features); the replies describe the draft
as two FC layers, one decoder layer and the LM head, the first FC mapping the
three recorded states to one feature g that feeds the decoder layer.

Reading: g = W_fc [h_low ; h_mid ; h_high], the three concatenated in that
order along the feature axis, no bias (the draft's layers carry none).  fp64.
"""
from __future__ import annotations

import numpy as np

from ._util import f64 as _f64


def fuse3(h_low, h_mid, h_high, W_fc) -> np.ndarray:
    """``h_*`` [M][d], ``W_fc`` [N][3 d] -> g [M][N] (fp64)."""
    x = np.concatenate([_f64(h_low), _f64(h_mid), _f64(h_high)], axis=1)
    return x @ _f64(W_fc).T
