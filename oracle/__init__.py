"""CPU oracle for one EAGLE-2 draft-and-verify cycle.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the hot path computes, written from the pages' description
of EAGLE-2 in numpy (fp64 for floating point, except where the method's own
definition fixes a narrower type: cumulative tree values are single fp32
additions, and sampling decisions are taken in fp64).  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path in
``speculative_decoding_parent_amd`` and imports nothing from it; the product
path never calls it.

Sources (the pages):
  * "EAGLE-2: Feature-Level Speculative Decoding Guide" (aifetchly blog),
    Key Architectural Mechanics sections 1-3 and the Reference Implementation
    listing;
  * "Support Eagle-3 Speculative Decoding in llama.cpp" (llama.cpp discussion
    #15902), the opening post, the yuhuili/EAGLE3-LLaMA3.1-Instruct-8B
    module printout and the reply on the draft's KV cache and its eviction;
  * "EAGLE-2 Speculative Decoding Support for llama.cpp - Phase 1" (llama.cpp
    PR #13908), Implementation Characteristics (single-sequence inference)
    and the test setup (mixed sampling: temperature, top_k, top_p).

Parity status: every public function here, the layer's building blocks
(``linear``, ``swiglu_mlp_hidden``, ``rms_norm``, ``silu``, ``rope``) included,
is pinned by tests under ``tests/`` that run without a GPU: closed forms,
library routines on special cases, brute force on tiny integer inputs, and
invariants the pages state.  No function is parity unpinned.
"""
from .mask import build_tree_mask, mask_bits, mask_popcount  # noqa: F401
from .attention import tree_attention  # noqa: F401
from .lmhead import lm_head_logits, softmax_stats, topk_ids, lm_head_topk, confidence_ratio  # noqa: F401
from .tree import Pool, expand, rerank  # noqa: F401
from .accept import accept_greedy, accept_sample, accept_sample_q  # noqa: F401
from .layer import rms_norm, rope, silu, linear, swiglu_mlp_hidden, decoder_layer, LayerWeights  # noqa: F401
from .cycle import CycleWeights, draft_and_verify_cycle  # noqa: F401
from .kv import kv_commit, kv_commit_in_place  # noqa: F401
from .gate import gate_children  # noqa: F401
from .fusion import fuse3  # noqa: F401
from .sampling import process_logits  # noqa: F401
