"""Python binding of the eagle.h C ABI (argument marshalling only).

Every function here has the name of the C entry point it calls, takes torch
tensors where the C call takes device pointers, and enqueues on torch's
current HIP stream.  Output and workspace tensors may be passed in; when they
are not, they are allocated with torch (device memory is the only thing torch
provides).  Every step of the path runs in libeagle.so; if the library is
missing this module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libeagle.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "eagle.h")

EAGLE_OK, EAGLE_EINVAL, EAGLE_EUNSUPPORTED, EAGLE_EWORKSPACE, EAGLE_EHIP = 0, -1, -2, -3, -4
EAGLE_F32, EAGLE_BF16 = 0, 1
EAGLE_EXPAND, EAGLE_RERANK = 0, 1
EAGLE_GREEDY, EAGLE_SAMPLE = 0, 1
DEV_BAD_PARENT, DEV_BAD_ROOT, DEV_BAD_TOKEN, DEV_BAD_INDEX, DEV_ORPHAN, DEV_PATH_TRUNC = (
    1, 2, 4, 8, 16, 32)
DEV_TIMEOUT = 64

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

_PROTOS = {
    "eagle_abi_version": (_I32, []),
    "eagle_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "eagle_build_tree_mask": (_I32, [_P, _I32, _I32, _P, _P, _P, _P]),
    "eagle_tree_attn_workspace": (_SZ, [_I32, _I32, _I32, _I32, _I64, _I32, ctypes.c_int]),
    "eagle_tree_attn": (_I32, [_P, _P, _P, _I64, _I64, _P, _P, _I32, _I32, _P, _I32, _I32, _P,
                               _I32, _I32, _I32, _I32, _F32, ctypes.c_int, ctypes.c_int, _P, _P,
                               _SZ, _P, _P]),
    "eagle_lmhead_topk_workspace": (_SZ, [_I32, _I32, _I32, _I32, ctypes.c_int]),
    "eagle_lmhead_topk": (_I32, [_P, _P, _I32, _I32, _I32, _I32, ctypes.c_int, _P, _I32, _F32, _P,
                                 _P, _P, _P, _P, _SZ, _P]),
    "eagle_lmhead_topk_noalloc": (_I32, [_P, _P, _I32, _I32, _I32, _I32, ctypes.c_int, _P, _I32,
                                         _F32, _P, _P, _P, _P, _P]),
    "eagle_expand_rerank": (_I32, [_I32, _P, _P, _P, _P, _I32, _I32, _P, _I32, _P, _P, _I32, _I32,
                                   _P, _I32, _P, _P, _P, _P, _P, _P]),
    "eagle_accept_workspace": (_SZ, [_I32, _I32]),
    "eagle_accept": (_I32, [_I32, _I32, _P, _P, _P, _I32, _P, _I32, _F32, _P, _I32, _P, _P, _P, _P,
                            _SZ, _P, _P]),
    "eagle_linear_workspace": (_SZ, [_I32, _I32, _I32, _I32]),
    "eagle_linear": (_I32, [_P, _I32, _I32, _P, _I32, _P, _P, ctypes.c_int, _P, _SZ, _P]),
    "eagle_linear_swiglu": (_I32, [_P, _I32, _I32, _P, _I32, _F32, _P, _P, _I32, _P, _P, _SZ, _P]),
    "eagle_rmsnorm": (_I32, [_P, _P, _I32, _I32, _F32, _P, _P]),
    "eagle_linear_rows_workspace": (_SZ, [_I32, _I32, _I32]),
    "eagle_linear_rmsnorm": (_I32, [_P, _I32, _I32, _P, _I32, _P, _P, _P, _F32, _P, _P, _SZ, _P]),
    "eagle_linear_norm_parts": (_I32, [_I32, _I32, _I32]),
    "eagle_linear_rmsnorm_deferred": (_I32, [_P, _I32, _I32, _P, _I32, _P, _P, _P, _P, _P, _P, _SZ,
                                             _P]),
    "eagle_linear_rope_qkv": (_I32, [_P, _I32, _I32, _P, _I32, _F32, _P, _I32, _I32, _I32, _P, _I64,
                                     _F32, _P, _I32, _P, _P, _P, _I32, _P, _SZ, _P, _P]),
    "eagle_rope_qkv": (_I32, [_P, _I32, _I32, _I32, _I32, _P, _I64, _F32, _P, _I32, _P, _P, _P,
                              _I32, _P, _P]),
    "eagle_draft_prepare": (_I32, [_P, _I32, _P, _P, _P, _I32, _P, _I32, _I32, _P, _P, _I32, _P, _P,
                                   _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _P]),
    "eagle_embed": (_I32, [_I32, _P, _P, _I32, _I32, _P, _P, _P]),
    "eagle_embed_deferred": (_I32, [_I32, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "eagle_accept_q_workspace": (_SZ, [_I32, _I32]),
    "eagle_accept_q": (_I32, [_I32, _P, _P, _P, _P, _I32, _F32, _P, _I32, _P, _P, _P, _P, _SZ, _P,
                              _P]),
    "eagle_logits_process_workspace": (_SZ, [_I32, _I32, _I32]),
    "eagle_logits_process": (_I32, [_P, _I32, _I32, _F32, _I32, _F32, _P, _P, _P, _SZ, _P]),
    "eagle_fuse3": (_I32, [_P, _P, _P, _I32, _I32, _P, _I32, _P, ctypes.c_int, _P, _SZ, _P]),
    "eagle_gate_children": (_I32, [_P, _I32, _I32, _F32, _I32, _P, _P, _P, _P]),
    "eagle_path_slots": (_I32, [_P, _P, _I32, _P, _I32, _P, _I32, _I32, _P, _P, _P, _P]),
    "eagle_kv_commit_pair": (_I32, [_P, _P, _I32, _I32, _P, _P, _I64, _P, _P, _I32, _I32, _P, _P,
                                    _I64, _I64, _P, _P, _I32, _P, _I32, _P, _I32, _I32, _I32,
                                    _I32, ctypes.c_int, _P, _P]),
    "eagle_kv_commit": (_I32, [_P, _P, _I32, _I32, _I64, _P, _P, _I32, _P, _P, _I64, _I64, _I64, _I32,
                               _I32, _I32, ctypes.c_int, _P, _P]),
}

_lib = None


class EagleError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        msg = lib().eagle_status_string(code).decode() if _lib else str(code)
        super().__init__(f"{fn} returned {code} ({msg})")


def lib() -> ctypes.CDLL:
    """Load libeagle.so once and declare every prototype."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m speculative_decoding_parent_amd.build`")
        so = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            if hasattr(so, name):
                fn = getattr(so, name)
                fn.restype = res
                fn.argtypes = args
        _lib = so
    return _lib


def declared_symbols() -> list:
    """Names of the entry points declared in include/eagle.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*\s]+?)\b(eagle_\w+)\s*\(", text, re.M)))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, rc: int):
    if rc != EAGLE_OK:
        raise EagleError(fn, rc)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return EAGLE_BF16
    if t.dtype == torch.float32:
        return EAGLE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    # zero-filled: the projection entry points keep self-resetting counters,
    # and the LM head its per-row key bounds, at the start of their workspace,
    # which must be zero before first use
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- entry points

def eagle_abi_version() -> int:
    return lib().eagle_abi_version()


def eagle_build_tree_mask(parents: torch.Tensor, words: Optional[int] = None,
                          mask: Optional[torch.Tensor] = None, depth: Optional[torch.Tensor] = None,
                          dev_status: Optional[torch.Tensor] = None):
    """Returns (mask int64[T][words] holding the uint64 bit patterns, depth int32[T])."""
    T = parents.shape[0]
    words = (T + 63) // 64 if words is None else words
    dev = parents.device
    mask = torch.empty((T, words), dtype=torch.int64, device=dev) if mask is None else mask
    depth = torch.empty(T, dtype=torch.int32, device=dev) if depth is None else depth
    _check("eagle_build_tree_mask",
           lib().eagle_build_tree_mask(_ptr(parents), T, words, _ptr(mask), _ptr(depth),
                                       _ptr(dev_status), _stream()))
    return mask, depth


def eagle_tree_attn(q, k_cache, v_cache, L, k_tree, v_tree, Tk, mask, q_mask_row=None,
                    scale=None, out_dtype=None, out=None, workspace=None, dev_status=None):
    """q [Tq][Hq][hd]; caches [Hkv][ld][hd]; mask int64 [rows][words]."""
    Tq, Hq, hd = q.shape
    Hkv = k_tree.shape[0]
    in_dt = _dt(q)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((Tq, Hq, hd), dtype=out_dtype, device=q.device)
    scale = 1.0 / (hd ** 0.5) if scale is None else scale
    ld_cache = k_cache.shape[1] if k_cache is not None else 0
    nb = lib().eagle_tree_attn_workspace(Tq, Hq, Hkv, hd, L, Tk, in_dt)
    ws = _workspace(nb, q.device, workspace)
    _check("eagle_tree_attn", lib().eagle_tree_attn(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), L, ld_cache, _ptr(k_tree), _ptr(v_tree), Tk,
        k_tree.shape[1], _ptr(mask), mask.shape[1], mask.shape[0], _ptr(q_mask_row), Tq, Hq, Hkv,
        hd, scale, in_dt, _dt(out), _ptr(out), _ptr(ws), nb, _ptr(dev_status), _stream()))
    return out


def eagle_logits_process(logits, temperature, top_k=0, top_p=1.0, out=None, kept=None,
                         workspace=None):
    """Temperature / top-k / top-p processing of f32 [T][V] logits; returns
    (processed logits with removed tokens at -inf, kept int32 [T]).  ``out``
    may be ``logits`` itself."""
    T, V = logits.shape
    out = torch.empty_like(logits) if out is None else out
    kept = torch.empty(T, dtype=torch.int32, device=logits.device) if kept is None else kept
    nb = lib().eagle_logits_process_workspace(T, V, int(top_k))
    ws = _workspace(nb, logits.device, workspace) if nb else None
    _check("eagle_logits_process", lib().eagle_logits_process(
        _ptr(logits), T, V, float(temperature), int(top_k), float(top_p), _ptr(out), _ptr(kept),
        _ptr(ws), nb, _stream()))
    return out, kept


def eagle_fuse3(h_low, h_mid, h_high, W, out=None, out_dtype=torch.float32, workspace=None):
    """Eagle-3 fusion: [h_low ; h_mid ; h_high] (each [M][d] bf16) times W^T
    (W [N][3 d] bf16), without forming the concatenation."""
    M, d = h_low.shape
    N = W.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=h_low.device)
    nb = lib().eagle_linear_workspace(M, 3 * d, N, 0)
    ws = _workspace(nb, h_low.device, workspace)
    _check("eagle_fuse3", lib().eagle_fuse3(_ptr(h_low), _ptr(h_mid), _ptr(h_high), M, d, _ptr(W),
                                            N, _ptr(out), _dt(out), _ptr(ws), nb, _stream()))
    return out


def eagle_gate_children(logp, tau=2.0, max_branch=4, out=None, kept=None, confidence=None):
    """Confidence gate over sorted top-k log-probs f32 [rows][k]; returns
    (gated log-probs, kept int32 [rows], confidence f32 [rows]).  ``out`` may
    be ``logp`` itself (in place)."""
    rows, k = logp.shape
    dev = logp.device
    out = torch.empty_like(logp) if out is None else out
    kept = torch.empty(rows, dtype=torch.int32, device=dev) if kept is None else kept
    confidence = torch.empty(rows, dtype=torch.float32, device=dev) if confidence is None else confidence
    _check("eagle_gate_children", lib().eagle_gate_children(
        _ptr(logp), rows, k, float(tau), max_branch, _ptr(out), _ptr(kept), _ptr(confidence),
        _stream()))
    return out, kept, confidence


def eagle_kv_commit(k_src, v_src, rows, k_cache, v_cache, L, n_accepted=None, src_rows=None,
                    max_rows=None, dev_status=None):
    """Append source rows ``rows[0 .. n)`` to the caches at positions L, L + 1, ...

    Sources and caches are [Hkv][ld][hd] or [layers][Hkv][ld][hd] views whose
    last two dimensions are contiguous (a source may be a view into the cache
    itself).  n = n_accepted[0] + 1 (device int32) or max_rows (default
    ``rows.shape[0]``)."""
    if k_src.dim() == 3:
        k_src, v_src, k_cache, v_cache = (t.unsqueeze(0) for t in (k_src, v_src, k_cache, v_cache))
    layers, Hkv, nsrc, hd = k_src.shape
    for t in (k_src, v_src, k_cache, v_cache):
        if t.stride(3) != 1 or t.stride(2) != hd or t.stride(1) % hd or t.stride(1) < t.shape[2] * hd:
            raise ValueError("sources and caches need [Hkv][ld][hd] blocks with contiguous rows")
    if v_src.stride(0) != k_src.stride(0) or v_src.stride(1) != k_src.stride(1) or \
            v_cache.stride(0) != k_cache.stride(0) or v_cache.stride(1) != k_cache.stride(1):
        raise ValueError("K and V need the same strides")
    ld_src = k_src.stride(1) // hd          # rows per head block (the cache's, for a view into it)
    ld_cache = k_cache.stride(1) // hd
    max_rows = rows.shape[0] if max_rows is None else max_rows
    src_rows = nsrc if src_rows is None else src_rows
    _check("eagle_kv_commit", lib().eagle_kv_commit(
        _ptr(k_src), _ptr(v_src), ld_src, src_rows, k_src.stride(0), _ptr(rows), _ptr(n_accepted),
        max_rows, _ptr(k_cache), _ptr(v_cache), L, ld_cache, k_cache.stride(0), layers, Hkv, hd,
        _dt(k_src), _ptr(dev_status), _stream()))


def eagle_path_slots(path, n_accepted, node_pool_idx, slot_of_pool, n_slots, slot_rows=None,
                     n_rows_minus_one=None, dev_status=None):
    """The draft slots of the accepted path's leading expanded nodes; returns
    (slot_rows int32[max_path], n_rows_minus_one int32[1])."""
    max_path = path.shape[0]
    dev = path.device
    slot_rows = torch.empty(max_path, dtype=torch.int32, device=dev) if slot_rows is None else slot_rows
    n_rows_minus_one = (torch.empty(1, dtype=torch.int32, device=dev) if n_rows_minus_one is None
                        else n_rows_minus_one)
    _check("eagle_path_slots", lib().eagle_path_slots(
        _ptr(path), _ptr(n_accepted), max_path, _ptr(node_pool_idx), node_pool_idx.shape[0],
        _ptr(slot_of_pool), slot_of_pool.shape[0], n_slots, _ptr(slot_rows), _ptr(n_rows_minus_one),
        _ptr(dev_status), _stream()))
    return slot_rows, n_rows_minus_one


def eagle_kv_commit_pair(t_k, t_v, t_kc, t_vc, d_k, d_v, d_kc, d_vc, L, path, n_accepted,
                         node_pool_idx, slot_of_pool, max_path, dev_status=None):
    """eagle_kv_commit of the target's rows path[0 .. n) and of the draft's
    rows of the same nodes (eagle_path_slots' rule over path[:max_path]) in
    one launch; every tensor is [Hkv][rows][hd] with contiguous rows."""
    Hkv, _, hd = t_k.shape
    for t in (t_k, t_v, t_kc, t_vc, d_k, d_v, d_kc, d_vc):
        if t.dim() != 3 or t.shape[0] != Hkv or t.shape[2] != hd or not t.is_contiguous():
            raise ValueError("sources and caches need contiguous [Hkv][rows][hd] tensors")
    _check("eagle_kv_commit_pair", lib().eagle_kv_commit_pair(
        _ptr(t_k), _ptr(t_v), t_k.shape[1], t_k.shape[1], _ptr(t_kc), _ptr(t_vc), t_kc.shape[1],
        _ptr(d_k), _ptr(d_v), d_k.shape[1], d_k.shape[1], _ptr(d_kc), _ptr(d_vc), d_kc.shape[1],
        L, _ptr(path), _ptr(n_accepted), path.shape[0], _ptr(node_pool_idx), node_pool_idx.shape[0],
        _ptr(slot_of_pool), slot_of_pool.shape[0], max_path, Hkv, hd, _dt(t_k), _ptr(dev_status),
        _stream()))


def _norm_args(in_norm):
    """(in_ssq, in_parts, in_eps) of an optional deferred RMSNorm given as
    (ssq f32 [P][M], eps), e.g. the last two results of
    eagle_linear_rmsnorm_deferred and the norm's eps."""
    if in_norm is None:
        return None, 0, 0.0
    ssq, eps = in_norm
    return _ptr(ssq), ssq.shape[0], float(eps)


def eagle_lmhead_topk(f, W, k, want_logits=False, topk_id=None, topk_logp=None, lse=None,
                      logits=None, workspace=None, in_norm=None):
    """Returns (topk_id int32[T][k], topk_logp f32[T][k], lse f32[T], logits or None);
    k = 0 computes lse (and logits) only and returns None for the top-k."""
    T, d = f.shape
    V = W.shape[0]
    dt = _dt(f)
    dev = f.device
    if k > 0:
        topk_id = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_id is None else topk_id
        topk_logp = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_logp is None else topk_logp
    lse = torch.empty(T, dtype=torch.float32, device=dev) if lse is None else lse
    if want_logits and logits is None:
        logits = torch.empty((T, V), dtype=torch.float32, device=dev)
    nb = lib().eagle_lmhead_topk_workspace(T, d, V, k, dt)
    ws = _workspace(nb, dev, workspace)
    _check("eagle_lmhead_topk", lib().eagle_lmhead_topk(
        _ptr(f), _ptr(W), T, d, V, k, dt, *_norm_args(in_norm), _ptr(topk_id), _ptr(topk_logp),
        _ptr(lse), _ptr(logits), _ptr(ws), nb, _stream()))
    return topk_id, topk_logp, lse, logits


def eagle_lmhead_topk_noalloc(f, W, k, topk_id, topk_logp, lse, logits=None, in_norm=None):
    """eagle_lmhead_topk with the library's own scratch: every output is passed
    in by the caller and nothing is allocated on the way to the kernels."""
    T, d = f.shape
    V = W.shape[0]
    _check("eagle_lmhead_topk_noalloc", lib().eagle_lmhead_topk_noalloc(
        _ptr(f), _ptr(W), T, d, V, k, _dt(f), *_norm_args(in_norm), _ptr(topk_id), _ptr(topk_logp),
        _ptr(lse), _ptr(logits), _stream()))
    return topk_id, topk_logp, lse, logits


def eagle_expand_rerank(mode, pool_token, pool_parent, pool_depth, pool_value, pool_n,
                        frontier=None, child_id=None, child_logp=None, k_select=0,
                        new_frontier=None, T=0, node_token=None, node_parent=None,
                        node_depth=None, node_pool_idx=None, dev_status=None):
    """EXPAND returns new_frontier; RERANK returns (token, parent, depth, pool_idx)."""
    cap = pool_token.shape[0]
    dev = pool_token.device
    if mode == EAGLE_EXPAND:
        kf, k = child_id.shape
        if new_frontier is None:
            new_frontier = torch.empty(k_select, dtype=torch.int32, device=dev)
        _check("eagle_expand_rerank", lib().eagle_expand_rerank(
            mode, _ptr(pool_token), _ptr(pool_parent), _ptr(pool_depth), _ptr(pool_value), pool_n,
            cap, _ptr(frontier), kf, _ptr(child_id), _ptr(child_logp), k, k_select,
            _ptr(new_frontier), 0, None, None, None, None, _ptr(dev_status), _stream()))
        return new_frontier
    mk = lambda t: torch.empty(T, dtype=torch.int32, device=dev) if t is None else t
    node_token, node_parent, node_depth, node_pool_idx = (mk(node_token), mk(node_parent),
                                                          mk(node_depth), mk(node_pool_idx))
    _check("eagle_expand_rerank", lib().eagle_expand_rerank(
        mode, _ptr(pool_token), _ptr(pool_parent), _ptr(pool_depth), _ptr(pool_value), pool_n, cap,
        None, 0, None, None, 0, 0, None, T, _ptr(node_token), _ptr(node_parent), _ptr(node_depth),
        _ptr(node_pool_idx), _ptr(dev_status), _stream()))
    return node_token, node_parent, node_depth, node_pool_idx


def eagle_accept(mode, node_token, node_parent, target_top1=None, target_logits=None,
                 temperature=1.0, uniforms=None, max_path=None, path=None, n_accepted=None,
                 bonus_token=None, workspace=None, dev_status=None):
    """Returns (path int32[max_path], n_accepted int32[1], bonus int32[1])."""
    T = node_token.shape[0]
    dev = node_token.device
    max_path = T if max_path is None else max_path
    path = torch.empty(max_path, dtype=torch.int32, device=dev) if path is None else path
    n_accepted = torch.empty(1, dtype=torch.int32, device=dev) if n_accepted is None else n_accepted
    bonus_token = torch.empty(1, dtype=torch.int32, device=dev) if bonus_token is None else bonus_token
    V = target_logits.shape[1] if target_logits is not None else 0
    nb = lib().eagle_accept_workspace(T, V) if mode == EAGLE_SAMPLE else 0
    ws = _workspace(nb, dev, workspace) if mode == EAGLE_SAMPLE else None
    # target_top1 may be a strided view, e.g. column 0 of the LM head's topk_id [T][k]
    top1_stride = target_top1.stride(0) if target_top1 is not None else 1
    _check("eagle_accept", lib().eagle_accept(
        mode, T, _ptr(node_token), _ptr(node_parent), _ptr(target_top1), top1_stride,
        _ptr(target_logits), V,
        temperature, _ptr(uniforms), max_path, _ptr(path), _ptr(n_accepted), _ptr(bonus_token),
        _ptr(ws), nb, _ptr(dev_status), _stream()))
    return path, n_accepted, bonus_token


def eagle_accept_q(node_token, node_parent, target_logits, draft_logits, temperature, uniforms,
                   max_path=None, path=None, n_accepted=None, bonus_token=None, workspace=None,
                   dev_status=None):
    """Speculative sampling with the draft's distribution; returns
    (path int32[max_path], n_accepted int32[1], bonus int32[1])."""
    T = node_token.shape[0]
    dev = node_token.device
    V = target_logits.shape[1]
    max_path = T if max_path is None else max_path
    path = torch.empty(max_path, dtype=torch.int32, device=dev) if path is None else path
    n_accepted = torch.empty(1, dtype=torch.int32, device=dev) if n_accepted is None else n_accepted
    bonus_token = torch.empty(1, dtype=torch.int32, device=dev) if bonus_token is None else bonus_token
    nb = lib().eagle_accept_q_workspace(T, V)
    ws = _workspace(nb, dev, workspace)
    _check("eagle_accept_q", lib().eagle_accept_q(
        T, _ptr(node_token), _ptr(node_parent), _ptr(target_logits), _ptr(draft_logits), V,
        temperature, _ptr(uniforms), max_path, _ptr(path), _ptr(n_accepted), _ptr(bonus_token),
        _ptr(ws), nb, _ptr(dev_status), _stream()))
    return path, n_accepted, bonus_token


# ---------------------------------------------------------------- layer support

def eagle_linear(x, W, residual=None, out=None, out_dtype=torch.float32, workspace=None):
    """out = x W^T (+ residual); x [M][K] bf16, W [N][K] bf16."""
    M, K = x.shape
    N = W.shape[0]
    out = torch.empty((M, N), dtype=out_dtype, device=x.device) if out is None else out
    nb = lib().eagle_linear_workspace(M, K, N, 0)
    ws = _workspace(nb, x.device, workspace) if nb else None
    _check("eagle_linear", lib().eagle_linear(_ptr(x), M, K, _ptr(W), N, _ptr(residual), _ptr(out),
                                              _dt(out), _ptr(ws), nb, _stream()))
    return out


def eagle_linear_swiglu(x, w_gate, w_up, out=None, workspace=None, in_norm=None):
    M, K = x.shape
    N = w_gate.shape[0]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if out is None else out
    nb = lib().eagle_linear_workspace(M, K, N, 1)
    ws = _workspace(nb, x.device, workspace) if nb else None
    _check("eagle_linear_swiglu", lib().eagle_linear_swiglu(
        _ptr(x), M, K, *_norm_args(in_norm), _ptr(w_gate), _ptr(w_up), N, _ptr(out), _ptr(ws), nb,
        _stream()))
    return out


def eagle_linear_rmsnorm(x, W, gamma, residual=None, out=None, norm_out=None, eps=1e-5,
                         workspace=None):
    """out = x W^T (+ residual) in f32; norm_out = RMSNorm(out) * gamma in bf16."""
    M, K = x.shape
    N = W.shape[0]
    out = torch.empty((M, N), dtype=torch.float32, device=x.device) if out is None else out
    norm_out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if norm_out is None else norm_out
    nb = lib().eagle_linear_rows_workspace(M, K, N)
    ws = _workspace(nb, x.device, workspace)
    _check("eagle_linear_rmsnorm", lib().eagle_linear_rmsnorm(
        _ptr(x), M, K, _ptr(W), N, _ptr(residual), _ptr(out), _ptr(gamma), eps, _ptr(norm_out),
        _ptr(ws), nb, _stream()))
    return out, norm_out


def eagle_linear_rmsnorm_deferred(x, W, gamma, residual=None, out=None, xg_out=None, ssq_out=None,
                                  workspace=None):
    """out = x W^T (+ residual) in f32; xg = out * gamma in bf16; ssq [P][M] f32
    partial row sums of out^2 (a deferred RMSNorm for the next product)."""
    M, K = x.shape
    N = W.shape[0]
    P = lib().eagle_linear_norm_parts(M, K, N)
    out = torch.empty((M, N), dtype=torch.float32, device=x.device) if out is None else out
    xg_out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if xg_out is None else xg_out
    ssq_out = torch.empty((P, M), dtype=torch.float32, device=x.device) if ssq_out is None else ssq_out
    assert ssq_out.is_contiguous() and ssq_out.shape == (P, M), (ssq_out.shape, P, M)
    nb = lib().eagle_linear_rows_workspace(M, K, N)
    ws = _workspace(nb, x.device, workspace)
    _check("eagle_linear_rmsnorm_deferred", lib().eagle_linear_rmsnorm_deferred(
        _ptr(x), M, K, _ptr(W), N, _ptr(residual), _ptr(out), _ptr(gamma), _ptr(xg_out),
        _ptr(ssq_out), _ptr(ws), nb, _stream()))
    return out, xg_out, ssq_out


def eagle_linear_rope_qkv(x, w_qkv, Hq, Hkv, hd, depth, pos_base, k_tree, v_tree, row_slot=None,
                          theta=500000.0, q_out=None, workspace=None, dev_status=None,
                          in_norm=None):
    M, K = x.shape
    N = (Hq + 2 * Hkv) * hd
    q_out = torch.empty((M, Hq, hd), dtype=torch.bfloat16, device=x.device) if q_out is None else q_out
    nb = lib().eagle_linear_rows_workspace(M, K, N)
    ws = _workspace(nb, x.device, workspace)
    ld = k_tree.shape[1]
    _check("eagle_linear_rope_qkv", lib().eagle_linear_rope_qkv(
        _ptr(x), M, K, *_norm_args(in_norm), _ptr(w_qkv), Hq, Hkv, hd, _ptr(depth), pos_base, theta, _ptr(row_slot), ld,
        _ptr(q_out), _ptr(k_tree), _ptr(v_tree), ld, _ptr(ws), nb, _ptr(dev_status), _stream()))
    return q_out


def eagle_rmsnorm(x, gamma, eps=1e-5, out=None):
    M, N = x.shape
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _check("eagle_rmsnorm", lib().eagle_rmsnorm(_ptr(x), _ptr(gamma), M, N, eps, _ptr(out),
                                                _stream()))
    return out


def eagle_rope_qkv(qkv, Hq, Hkv, hd, depth, pos_base, k_tree, v_tree, row_slot=None,
                   theta=500000.0, q_out=None, dev_status=None):
    M = qkv.shape[0]
    q_out = torch.empty((M, Hq, hd), dtype=torch.bfloat16, device=qkv.device) if q_out is None else q_out
    ld = k_tree.shape[1]
    _check("eagle_rope_qkv", lib().eagle_rope_qkv(
        _ptr(qkv), M, Hq, Hkv, hd, _ptr(depth), pos_base, theta, _ptr(row_slot), ld, _ptr(q_out),
        _ptr(k_tree), _ptr(v_tree), ld, _ptr(dev_status), _stream()))
    return q_out


def eagle_draft_prepare(frontier, pool_token, pool_parent, pool_depth, pool_n, slot_of_pool,
                        slot_base, slot_parent, rows, slot_mask=None, feat=None, root_feat=None,
                        embed=None, x_in=None, dev_status=None):
    """rows: (row_token, row_depth, row_slot, row_src) int32 tensors of >= kf entries."""
    kf = frontier.shape[0]
    words = slot_mask.shape[1] if slot_mask is not None else 0
    V, d = embed.shape if embed is not None else (1, 0)
    _check("eagle_draft_prepare", lib().eagle_draft_prepare(
        _ptr(frontier), kf, _ptr(pool_token), _ptr(pool_parent), _ptr(pool_depth), pool_n,
        _ptr(slot_of_pool), slot_base, slot_parent.shape[0], _ptr(slot_parent), _ptr(slot_mask),
        words, *[_ptr(r) for r in rows], _ptr(feat), _ptr(root_feat), _ptr(embed), V, d, _ptr(x_in),
        _ptr(dev_status), _stream()))


def eagle_embed(token, embed, out=None, dev_status=None):
    M = token.shape[0]
    V, d = embed.shape
    out = torch.empty((M, d), dtype=torch.float32, device=embed.device) if out is None else out
    _check("eagle_embed", lib().eagle_embed(M, _ptr(token), _ptr(embed), V, d, _ptr(out),
                                            _ptr(dev_status), _stream()))
    return out


def eagle_embed_deferred(token, embed, gamma, out=None, xg_out=None, ssq_out=None,
                         dev_status=None):
    """out = f32 embed rows, xg = bf16(out * gamma), ssq [1][M] = row sums of
    out^2 (the RMSNorm that follows, deferred)."""
    M = token.shape[0]
    V, d = embed.shape
    dev = embed.device
    out = torch.empty((M, d), dtype=torch.float32, device=dev) if out is None else out
    xg_out = torch.empty((M, d), dtype=torch.bfloat16, device=dev) if xg_out is None else xg_out
    ssq_out = torch.empty((1, M), dtype=torch.float32, device=dev) if ssq_out is None else ssq_out
    _check("eagle_embed_deferred", lib().eagle_embed_deferred(
        M, _ptr(token), _ptr(embed), V, d, _ptr(gamma), _ptr(out), _ptr(xg_out), _ptr(ssq_out),
        _ptr(dev_status), _stream()))
    return out, xg_out, ssq_out
