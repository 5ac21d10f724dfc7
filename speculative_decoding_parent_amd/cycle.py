"""One EAGLE-2 draft-and-verify cycle on the GPU, driven through the C ABI.

The draft grows a dynamic tree for ``rounds`` rounds: each round fuses every
frontier row's parent feature with its token embedding, runs one decoder layer
(attention over the draft's KV prefix and the K/V of every node expanded so
far, under the slot tree's ancestor mask), scores the rows with the shared LM
head and appends the top-k children by cumulative log-probability.  The tree is
then pruned to T nodes, verified by one target layer under the tree mask, a
path is accepted by speculative sampling, and the accepted path's K/V rows are
committed to both caches ("EAGLE-2: Feature-Level Speculative
Decoding Guide", Key Architectural Mechanics 1-3; "Support Eagle-3 Speculative
Decoding in llama.cpp", the dynamic-tree and KV-cache replies).

Every buffer is allocated once here (torch provides the device memory) and the
whole cycle is a fixed sequence of launches on one stream whose sizes follow
from (rounds, k, k_select, T) alone: the host never reads device data inside a
cycle, so the sequence can be captured into a HIP graph and replayed.
"""
from __future__ import annotations

import torch

from . import _lib
from .inputs import Workload


class DraftVerifyCycle:
    def __init__(self, w: Workload, ci: dict, device, temperature: float = 1.0):
        self.w = w
        dev = self.dev = torch.device(device)
        d, hq, hkv, hd, F, V, L = w.d, w.hq, w.hkv, w.hd, w.ffn, w.vocab, w.L
        R, k, ks, T = w.rounds, w.topk, w.k_select, w.T
        self.R, self.k, self.ks, self.T, self.L = R, k, ks, T, L
        self.temperature = temperature
        to = lambda t: t.to(dev).contiguous()
        self.w_fuse = to(ci["w_fuse"])
        self.draft = {n: to(t) for n, t in ci["draft"].items()}
        self.target = {n: to(t) for n, t in ci["target"].items()}
        self.draft_norm = to(ci["draft_norm"])
        self.target_norm = to(ci["target_norm"])
        self.embed = to(ci["embed"])
        self.w_lm = to(ci["w_lm"])
        # KV caches with room for one cycle's commit: positions 0..L-1 hold the
        # prefix, and the accepted path's rows are written at L, L+1, ...
        def cache(t):
            c = torch.zeros((t.shape[0], L + T, t.shape[2]), dtype=t.dtype, device=dev)
            c[:, :L] = t[:, :L].to(dev)
            return c
        self.dkc, self.dvc = cache(ci["draft_k_cache"]), cache(ci["draft_v_cache"])
        self.tkc, self.tvc = cache(ci["target_k_cache"]), cache(ci["target_v_cache"])
        self.root_feat = to(ci["root_feature"]).float()
        self.uniforms = torch.as_tensor(ci["uniforms"]).to(dev)

        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        bf = dict(dtype=torch.bfloat16, device=dev)
        nqkv = (hq + 2 * hkv) * hd
        # candidate pool (entry 0 = root, never overwritten) and per-round frontiers
        self.pool_n = [1] + [1 + k + r * ks * k for r in range(R)]
        cap = self.pool_n[R]
        self.pool_token = torch.zeros(cap, **i32)
        self.pool_parent = torch.full((cap,), -1, **i32)
        self.pool_depth = torch.zeros(cap, **i32)
        self.pool_value = torch.zeros(cap, **f32)
        self.pool_token[0] = int(ci["root_token"])
        self.frontier = [torch.zeros(1 if r == 0 else ks, **i32) for r in range(R + 1)]
        # draft slots: one per expanded row (K/V, output feature, mask row)
        self.S = 1 + (R - 1) * ks
        self.slot_base = [0] + [1 + r * ks for r in range(R - 1)]
        self.slot_of_pool = torch.full((cap,), -1, **i32)
        self.slot_parent = torch.full((self.S,), -1, **i32)
        self.smask = torch.zeros((self.S, (self.S + 63) // 64), dtype=torch.int64, device=dev)
        self.sdepth = torch.zeros(self.S, **i32)
        self.rows = [torch.zeros(ks, **i32) for _ in range(4)]      # token, depth, slot, src
        self.feat = torch.zeros((self.S, d), **f32)
        self.dkt = torch.zeros((hkv, self.S, hd), **bf)
        self.dvt = torch.zeros((hkv, self.S, hd), **bf)
        m = max(ks, T)
        self.x_in = torch.zeros((ks, 2 * d), **bf)
        self.h = torch.zeros((m, d), **f32)
        self.n1 = torch.zeros((m, d), **bf)
        self.qkv = torch.zeros((m, nqkv), **f32)
        self.q = torch.zeros((m, hq, hd), **bf)
        self.attn = torch.zeros((m, hq, hd), **bf)
        self.x2 = torch.zeros((m, d), **f32)
        self.n2 = torch.zeros((m, d), **bf)
        self.gu = torch.zeros((m, F), **bf)
        self.z = torch.zeros((m, d), **bf)
        # partial row sums of squares of the deferred norms (norm1, norm2, final)
        P = max(_lib.lib().eagle_linear_norm_parts(mm, d, d) * mm for mm in (1, ks, T))
        self.s1, self.s2, self.sz = (torch.zeros(P, **f32) for _ in range(3))
        self.ids = [torch.zeros((1 if r == 0 else ks, k), **i32) for r in range(R)]
        self.logp = [torch.zeros((1 if r == 0 else ks, k), **f32) for r in range(R)]
        self.lse = torch.zeros(m, **f32)
        # verify pass
        self.node_token = torch.zeros(T, **i32)
        self.node_parent = torch.zeros(T, **i32)
        self.node_depth = torch.zeros(T, **i32)
        self.node_pool_idx = torch.zeros(T, **i32)
        self.vmask = torch.zeros((T, (T + 63) // 64), dtype=torch.int64, device=dev)
        self.vdepth = torch.zeros(T, **i32)
        self.vx = torch.zeros((T, d), **f32)
        self.vssq = torch.zeros((1, T), **f32)     # the embedded rows' sums of squares
        self.vout = torch.zeros((T, d), **f32)
        self.tkt = torch.zeros((hkv, T, hd), **bf)
        self.tvt = torch.zeros((hkv, T, hd), **bf)
        self.v_logits = torch.zeros((T, V), **f32)
        self.path = torch.zeros(T, **i32)
        self.n_accepted = torch.zeros(1, **i32)
        self.bonus = torch.zeros(1, **i32)
        self.status = torch.zeros(1, **i32)
        self.draft_rows = torch.zeros(R + 1, **i32)      # the draft's slots of the accepted path
        self.draft_n = torch.zeros(1, **i32)
        lib = _lib.lib()
        ws_attn = max(lib.eagle_tree_attn_workspace(ks, hq, hkv, hd, L, self.S, _lib.EAGLE_BF16),
                      lib.eagle_tree_attn_workspace(T, hq, hkv, hd, L, T, _lib.EAGLE_BF16))
        ws_lm = max(lib.eagle_lmhead_topk_workspace(ks, d, V, k, _lib.EAGLE_BF16),
                    lib.eagle_lmhead_topk_workspace(T, d, V, k, _lib.EAGLE_BF16))
        self.ws_attn = torch.empty(ws_attn, dtype=torch.uint8, device=dev)
        self.ws_lm = torch.zeros(ws_lm, dtype=torch.uint8, device=dev)     # row bounds start at 0
        self.ws_acc = torch.empty(lib.eagle_accept_workspace(T, V), dtype=torch.uint8, device=dev)
        ws_lin = 256
        for M in (1, ks, T):
            for (K, N) in ((2 * d, d), (d, nqkv), (hq * hd, d), (F, d)):
                ws_lin = max(ws_lin, lib.eagle_linear_rows_workspace(M, K, N))
            ws_lin = max(ws_lin, lib.eagle_linear_workspace(M, d, F, 1))
        self.ws_lin = torch.zeros(ws_lin, dtype=torch.uint8, device=dev)   # counters start at 0
        self.graph = None

    # ------------------------------------------------------------ one layer
    def _ssq(self, buf, n):
        """[P][n] view of a partial-sums buffer for n rows of width d."""
        P = _lib.lib().eagle_linear_norm_parts(n, self.w.d, self.w.d)
        return buf[:P * n].view(P, n)

    def _layer(self, lw, n, x_in, in1, x_res, depth, row_slot, kc, vc, kt, vt, Tk, mask, out,
               q_mask_row, final_norm):
        """Decoder layer on rows 0..n-1.  x_in (bf16) is the attention input:
        RMSNorm(x_res) itself (in1 None) or x_res * gamma with its deferred row
        scale in1 = (ssq, eps); x_res is the fp32 residual stream.  Writes the
        fp32 output to ``out`` and its final norm, deferred, to self.z[:n];
        returns that norm's partial sums."""
        w = self.w
        eps = w.rms_eps
        _lib.eagle_linear_rope_qkv(x_in, lw["wqkv"], w.hq, w.hkv, w.hd, depth, self.L, kt, vt,
                                   row_slot=row_slot, theta=w.rope_theta, q_out=self.q[:n],
                                   workspace=self.ws_lin, dev_status=self.status, in_norm=in1)
        _lib.eagle_tree_attn(self.q[:n], kc, vc, self.L, kt, vt, Tk, mask, q_mask_row=q_mask_row,
                             out=self.attn[:n], workspace=self.ws_attn, dev_status=self.status)
        s2 = self._ssq(self.s2, n)
        _lib.eagle_linear_rmsnorm_deferred(self.attn[:n].view(n, -1), lw["wo"], lw["norm2"],
                                           residual=x_res, out=self.x2[:n], xg_out=self.n2[:n],
                                           ssq_out=s2, workspace=self.ws_lin)
        _lib.eagle_linear_swiglu(self.n2[:n], lw["wgate"], lw["wup"], out=self.gu[:n],
                                 workspace=self.ws_lin, in_norm=(s2, eps))
        sz = self._ssq(self.sz, n)
        _lib.eagle_linear_rmsnorm_deferred(self.gu[:n], lw["wdown"], final_norm,
                                           residual=self.x2[:n], out=out, xg_out=self.z[:n],
                                           ssq_out=sz, workspace=self.ws_lin)
        return sz

    # ------------------------------------------------------------ the cycle
    def draft_round(self, r: int):
        w = self.w
        kf = 1 if r == 0 else self.ks
        base = self.slot_base[r]
        Sr = base + kf
        fr = self.frontier[r]
        tok, depth, slot, src = (t[:kf] for t in self.rows)
        _lib.eagle_draft_prepare(fr, self.pool_token, self.pool_parent, self.pool_depth,
                                 self.pool_n[r], self.slot_of_pool, base, self.slot_parent,
                                 (tok, depth, slot, src), slot_mask=self.smask, feat=self.feat,
                                 root_feat=self.root_feat, embed=self.embed, x_in=self.x_in[:kf],
                                 dev_status=self.status)
        s1 = self._ssq(self.s1, kf)
        _lib.eagle_linear_rmsnorm_deferred(self.x_in[:kf], self.w_fuse, self.draft["norm1"],
                                           out=self.h[:kf], xg_out=self.n1[:kf], ssq_out=s1,
                                           workspace=self.ws_lin)
        feat_rows = self.feat[base:base + kf]
        sz = self._layer(self.draft, kf, self.n1[:kf], (s1, w.rms_eps), self.h[:kf], depth, slot,
                         self.dkc, self.dvc, self.dkt, self.dvt, Sr, self.smask[:Sr], feat_rows,
                         slot, self.draft_norm)
        _lib.eagle_lmhead_topk(self.z[:kf], self.w_lm, self.k, topk_id=self.ids[r],
                               topk_logp=self.logp[r], lse=self.lse[:kf], workspace=self.ws_lm,
                               in_norm=(sz, w.rms_eps))
        _lib.eagle_expand_rerank(_lib.EAGLE_EXPAND, self.pool_token, self.pool_parent,
                                 self.pool_depth, self.pool_value, self.pool_n[r], frontier=fr,
                                 child_id=self.ids[r], child_logp=self.logp[r], k_select=self.ks,
                                 new_frontier=self.frontier[r + 1], dev_status=self.status)

    def verify(self):
        w, T = self.w, self.T
        _lib.eagle_expand_rerank(_lib.EAGLE_RERANK, self.pool_token, self.pool_parent,
                                 self.pool_depth, self.pool_value, self.pool_n[self.R], T=T,
                                 node_token=self.node_token, node_parent=self.node_parent,
                                 node_depth=self.node_depth, node_pool_idx=self.node_pool_idx,
                                 dev_status=self.status)
        _lib.eagle_build_tree_mask(self.node_parent, mask=self.vmask, depth=self.vdepth,
                                   dev_status=self.status)
        _lib.eagle_embed_deferred(self.node_token, self.embed, self.target["norm1"], out=self.vx,
                                  xg_out=self.n1[:T], ssq_out=self.vssq, dev_status=self.status)
        sz = self._layer(self.target, T, self.n1[:T], (self.vssq, w.rms_eps), self.vx,
                         self.node_depth, None,
                         self.tkc, self.tvc, self.tkt, self.tvt, T, self.vmask, self.vout, None,
                         self.target_norm)
        # sampling acceptance reads the logits; no top-k is needed (k = 0)
        _lib.eagle_lmhead_topk(self.z[:T], self.w_lm, 0, lse=self.lse[:T], logits=self.v_logits,
                               workspace=self.ws_lm, in_norm=(sz, w.rms_eps))
        _lib.eagle_accept(_lib.EAGLE_SAMPLE, self.node_token, self.node_parent,
                          target_logits=self.v_logits, temperature=self.temperature,
                          uniforms=self.uniforms, path=self.path, n_accepted=self.n_accepted,
                          bonus_token=self.bonus, workspace=self.ws_acc, dev_status=self.status)
        self.commit()

    def commit(self):
        """KV commit after acceptance: the target keeps K/V only for the
        accepted path (root first) and the draft keeps its rows of the same
        nodes, both appended at cache position L; every other candidate's rows
        are dropped ("Support Eagle-3 Speculative Decoding in llama.cpp", the
        reply on the draft's context).  Counts are read on the device."""
        _lib.eagle_kv_commit_pair(self.tkt, self.tvt, self.tkc, self.tvc, self.dkt, self.dvt,
                                  self.dkc, self.dvc, self.L, self.path,
                                  self.n_accepted, self.node_pool_idx, self.slot_of_pool,
                                  self.R + 1, dev_status=self.status)

    def enqueue(self):
        """Enqueue one whole cycle on the current stream."""
        for r in range(self.R):
            self.draft_round(r)
        self.verify()

    def capture(self):
        """Capture one cycle into a HIP graph (buffers stay fixed)."""
        s = torch.cuda.Stream(device=self.dev)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.enqueue()          # warm-up outside the graph
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.enqueue()
        torch.cuda.synchronize()

    def run(self):
        if self.graph is not None:
            self.graph.replay()
        else:
            self.enqueue()
