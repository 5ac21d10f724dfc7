"""Throughput of one EAGLE-2 draft-and-verify cycle on one MI355X.

A step is the whole hot path over one synthetic Llama-3-8B-shaped cycle:
6 draft rounds (fuse 8192->4096, one decoder layer with 32/8 heads of 128
over a 4096-token prefix plus the draft tree, SwiGLU 14336, LM head over a
128256-token vocabulary with top-10, expansion by cumulative log-probability),
rerank to 64 nodes, tree mask, one target layer verifying the 64 nodes,
LM head with logits, and speculative-sampling acceptance.  The cycle is
replayed from a HIP graph with every input already resident in HBM.

Prints one JSON line: nodes verified per second, the roofline of the dominant
kernel (the LM head at the draft-round shape, timed with HIP events on its
launch stream) and the CPU oracle's throughput on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

CORES = len(os.sched_getaffinity(0))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(CORES))

import numpy as np  # noqa: E402
import torch  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from speculative_decoding_parent_amd import _lib, inputs  # noqa: E402
from speculative_decoding_parent_amd.cycle import DraftVerifyCycle  # noqa: E402

METRIC = "tree-verify nodes/s + KV/LM-head HBM GB/s (% roofline), Llama-3-8B shape"
HBM_PEAK_GBS = 8000.0


CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "speculative_decoding_parent_amd",
                    "csrc")


def measured_traffic(key, sources):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/
    hbm_traffic.json), or None when the kernel sources have changed since."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))[key]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return int(round(rec["fetch_bytes"] + rec["write_bytes"]))


def lmhead_bytes(T, d, V, k):
    """Algorithmic bytes of one LM-head call: W once, the features once, the
    top-k ids/log-probs and lse out."""
    return V * d * 2 + T * d * 2 + T * (8 * k + 4)


def time_lmhead(cyc, T, iters):
    """Average duration (s) of eagle_lmhead_topk at T rows, HIP events on the
    stream the kernels are launched on."""
    z = cyc.z[:T]
    in_norm = (cyc._ssq(cyc.sz, T), cyc.w.rms_eps)      # the draft rounds' deferred final norm
    ids = torch.empty((T, cyc.k), dtype=torch.int32, device=cyc.dev)
    lp = torch.empty((T, cyc.k), dtype=torch.float32, device=cyc.dev)
    lse = torch.empty(T, dtype=torch.float32, device=cyc.dev)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for a, b in evs:
        a.record(stream)
        _lib.eagle_lmhead_topk(z, cyc.w_lm, cyc.k, topk_id=ids, topk_logp=lp, lse=lse,
                               workspace=cyc.ws_lm, in_norm=in_norm)
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return float(np.mean(ms)) / 1e3, float(np.min(ms)) / 1e3


def graph_time_us(fn, n_calls=20, reps=5):
    """Mean µs per call of a call whose GPU work is shorter than the binding's
    own host time: n_calls back-to-back calls are captured in a HIP graph
    and the replays are timed with HIP events on the replay stream."""
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn()
    stream.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n_calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * n_calls)


def attn_bytes(Tq, hq, hkv, hd, L, Tk):
    """Algorithmic bytes of one tree-attention call: the prefix K/V, the tree
    K/V, q in and out (bf16), and the mask rows."""
    return 2 * hkv * L * hd * 2 + 2 * hkv * Tk * hd * 2 + Tq * hq * hd * 4 + Tq * 8


def long_context_verify(dev, steps):
    """Tree mask + tree attention over 32 distinct layers' KV caches (Llama-3-8B
    attention shape, L = 32768, T = 64), layer after layer; HIP events around
    every attention call on its launch stream.  Then the KV commit of the
    accepted path into all 32 caches, one launch."""
    w = inputs.LONG_CONTEXT
    vi = inputs.verify_inputs(w, L=0, with_lmhead=False)   # tree, q and tree K/V
    C = w.L + w.T                                          # each cache: prefix, then the tree rows
    kc = torch.empty((w.layers, w.hkv, C, w.hd), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    for l in range(w.layers):
        kc[l, :, :w.L] = inputs.device_normal((w.hkv, w.L, w.hd), 4000 + 2 * l, dev)
        vc[l, :, :w.L] = inputs.device_normal((w.hkv, w.L, w.hd), 4001 + 2 * l, dev)
    par = torch.from_numpy(vi.parents).to(dev)
    q, kt, vt = vi.q.to(dev), vi.k_tree.to(dev), vi.v_tree.to(dev)
    kc[:, :, w.L:] = kt
    vc[:, :, w.L:] = vt
    out = torch.empty_like(q)
    lib = _lib.lib()
    ws = torch.zeros(lib.eagle_tree_attn_workspace(w.T, w.hq, w.hkv, w.hd, w.L, w.T, 1),
                     dtype=torch.uint8, device=dev)
    mask = torch.empty((w.T, 1), dtype=torch.int64, device=dev)
    depth = torch.empty(w.T, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def one_pass(evs=None):
        _lib.eagle_build_tree_mask(par, mask=mask, depth=depth)
        for l in range(w.layers):
            if evs is not None:
                evs[l][0].record(stream)
            _lib.eagle_tree_attn(q, kc[l], vc[l], w.L, kt, vt, w.T, mask, out=out, workspace=ws)
            if evs is not None:
                evs[l][1].record(stream)

    one_pass()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_pass()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(w.layers)]
    one_pass(evs)
    torch.cuda.synchronize()
    per = float(np.mean([a.elapsed_time(b) for a, b in evs])) / 1e3
    nb = attn_bytes(w.T, w.hq, w.hkv, w.hd, w.L, w.T)
    achieved = nb / per / 1e9

    # KV commit of the deepest root path (the tree rows sit right after each
    # layer's prefix), all 32 layers in one launch
    depths = [0] * w.T
    for i in range(1, w.T):
        depths[i] = depths[int(vi.parents[i])] + 1
    node = int(np.argmax(depths))
    path = []
    while node != -1:
        path.append(node)
        node = int(vi.parents[node])
    path = path[::-1]
    rows = torch.tensor(path, dtype=torch.int32, device=dev)
    n_acc = torch.tensor([len(path) - 1], dtype=torch.int32, device=dev)
    kv_us = graph_time_us(lambda: _lib.eagle_kv_commit(kc[:, :, w.L:], vc[:, :, w.L:], rows, kc,
                                                        vc, w.L, n_accepted=n_acc))
    kv_bytes = 2 * 2 * w.layers * w.hkv * len(path) * w.hd * 2       # K and V, read and written
    del kc, vc
    return {"workload": "llama3-8b-long-verify: tree mask + 32 layers of tree attention, 32 Q / 8 "
                        "KV heads, hd 128, bf16 KV prefix L=32768 per layer, T=64 depth <= 7",
            "value": round(w.T / dt, 1), "unit": "nodes/s", "ms_per_step": round(dt * 1e3, 4),
            "roofline": {"kernel": "eagle_tree_attn (tree_attn_ring_kernel + attn_merge_bf16_kernel), "
                                   "one layer", "bound": "hbm", "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("eagle_tree_attn_c4_layer_L32768_T64",
                                                     ["attn.hip", "common.h"]),
                         "avg_us": round(per * 1e6, 2), "bytes_per_launch": nb},
            "kv_commit": {"kernel": "eagle_kv_commit (kv_commit_kernel), accepted path of "
                                    f"{len(path)} rows into 32 layers x 8 KV heads, one launch, "
                                    "in place", "bound": "hbm",
                          "achieved": round(kv_bytes / kv_us / 1e3, 2), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(kv_bytes / kv_us / 1e3 / HBM_PEAK_GBS, 5),
                          "avg_us": round(kv_us, 2), "bytes_per_launch": kv_bytes,
                          "timing": "HIP graph of 20 back-to-back calls, replayed 5 times",
                          "note": "2 MB per launch: the call is bound by launch and memory "
                                  "latency, not by the HBM roofline"}}


MFMA_PEAK_TFLOPS = 2500.0        # dense bf16 (fp32 vector peak 157.3 TFLOP/s for the fp32 config)


def roofline_entry(kernel, nbytes, flops, us, mfma_peak=MFMA_PEAK_TFLOPS):
    """Achieved rate against the roofline that bounds the call: HBM when its
    bytes take longer at 8 TB/s than its flops at the MFMA peak, else MFMA."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e3)          # µs
    t_mfma = flops / (mfma_peak * 1e6)             # µs
    if t_hbm >= t_mfma:
        a = nbytes / us / 1e3
        return {"kernel": kernel, "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4), "avg_us": round(us, 2),
                "bytes_per_launch": int(nbytes), "flops_per_launch": int(flops)}
    a = flops / us / 1e6
    return {"kernel": kernel, "bound": "mfma", "achieved": round(a, 1), "peak": mfma_peak,
            "unit": "TFLOP/s", "frac": round(a / mfma_peak, 4), "avg_us": round(us, 2),
            "bytes_per_launch": int(nbytes), "flops_per_launch": int(flops),
            "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}


def event_time_us(fn, iters):
    """Mean µs per call of calls long enough to time one by one: HIP events
    around each call on the stream it is launched on."""
    stream = torch.cuda.current_stream()
    fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3


def rotated_graph_time_us(fns, reps=3):
    """Mean µs per call of short calls over distinct buffers (caches kept
    cold: the calls of one replay read more than the 256 MB last-level cache
    holds), captured back to back in one HIP graph."""
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fns[0]()
    stream.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for fn in fns:
            fn()
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * len(fns))


VERIFY_NAMES = {
    1: "tiny: d=256, 4 Q / 1 KV heads, hd 64, V=1024, fp32, L=128, T=15 depth <= 4, top-4, greedy",
    2: "qwen2-7b-verify: d=3584, 28 Q / 4 KV heads, hd 128, bf16 L=2048, T=60 depth <= 7, "
       "LM head V=152064 for all 60 nodes, top-10, greedy",
    5: "70b-wide-tree: d=8192, 64 Q / 8 KV heads, hd 128, bf16 L=8192, T=128 depth <= 7 (4-way "
       "near the root), LM head V=128256 with logits, top-10, greedy and sampling acceptance",
}


def verify_leg(dev, cfg, steps):
    """One verify pass of a workload: tree mask -> tree attention -> LM head
    -> acceptance (greedy, and sampling where the workload has it), replayed
    from a HIP graph with every input resident in HBM.  The LM-head weight and
    the large feature inputs are drawn on the GPU (same distributions as the
    host generator, other values); the tree, tokens, q and K/V come from the
    host generator.  Tokens follow the target's top-1 along one deepest path
    (planted), so acceptance walks to full depth."""
    w = inputs.WORKLOADS[cfg]
    fp32 = w.dtype == "f32"
    dt = torch.float32 if fp32 else torch.bfloat16
    vi = inputs.verify_inputs(w, with_lmhead=fp32)
    T, L, V, k = w.T, w.L, w.vocab, w.topk
    if fp32:
        f = vi.f.to(dev)
        W = inputs.lm_head_weight(w).to(dev)
    else:
        f = inputs.device_normal((T, w.d), 6000 + cfg, dev)
        W = (inputs.device_normal((V, w.d), 6100 + cfg, dev, dtype=torch.float32)
             * float(1.0 / np.sqrt(w.d))).to(torch.bfloat16)
    par = torch.from_numpy(vi.parents).to(dev)
    q, kc, vc, kt, vt = (t.to(dev) for t in (vi.q, vi.k_cache, vi.v_cache, vi.k_tree, vi.v_tree))
    lib = _lib.lib()
    i32 = dict(dtype=torch.int32, device=dev)
    mask = torch.empty((T, w.words), dtype=torch.int64, device=dev)
    depth = torch.empty(T, **i32)
    attn_out = torch.empty_like(q)
    ws_attn = torch.zeros(max(lib.eagle_tree_attn_workspace(T, w.hq, w.hkv, w.hd, L, T,
                                                            _lib._dt(q)), 256),
                          dtype=torch.uint8, device=dev)
    ws_lm = torch.zeros(lib.eagle_lmhead_topk_workspace(T, w.d, V, k, _lib._dt(f)),
                        dtype=torch.uint8, device=dev)
    ids = torch.empty((T, k), **i32)
    lp = torch.empty((T, k), dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    logits = torch.empty((T, V), dtype=torch.float32, device=dev) if w.sampling else None
    ws_acc = torch.zeros(max(lib.eagle_accept_workspace(T, V), 256), dtype=torch.uint8,
                         device=dev)
    u = torch.from_numpy(vi.uniforms).to(dev)
    outs_g = [torch.empty(T, **i32), torch.empty(1, **i32), torch.empty(1, **i32)]
    outs_s = [torch.empty(T, **i32), torch.empty(1, **i32), torch.empty(1, **i32)]
    status = torch.zeros(1, **i32)

    def lmhead():
        _lib.eagle_lmhead_topk(f, W, k, topk_id=ids, topk_logp=lp, lse=lse, logits=logits,
                               workspace=ws_lm)

    # plant the target's top-1 along a deepest path (setup, not timed)
    lmhead()
    top1 = ids[:, 0].cpu().numpy()
    g = inputs.rng(w.cfg, inputs.STREAM_TOK, 99)
    tok_np = inputs.plant_path(vi.tokens, vi.parents, top1, inputs.deepest_leaf(g, vi.parents))
    tok = torch.from_numpy(tok_np).to(dev)

    def attn():
        _lib.eagle_tree_attn(q, kc, vc, L, kt, vt, T, mask, out=attn_out, workspace=ws_attn,
                             dev_status=status)

    def step():
        _lib.eagle_build_tree_mask(par, mask=mask, depth=depth, dev_status=status)
        attn()
        lmhead()
        _lib.eagle_accept(_lib.EAGLE_GREEDY, tok, par, target_top1=ids[:, 0], path=outs_g[0],
                          n_accepted=outs_g[1], bonus_token=outs_g[2], dev_status=status)
        if w.sampling:
            _lib.eagle_accept(_lib.EAGLE_SAMPLE, tok, par, target_logits=logits,
                              temperature=1.0, uniforms=u, path=outs_s[0], n_accepted=outs_s[1],
                              bonus_token=outs_s[2], workspace=ws_acc, dev_status=status)

    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    dt_step = (time.perf_counter() - t0) / steps
    assert int(status.item()) == 0, f"config {cfg}: device status {int(status.item())}"
    depths = depth.cpu().numpy()
    leg = {"workload": VERIFY_NAMES[cfg], "value": round(T / dt_step, 1), "unit": "nodes/s",
           "ms_per_step": round(dt_step * 1e3, 4), "steps": steps,
           "accepted_greedy": int(outs_g[1].item()),
           "timing": "one step = mask, attention, LM head, acceptance, replayed from a HIP graph"}
    if w.sampling:
        leg["accepted_sampling"] = int(outs_s[1].item())

    # attention alone over rotated K/V copies (cold caches), one HIP graph
    es = 4 if fp32 else 2
    kv_bytes = 2 * w.hkv * L * w.hd * es
    n_rot = int(min(256, max(8, -(-(1 << 30) // kv_bytes))))
    if fp32:
        n_rot = 8
    kcs = [kc] + [kc.clone() for _ in range(n_rot - 1)]
    vcs = [vc] + [vc.clone() for _ in range(n_rot - 1)]
    fns = [(lambda a=a, b=b: _lib.eagle_tree_attn(q, a, b, L, kt, vt, T, mask, out=attn_out,
                                                  workspace=ws_attn)) for a, b in zip(kcs, vcs)]
    attn_us = rotated_graph_time_us(fns)
    del kcs, vcs, fns
    nvis = float(np.mean(depths + 1))
    a_bytes = (2 * w.hkv * L * w.hd * es + 2 * w.hkv * T * w.hd * es + T * w.hq * w.hd * 2 * es
               + T * w.words * 8)
    a_flops = 4 * T * w.hq * w.hd * (L + nvis)
    peak = 157.3 if fp32 else MFMA_PEAK_TFLOPS
    leg["attention"] = roofline_entry(f"eagle_tree_attn, Tq={T}, {w.hq}/{w.hkv} heads, hd "
                                      f"{w.hd}, L={L}", a_bytes, a_flops, attn_us, peak)
    leg["attention"]["timing"] = (f"HIP graph of {n_rot} calls over distinct K/V copies, "
                                  "replayed 3 times")
    # LM head alone (its weight alone exceeds the last-level cache at bf16)
    lm_us = event_time_us(lmhead, 20) if not fp32 else rotated_graph_time_us([lmhead] * 20)
    l_bytes = V * w.d * es + T * w.d * es + T * (8 * k + 4) + (4 * T * V if w.sampling else 0)
    l_flops = 2 * T * w.d * V
    leg["lmhead"] = roofline_entry(f"eagle_lmhead_topk, T={T}, d={w.d}, V={V}, k={k}"
                                   + (", logits written" if w.sampling else ""),
                                   l_bytes, l_flops, lm_us, peak)
    leg["lmhead"]["timing"] = ("HIP events around each of 20 calls" if not fp32
                               else "HIP graph of 20 calls, replayed 3 times")
    host = {"vi": vi, "tokens": tok_np, "top1": top1, "W": None if not fp32 else inputs.lm_head_weight(w),
            "f": vi.f}
    if not fp32:
        host["W"] = W.cpu()
        host["f"] = f.cpu()
    del W
    torch.cuda.empty_cache()
    return leg, host


def blas_vendor():
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version')}"
    except Exception:                                   # noqa: BLE001
        return "unknown"


def cpu_verify_pass(w, host):
    """The oracle's verify pass of a workload on the host: mask, attention,
    LM head (all rows), greedy acceptance; sampling acceptance where the
    workload has it.  Returns seconds."""
    import oracle
    vi = host["vi"]
    t0 = time.perf_counter()
    m, _ = oracle.build_tree_mask(vi.parents)
    oracle.tree_attention(vi.q, vi.k_cache, vi.v_cache, w.L, vi.k_tree, vi.v_tree, m)
    lg = oracle.lm_head_logits(host["f"], host["W"])
    ids = oracle.topk_ids(lg, w.topk)
    oracle.accept_greedy(host["tokens"], vi.parents, ids[:, 0])
    if w.sampling:
        oracle.accept_sample(host["tokens"], vi.parents, lg.astype(np.float32), 1.0, vi.uniforms)
    return time.perf_counter() - t0


def cpu_baseline(w, ci):
    """The oracle's full cycle on the host cores (one cycle: 6 draft rounds,
    rerank, verify layer, LM head, acceptance)."""
    import oracle
    from oracle.cycle import CycleWeights
    from oracle.layer import LayerWeights

    torch.set_num_threads(CORES)

    def lw(x):
        nq, nk = w.hq * w.hd, w.hkv * w.hd
        return LayerWeights(norm1=x["norm1"], wq=x["wqkv"][:nq], wk=x["wqkv"][nq:nq + nk],
                            wv=x["wqkv"][nq + nk:], wo=x["wo"], norm2=x["norm2"],
                            wgate=x["wgate"], wup=x["wup"], wdown=x["wdown"])
    cw = CycleWeights(ci["w_fuse"], lw(ci["draft"]), ci["draft_norm"], ci["embed"], ci["w_lm"],
                      lw(ci["target"]), ci["target_norm"], ci["draft_k_cache"],
                      ci["draft_v_cache"], ci["target_k_cache"], ci["target_v_cache"])
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.draft_and_verify_cycle(cw, ci["root_token"], ci["root_feature"], hq=w.hq,
                                      hkv=w.hkv, hd=w.hd, L=w.L, rounds=w.rounds, k=w.topk,
                                      k_select=w.k_select, T=w.T, temperature=w.temperature,
                                      uniforms=ci["uniforms"], theta=w.rope_theta, eps=w.rms_eps)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": round(w.T / dt, 3), "unit": "nodes/s", "cores": CORES, "kind": "oracle",
            "blas": blas_vendor(),
            "sample": "the full cycle of the same workload (6 draft rounds, rerank, verify layer, "
                      "LM head with logits, sampling acceptance), median of 3 runs: "
                      + ", ".join(f"{t:.1f}" for t in times) + " s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lm-iters", type=int, default=30)
    ap.add_argument("--no-long-context", action="store_true")
    ap.add_argument("--no-verify-configs", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="copy 512 MiB device to device first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the sharded design is described, not built)", file=sys.stderr)
        sys.exit(2)
    w = inputs.LLAMA3_8B_CYCLE
    dev = torch.device("cuda:0")
    if args.copy_probe:
        src = torch.zeros(256 << 20, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)      # one elementwise kernel: reads src once, writes dst once
        torch.cuda.synchronize()
        print("[bench] copy probe: 536870912 bytes read, 536870912 bytes written",
              file=sys.stderr, flush=True)
        del src, dst
    print(f"[bench] drawing inputs for {w.name}", file=sys.stderr, flush=True)
    ci = inputs.cycle_inputs(w)
    cyc = DraftVerifyCycle(w, ci, dev, temperature=w.temperature)
    print("[bench] inputs resident; capturing the cycle", file=sys.stderr, flush=True)
    if not args.no_graph:
        cyc.capture()
    for _ in range(args.warmup):
        cyc.run()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} cycles", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        cyc.run()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert int(cyc.status.item()) == 0, "device status reported bad data"
    ms = dt / args.steps * 1e3
    value = w.T * args.steps / dt

    # dominant kernel: the LM head at the draft-round shape (6 of the 7 LM-head
    # passes of a cycle), timed with HIP events on its launch stream
    Td = w.k_select
    avg_s, min_s = time_lmhead(cyc, Td, args.lm_iters)
    nbytes = lmhead_bytes(Td, w.d, w.vocab, w.topk)
    achieved = nbytes / avg_s / 1e9
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3-8b-cycle: fuse 8192->4096, one decoder layer (32 Q / 8 KV "
                               "heads, hd 128, SwiGLU 14336) over L=4096 + tree, LM head V=128256, "
                               "6 rounds of top-10, rerank to T=64, one target verify layer, "
                               "seeded-sampling accept",
                   "tree_nodes": w.T, "prefix": w.L, "rounds": w.rounds, "topk": w.topk,
                   "graph": not args.no_graph},
        "roofline": {"kernel": "eagle_lmhead_topk (lmhead_bf16_kernel + lmhead_merge_kernel), "
                               f"T={Td}, d={w.d}, V={w.vocab}, k={w.topk}",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("eagle_lmhead_topk_T10_d4096_V128256_k10",
                                                 ["lmhead.hip", "wstream.h", "common.h"]),
                     "avg_us": round(avg_s * 1e6, 2), "min_us": round(min_s * 1e6, 2),
                     "bytes_per_launch": nbytes},
    }
    # confidence gate at a draft round's shape (10 nodes x top-10), in place
    glp = -torch.sort(torch.rand((Td, w.topk), device=dev) * 8, dim=1).values
    gate_us = graph_time_us(lambda: _lib.eagle_gate_children(glp, 2.0, 4, out=glp))
    line["gate"] = {"kernel": f"eagle_gate_children (gate_children_kernel), {Td} nodes x top-"
                              f"{w.topk}, tau 2, up to 4 branches", "avg_us": round(gate_us, 2),
                    "bytes_per_launch": Td * w.topk * 8 + Td * 8,
                    "timing": "HIP graph of 20 back-to-back calls, replayed 5 times",
                    "note": "under 1 KB per launch: launch-latency bound"}
    # mixed-sampling processing of the verify pass's logits (64 rows of the
    # vocabulary; llama.cpp-like settings: temperature 0.8, top-k 40, top-p 0.95)
    lg = inputs.device_normal((w.T, w.vocab), 5100, dev, dtype=torch.float32) * 2.0
    lg_out = torch.empty_like(lg)
    lp_kept = torch.empty(w.T, dtype=torch.int32, device=dev)
    lp_ws = torch.zeros(max(_lib.lib().eagle_logits_process_workspace(w.T, w.vocab, 40), 256),
                        dtype=torch.uint8, device=dev)   # zero: its counters
    lp_us = graph_time_us(lambda: _lib.eagle_logits_process(lg, 0.8, 40, 0.95, out=lg_out,
                                                            kept=lp_kept, workspace=lp_ws),
                          n_calls=10)
    lp_bytes = 2 * w.T * w.vocab * 4
    line["logits_process"] = {"kernel": f"eagle_logits_process (lp_chunk_kernel), {w.T} rows x "
                                        f"V={w.vocab}, temperature 0.8, top-k 40, top-p 0.95",
                              "bound": "hbm", "achieved": round(lp_bytes / lp_us / 1e3, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(lp_bytes / lp_us / 1e3 / HBM_PEAK_GBS, 4),
                              "avg_us": round(lp_us, 2), "bytes_per_launch": lp_bytes,
                              "timing": "HIP graph of 10 back-to-back calls, replayed 5 times"}
    del lg, lg_out, lp_ws
    # speculative sampling with the draft's distribution over the verify tree
    # (64 nodes, V = 128256, target and draft logits, a planted path)
    g = inputs.rng(w.cfg, inputs.STREAM_U, 7)
    par_np = inputs.random_tree(g, w.T, 7, 4)
    tl = inputs.device_normal((w.T, w.vocab), 5200, dev, dtype=torch.float32) * 2.0
    dlq = 0.5 * tl + inputs.device_normal((w.T, w.vocab), 5201, dev, dtype=torch.float32)
    tok_np = inputs.sibling_distinct_tokens(g, par_np, w.vocab)
    tok_np = inputs.plant_path(tok_np, par_np, tl.argmax(1).int().cpu().numpy(),
                               inputs.deepest_leaf(g, par_np))
    tok_q, par_q = torch.from_numpy(tok_np).to(dev), torch.from_numpy(par_np).to(dev)
    u_q = torch.from_numpy(inputs.uniforms(g, 2 * w.T)).to(dev)
    q_ws = torch.zeros(_lib.lib().eagle_accept_q_workspace(w.T, w.vocab), dtype=torch.uint8,
                       device=dev)
    q_out = [torch.empty(w.T, dtype=torch.int32, device=dev),
             torch.empty(1, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev)]
    aq_us = graph_time_us(lambda: _lib.eagle_accept_q(tok_q, par_q, tl, dlq, w.temperature, u_q,
                                                      path=q_out[0], n_accepted=q_out[1],
                                                      bonus_token=q_out[2], workspace=q_ws),
                          n_calls=5, reps=3)
    line["accept_q"] = {"kernel": f"eagle_accept_q (accept_q_grid_kernel), {w.T} nodes, "
                                  f"V={w.vocab}, draft distribution from draft logits",
                        "avg_us": round(aq_us, 1), "accepted": int(q_out[1].item()),
                        "timing": "HIP graph of 5 back-to-back calls, replayed 3 times",
                        "note": "one launch of 128 workgroups (256 beyond 262144 tokens), each "
                                "owning a slice of the vocabulary, walks the tree together and "
                                "meets only for sums over the vocabulary (row statistics of a "
                                "visited node, a rejection's residual mass, the bonus draw), each "
                                "meeting an all-gather of tagged records that every workgroup "
                                "combines in the same order"}
    del tl, dlq
    # Eagle-3 fusion of the accepted path's three recorded hidden states
    # (8 rows: root + 7 accepted at the tree's depth bound), d = 4096 -> 4096
    Mf = 8
    hs = [inputs.device_normal((Mf, w.d), 5000 + i, dev) for i in range(3)]
    w_fc = inputs.device_normal((w.d, 3 * w.d), 5003, dev) * (1.0 / np.sqrt(3 * w.d))
    g_out = torch.empty((Mf, w.d), dtype=torch.float32, device=dev)
    f_ws = torch.zeros(max(_lib.lib().eagle_linear_workspace(Mf, 3 * w.d, w.d, 0), 256),
                       dtype=torch.uint8, device=dev)
    fuse_us = graph_time_us(lambda: _lib.eagle_fuse3(*hs, w_fc, out=g_out, workspace=f_ws))
    fuse_bytes = w.d * 3 * w.d * 2 + Mf * 3 * w.d * 2 + Mf * w.d * 4
    line["fusion"] = {"kernel": f"eagle_fuse3 (linear_rows_kernel, three input segments), M={Mf}, "
                                f"3x{w.d} -> {w.d}", "bound": "hbm",
                      "achieved": round(fuse_bytes / fuse_us / 1e3, 1), "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": round(fuse_bytes / fuse_us / 1e3 / HBM_PEAK_GBS, 4),
                      "avg_us": round(fuse_us, 2), "bytes_per_launch": fuse_bytes,
                      "timing": "HIP graph of 20 back-to-back calls, replayed 5 times"}
    del hs, w_fc
    del cyc
    torch.cuda.empty_cache()
    hosts = {}
    if not args.no_verify_configs:
        for cfg in (2, 5, 1):
            print(f"[bench] verify pass, config {inputs.WORKLOADS[cfg].name}", file=sys.stderr,
                  flush=True)
            line[f"verify_{inputs.WORKLOADS[cfg].name}"], hosts[cfg] = verify_leg(dev, cfg,
                                                                                 args.steps)
    if not args.no_long_context:
        print("[bench] long-context verify (32 layers, L=32768)", file=sys.stderr, flush=True)
        line["long_context_verify"] = long_context_verify(dev, max(1, min(args.steps, 10)))
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on one cycle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, ci)
        per = {}
        for cfg, host in hosts.items():
            wc = inputs.WORKLOADS[cfg]
            print(f"[bench] timing the CPU oracle on one {wc.name} verify pass", file=sys.stderr,
                  flush=True)
            t = cpu_verify_pass(wc, host)
            per[wc.name] = {"value": round(wc.T / t, 2), "unit": "nodes/s",
                            "sample": f"one verify pass (mask, attention, LM head, acceptance) "
                                      f"in {t:.2f} s"}
        if not args.no_long_context:
            import oracle
            wl = inputs.LONG_CONTEXT
            print("[bench] timing the CPU oracle on one long-context layer", file=sys.stderr,
                  flush=True)
            vl = inputs.verify_inputs(wl, with_lmhead=False)
            t0 = time.perf_counter()
            ml, _ = oracle.build_tree_mask(vl.parents)
            oracle.tree_attention(vl.q, vl.k_cache, vl.v_cache, wl.L, vl.k_tree, vl.v_tree, ml)
            t = time.perf_counter() - t0
            per[wl.name] = {"value": round(wl.T / (wl.layers * t), 3), "unit": "nodes/s",
                            "sample": f"one of the 32 layers (mask and attention) in {t:.2f} s, "
                                      "scaled to 32 layers"}
        line["cpu_baseline"]["per_config"] = per
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
