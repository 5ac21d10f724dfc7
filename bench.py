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
    ws = torch.empty(lib.eagle_tree_attn_workspace(w.T, w.hq, w.hkv, w.hd, w.L, w.T, 1),
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
    t0 = time.perf_counter()
    oracle.draft_and_verify_cycle(cw, ci["root_token"], ci["root_feature"], hq=w.hq, hkv=w.hkv,
                                  hd=w.hd, L=w.L, rounds=w.rounds, k=w.topk,
                                  k_select=w.k_select, T=w.T, temperature=w.temperature,
                                  uniforms=ci["uniforms"], theta=w.rope_theta, eps=w.rms_eps)
    dt = time.perf_counter() - t0
    return {"value": w.T / dt, "unit": "nodes/s", "cores": CORES, "kind": "oracle",
            "sample": "one full cycle of the same workload (6 draft rounds, rerank, verify "
                      f"layer, LM head with logits, sampling acceptance) in {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lm-iters", type=int, default=30)
    ap.add_argument("--no-long-context", action="store_true")
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
    line["accept_q"] = {"kernel": f"eagle_accept_q (accept_sample_q_kernel), {w.T} nodes, "
                                  f"V={w.vocab}, draft distribution from draft logits",
                        "avg_us": round(aq_us, 1), "accepted": int(q_out[1].item()),
                        "timing": "HIP graph of 5 back-to-back calls, replayed 3 times",
                        "note": "row statistics from a many-workgroup prepass; one workgroup "
                                "walks the tree, passing over the vocabulary only for rejections "
                                "and the bonus draw"}
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
    if not args.no_long_context:
        del cyc
        torch.cuda.empty_cache()
        print("[bench] long-context verify (32 layers, L=32768)", file=sys.stderr, flush=True)
        line["long_context_verify"] = long_context_verify(dev, max(1, min(args.steps, 10)))
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on one cycle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, ci)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
