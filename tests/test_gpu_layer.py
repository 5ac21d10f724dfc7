"""GPU parity: decoder-layer support kernels against the oracle.

Tolerances follow from the arithmetic: the projections accumulate in fp32
(relative error ~1e-6 of the output scale); a bf16 output adds one rounding
(u = 2^-8 relative at most); the full layer passes its activations through
seven bf16 roundings (normed input, q/k/v, attention probabilities, attention
output, normed MLP input, MLP hidden), each adding about u/2 relative RMS
error, so its output is held to a relative L2 error of 8u = 3.1e-2 and a max
error of 16u = 6.3e-2 of the output scale."""
import numpy as np
import pytest
import torch

import oracle
from oracle.layer import LayerWeights, linear, swiglu_mlp_hidden
from speculative_decoding_parent_amd import _lib, inputs
from speculative_decoding_parent_amd.cycle import DraftVerifyCycle

pytestmark = pytest.mark.gpu
U = 2.0 ** -8


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("M,K,N", [(1, 128, 256), (10, 4096, 1000), (17, 512, 6144),
                                   (64, 4096, 4096), (130, 256, 300), (16, 8192, 4096),
                                   (3, 14336, 4096), (5, 384, 30), (12, 1024, 100)])
def test_linear(dev, M, K, N):
    print(f"linear M={M} K={K} N={N}", flush=True)
    g = inputs.rng(700, M, N)
    x = inputs.normal(g, (M, K))
    W = inputs.normal(g, (N, K), std=float(1 / np.sqrt(K)))
    res = inputs.normal(g, (M, N), dtype=torch.float32)
    ref = linear(x, W)
    got = _lib.eagle_linear(x.to(dev), W.to(dev)).cpu().numpy()
    assert np.abs(got - ref).max() <= 1e-4 * np.abs(ref).max() + 1e-6
    got = _lib.eagle_linear(x.to(dev), W.to(dev), residual=res.to(dev)).cpu().numpy()
    assert np.abs(got - (ref + res.numpy())).max() <= 1e-4 * np.abs(ref).max() + 1e-5
    gb = _lib.eagle_linear(x.to(dev), W.to(dev), out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.all(np.abs(gb - ref) <= U * np.abs(ref) + 1e-4 * np.abs(ref).max())


@pytest.mark.parametrize("M,K,N", [(1, 256, 512), (10, 4096, 14336), (64, 512, 1000),
                                   (16, 384, 100), (7, 14336, 64)])
def test_swiglu(dev, M, K, N):
    print(f"swiglu M={M} K={K} N={N}", flush=True)
    g = inputs.rng(701, M, N)
    x = inputs.normal(g, (M, K))
    wg = inputs.normal(g, (N, K), std=float(1 / np.sqrt(K)))
    wu = inputs.normal(g, (N, K), std=float(1 / np.sqrt(K)))
    ref = swiglu_mlp_hidden(x, wg, wu)
    got = _lib.eagle_linear_swiglu(x.to(dev), wg.to(dev), wu.to(dev)).float().cpu().numpy()
    assert np.all(np.abs(got - ref) <= U * np.abs(ref) + 1e-4 * np.abs(ref).max())


@pytest.mark.parametrize("M,K,N,res", [(1, 8192, 4096, False), (10, 4096, 4096, True),
                                       (64, 14336, 4096, True), (7, 256, 8192, True),
                                       (16, 14336, 4096, True), (1, 128, 256, False),
                                       (10, 8192, 4096, True), (3, 512, 100, True)])
def test_linear_rmsnorm(dev, M, K, N, res):
    print(f"linear_rmsnorm M={M} K={K} N={N}", flush=True)
    g = inputs.rng(707, M, K)
    x = inputs.normal(g, (M, K))
    W = inputs.normal(g, (N, K), std=float(1 / np.sqrt(K)))
    r = inputs.normal(g, (M, N), dtype=torch.float32) if res else None
    gamma = 1 + 0.1 * inputs.normal(g, (N,), dtype=torch.float32)
    out, nrm = _lib.eagle_linear_rmsnorm(x.to(dev), W.to(dev), gamma.to(dev),
                                         residual=None if r is None else r.to(dev))
    ref = linear(x, W) + (0 if r is None else r.numpy())
    assert np.abs(out.cpu().numpy() - ref).max() <= 1e-4 * np.abs(ref).max() + 1e-5
    rn = oracle.rms_norm(ref, gamma, 1e-5)
    assert np.all(np.abs(nrm.float().cpu().numpy() - rn) <= U * np.abs(rn) + 1e-4 * np.abs(rn).max())


@pytest.mark.parametrize("M,K,hq,hkv,hd", [(10, 4096, 32, 8, 128), (16, 256, 4, 2, 64),
                                           (20, 256, 4, 2, 64), (3, 256, 2, 1, 96),
                                           (1, 512, 8, 2, 128)])
def test_linear_rope_qkv(dev, M, K, hq, hkv, hd):
    print(f"linear_rope_qkv M={M} K={K} hq={hq} hkv={hkv} hd={hd}", flush=True)
    g = inputs.rng(708, M, hd)
    cap, L = 51, 4096
    x = inputs.normal(g, (M, K))
    W = inputs.normal(g, ((hq + 2 * hkv) * hd, K), std=float(1 / np.sqrt(K)))
    depth = g.integers(0, 7, M).astype(np.int32)
    slots = g.choice(cap, M, replace=False).astype(np.int32)
    kt = torch.zeros((hkv, cap, hd), dtype=torch.bfloat16, device=dev)
    vt = torch.zeros_like(kt)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    q = _lib.eagle_linear_rope_qkv(x.to(dev), W.to(dev), hq, hkv, hd, torch.from_numpy(depth).to(dev),
                                   L, kt, vt, row_slot=torch.from_numpy(slots).to(dev), dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    qkv = linear(x, W).reshape(M, hq + 2 * hkv, hd)
    pos = L + depth
    rq, rk = oracle.rope(qkv[:, :hq], pos), oracle.rope(qkv[:, hq:hq + hkv], pos)
    tol = lambda r: U * np.abs(r) + 1e-4 * np.abs(r).max()
    assert np.all(np.abs(q.float().cpu().numpy() - rq) <= tol(rq))
    ktn, vtn = kt.float().cpu().numpy(), vt.float().cpu().numpy()
    kmax, vmax = np.abs(rk).max(), np.abs(qkv[:, hq + hkv:]).max()
    for m in range(M):
        assert np.all(np.abs(ktn[:, slots[m]] - rk[m]) <= U * np.abs(rk[m]) + 1e-4 * kmax)
        vr = qkv[m, hq + hkv:]
        assert np.all(np.abs(vtn[:, slots[m]] - vr) <= U * np.abs(vr) + 1e-4 * vmax)


def bf16_round(a):
    """fp32 -> bf16 -> fp32, round to nearest even (numpy)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def deferred(dev, M, K, N, seed):
    g = inputs.rng(seed, M, K * 100003 + N)
    x = inputs.normal(g, (M, K))
    W = inputs.normal(g, (N, K), std=float(1 / np.sqrt(K)))
    res = inputs.normal(g, (M, N), dtype=torch.float32)
    gamma = 1 + 0.1 * inputs.normal(g, (N,), dtype=torch.float32)
    out, xg, ssq = _lib.eagle_linear_rmsnorm_deferred(x.to(dev), W.to(dev), gamma.to(dev),
                                                      residual=res.to(dev))
    torch.cuda.synchronize()
    return x, W, res, gamma, out.cpu().numpy(), xg.float().cpu().numpy(), ssq.cpu().numpy()


@pytest.mark.parametrize("M,K,N", [(10, 8192, 4096), (1, 4096, 4096), (16, 14336, 4096),
                                   (3, 256, 100), (64, 4096, 4096), (17, 512, 256)])
def test_linear_rmsnorm_deferred(dev, M, K, N):
    """Producer: out = x W^T + residual; xg = bf16(out * gamma) exactly; the
    partial sums of squares add up to sum out^2."""
    print(f"linear_rmsnorm_deferred M={M} K={K} N={N}", flush=True)
    x, W, res, gamma, out, xg, ssq = deferred(dev, M, K, N, 710)
    ref = linear(x, W) + res.numpy()
    assert np.abs(out - ref).max() <= 1e-4 * np.abs(ref).max() + 1e-5
    assert np.array_equal(xg, bf16_round(out * gamma.numpy()))
    assert ssq.shape == (_lib.lib().eagle_linear_norm_parts(M, K, N), M)
    want = (out.astype(np.float64) ** 2).sum(1)
    np.testing.assert_allclose(ssq.astype(np.float64).sum(0), want, rtol=1e-5)


def row_scale(out, eps=1e-5):
    return 1.0 / np.sqrt((out.astype(np.float64) ** 2).mean(1) + eps)


@pytest.mark.parametrize("M,K,N", [(10, 4096, 14336), (64, 512, 1000), (1, 256, 512)])
def test_swiglu_deferred_norm(dev, M, K, N):
    """Consumer: silu(r x W_g^T) * (r x W_u^T) with the row scale r taken from
    the producer's partial sums; compared on the producer's own bf16 rows."""
    print(f"swiglu deferred M={M} K={K} N={N}", flush=True)
    _, _, _, _, out, xg, ssq = deferred(dev, M, 256, K, 711)
    g = inputs.rng(712, M, N)
    wg = inputs.normal(g, (N, K), std=float(1 / np.sqrt(K)))
    wu = inputs.normal(g, (N, K), std=float(1 / np.sqrt(K)))
    xgt = torch.from_numpy(xg).to(torch.bfloat16)
    got = _lib.eagle_linear_swiglu(xgt.to(dev), wg.to(dev), wu.to(dev),
                                   in_norm=(torch.from_numpy(ssq).to(dev), 1e-5)).float().cpu().numpy()
    r = row_scale(out)[:, None]
    gt, up = r * linear(xgt, wg), r * linear(xgt, wu)
    ref = gt / (1 + np.exp(-gt)) * up
    assert np.all(np.abs(got - ref) <= U * np.abs(ref) + 1e-4 * np.abs(ref).max())


@pytest.mark.parametrize("M,hd", [(10, 128), (20, 64)])
def test_rope_qkv_deferred_norm(dev, M, hd):
    print(f"rope deferred M={M} hd={hd}", flush=True)
    hq, hkv, cap, L = 4, 2, 40, 4096
    N = (hq + 2 * hkv) * hd
    _, _, _, _, out, xg, ssq = deferred(dev, M, 256, 512, 713)
    g = inputs.rng(714, M, hd)
    W = inputs.normal(g, (N, 512), std=float(1 / np.sqrt(512)))
    depth = g.integers(0, 7, M).astype(np.int32)
    slots = g.choice(cap, M, replace=False).astype(np.int32)
    kt = torch.zeros((hkv, cap, hd), dtype=torch.bfloat16, device=dev)
    vt = torch.zeros_like(kt)
    xgt = torch.from_numpy(xg).to(torch.bfloat16)
    q = _lib.eagle_linear_rope_qkv(xgt.to(dev), W.to(dev), hq, hkv, hd,
                                   torch.from_numpy(depth).to(dev), L, kt, vt,
                                   row_slot=torch.from_numpy(slots).to(dev),
                                   in_norm=(torch.from_numpy(ssq).to(dev), 1e-5))
    qkv = (row_scale(out)[:, None] * linear(xgt, W)).reshape(M, hq + 2 * hkv, hd)
    rq = oracle.rope(qkv[:, :hq], L + depth)
    assert np.all(np.abs(q.float().cpu().numpy() - rq) <= U * np.abs(rq) + 1e-4 * np.abs(rq).max())
    rk = oracle.rope(qkv[:, hq:hq + hkv], L + depth)
    ktn = kt.float().cpu().numpy()
    for m in range(M):
        assert np.all(np.abs(ktn[:, slots[m]] - rk[m]) <= U * np.abs(rk[m]) + 1e-4 * np.abs(rk).max())


@pytest.mark.parametrize("T,V,k", [(10, 20000, 10), (64, 5000, 10), (1, 3000, 4)])
def test_lmhead_deferred_norm(dev, T, V, k):
    """LM head on deferred-norm rows: logits = r (xg W^T), top-k and lse of
    those logits."""
    print(f"lmhead deferred T={T} V={V}", flush=True)
    d = 512
    _, _, _, _, out, xg, ssq = deferred(dev, T, 256, d, 715)
    g = inputs.rng(716, T, V)
    W = inputs.normal(g, (V, d), std=float(1 / np.sqrt(d)))
    xgt = torch.from_numpy(xg).to(torch.bfloat16)
    ids, logp, lse, lg = _lib.eagle_lmhead_topk(xgt.to(dev), W.to(dev), k, want_logits=True,
                                                in_norm=(torch.from_numpy(ssq).to(dev), 1e-5))
    torch.cuda.synchronize()
    ref = row_scale(out)[:, None] * oracle.lm_head_logits(xgt, W)
    lg = lg.cpu().numpy()
    assert np.abs(lg - ref).max() <= 1e-4 * np.abs(ref).max() + 1e-5
    assert np.array_equal(ids.cpu().numpy(), oracle.topk_ids(lg, k))
    _, _, rlse = oracle.softmax_stats(ref)
    assert np.abs(lse.cpu().numpy() - rlse).max() <= 1e-3


def test_shared_workspace_reuse(dev):
    """One zeroed workspace serves a sequence of few-row projections of
    different shapes (and a many-row one); each result matches a fresh call and
    the counter area is zero again afterwards."""
    g = inputs.rng(709, 0)
    shapes = [(10, 8192, 4096), (10, 4096, 4096), (1, 14336, 4096), (64, 4096, 4096),
              (16, 4096, 6144), (10, 8192, 4096)]
    nb = max(_lib.lib().eagle_linear_rows_workspace(M, K, N) for M, K, N in shapes)
    ws = torch.zeros(nb, dtype=torch.uint8, device=dev)
    for rep in range(2):
        for (M, K, N) in shapes:
            print(f"shared ws rep={rep} M={M} K={K} N={N}", flush=True)
            x = inputs.normal(g, (M, K)).to(dev)
            W = inputs.normal(g, (N, K), std=float(1 / np.sqrt(K))).to(dev)
            gamma = (1 + 0.1 * inputs.normal(g, (N,), dtype=torch.float32)).to(dev)
            res = inputs.normal(g, (M, N), dtype=torch.float32).to(dev)
            o1, n1 = _lib.eagle_linear_rmsnorm(x, W, gamma, residual=res, workspace=ws)
            o2, n2 = _lib.eagle_linear_rmsnorm(x, W, gamma, residual=res)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(n1, n2)
            y1 = _lib.eagle_linear(x, W, workspace=ws)
            y2 = _lib.eagle_linear(x, W)
            assert torch.equal(y1, y2)
    torch.cuda.synchronize()
    assert int(ws[:65536].count_nonzero().item()) == 0


def test_rmsnorm(dev):
    g = inputs.rng(702, 0)
    x = inputs.normal(g, (33, 4096), std=3.0, dtype=torch.float32)
    gamma = 1 + 0.1 * inputs.normal(g, (4096,), dtype=torch.float32)
    ref = oracle.rms_norm(x, gamma, 1e-5)
    got = _lib.eagle_rmsnorm(x.to(dev), gamma.to(dev)).float().cpu().numpy()
    assert np.all(np.abs(got - ref) <= U * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("L,hd", [(4096, 128), (32768, 128), (64, 64)])
def test_rope_qkv(dev, L, hd):
    g = inputs.rng(703, L, hd)
    M, hq, hkv, cap = 10, 8, 2, 24
    qkv = inputs.normal(g, (M, (hq + 2 * hkv) * hd), dtype=torch.float32)
    depth = g.integers(0, 8, M).astype(np.int32)
    slots = g.choice(cap, M, replace=False).astype(np.int32)
    kt = torch.zeros((hkv, cap, hd), dtype=torch.bfloat16, device=dev)
    vt = torch.zeros((hkv, cap, hd), dtype=torch.bfloat16, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    q = _lib.eagle_rope_qkv(qkv.to(dev), hq, hkv, hd, torch.from_numpy(depth).to(dev), L, kt, vt,
                            row_slot=torch.from_numpy(slots).to(dev), dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    x = qkv.numpy().astype(np.float64).reshape(M, hq + 2 * hkv, hd)
    pos = L + depth
    rq = oracle.rope(x[:, :hq], pos)
    rk = oracle.rope(x[:, hq:hq + hkv], pos)
    tol = lambda r: U * np.abs(r) + 1e-6
    assert np.all(np.abs(q.float().cpu().numpy() - rq) <= tol(rq))
    ktn = kt.float().cpu().numpy()
    vtn = vt.float().cpu().numpy()
    for m in range(M):
        assert np.all(np.abs(ktn[:, slots[m]] - rk[m]) <= tol(rk[m]))
        assert np.all(np.abs(vtn[:, slots[m]] - x[m, hq + hkv:]) <= tol(x[m, hq + hkv:]))
    untouched = np.setdiff1d(np.arange(cap), slots)
    assert np.all(ktn[:, untouched] == 0)


def test_draft_prepare_and_embed(dev):
    """Round bookkeeping is integer work: compared exactly with a hand model;
    slot mask rows against the oracle's mask of the slot tree."""
    g = inputs.rng(704, 0)
    V, d, cap, S = 500, 128, 40, 12
    # pool: root, 4 children (first expansion), then 8 entries below frontier [1, 3]
    par = np.array([-1, 0, 0, 0, 0, 1, 1, 1, 1, 3, 3, 3, 3], np.int32)
    dep = np.array([0, 1, 1, 1, 1, 2, 2, 2, 2, 2, 2, 2, 2], np.int32)
    tok = g.integers(0, V, 13).astype(np.int32)
    P = lambda a, n=cap, fill=0: torch.from_numpy(np.concatenate([a, np.full(n - len(a), fill, np.int32)])).to(dev)
    pt, pp, pd = P(tok), P(par, fill=-1), P(dep)
    slot_of = torch.full((cap,), -1, dtype=torch.int32, device=dev)
    slot_parent = torch.full((S,), -1, dtype=torch.int32, device=dev)
    smask = torch.zeros((S, 1), dtype=torch.int64, device=dev)
    rows = [torch.zeros(4, dtype=torch.int32, device=dev) for _ in range(4)]
    feat = inputs.normal(g, (S, d), dtype=torch.float32)
    root = inputs.normal(g, (d,), dtype=torch.float32)
    emb = inputs.normal(g, (V, d))
    fd, rd, ed = feat.to(dev), root.to(dev), emb.to(dev)
    x_in = torch.zeros((4, 2 * d), dtype=torch.bfloat16, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    for fr, n, base in (([0], 1, 0), ([1, 3], 5, 1), ([6, 9, 12], 13, 3)):
        _lib.eagle_draft_prepare(torch.tensor(fr, dtype=torch.int32, device=dev), pt, pp, pd, n,
                                 slot_of, base, slot_parent, [r[:len(fr)] for r in rows],
                                 slot_mask=smask, feat=fd, root_feat=rd, embed=ed,
                                 x_in=x_in[:len(fr)], dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    sp = slot_parent.cpu().tolist()[:6]
    assert sp == [-1, 0, 0, 1, 2, 2]
    assert slot_of.cpu().tolist()[:13] == [0, 1, -1, 2, -1, -1, 3, -1, -1, 4, -1, -1, 5]
    assert rows[0].cpu().tolist()[:3] == [tok[6], tok[9], tok[12]]
    assert rows[1].cpu().tolist()[:3] == [2, 2, 2]
    assert rows[2].cpu().tolist()[:3] == [3, 4, 5]
    assert rows[3].cpu().tolist()[:3] == [1, 2, 2]
    ref_mask, _ = oracle.build_tree_mask(np.array(sp, np.int32))
    assert np.array_equal(smask[:6].cpu().numpy().view(np.uint64), ref_mask)
    want = torch.stack([torch.cat([feat[s].to(torch.bfloat16), emb[t]]) for s, t in
                        [(1, tok[6]), (2, tok[9]), (2, tok[12])]])
    assert torch.equal(x_in[:3].cpu(), want)
    tk = torch.tensor([7, 8, 499], dtype=torch.int32, device=dev)
    e = _lib.eagle_embed(tk, ed).cpu()
    assert torch.equal(e, emb[[7, 8, 499]].float())


@pytest.mark.parametrize("M,d", [(64, 4096), (3, 256), (1, 8)])
def test_embed_deferred(dev, M, d):
    """Embedding rows with the next RMSNorm deferred: out exact, xg the bf16
    rounding of out * gamma, ssq the row sums of squares; a bad token reads
    row 0 and sets the status."""
    g = inputs.rng(716, M, d)
    V = 500
    emb = inputs.normal(g, (V, d))
    gamma = inputs.normal(g, (d,), dtype=torch.float32)
    tok = torch.from_numpy(g.integers(0, V, M).astype(np.int32))
    if M > 1:
        tok[1] = V + 3
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    print(f"embed deferred M={M} d={d}", flush=True)
    out, xg, ssq = _lib.eagle_embed_deferred(tok.to(dev), emb.to(dev), gamma.to(dev),
                                             dev_status=status)
    torch.cuda.synchronize()
    rows = tok.clone().long()
    rows[(rows < 0) | (rows >= V)] = 0
    x = emb[rows].double()
    assert torch.equal(out.cpu(), emb[rows].float())
    want_xg = (emb[rows].float() * gamma).to(torch.bfloat16)
    assert torch.equal(xg.cpu(), want_xg)
    np.testing.assert_allclose(ssq.cpu().numpy()[0], (x * x).sum(1).numpy(), rtol=1e-5)
    assert int(status.item()) == (_lib.DEV_BAD_TOKEN if M > 1 else 0)


def layer_case(dev, w, seed, n, Tk, slots, slot_par):
    """One decoder layer on n rows at the given slots vs the oracle."""
    ci = inputs.cycle_inputs(w)
    lw = ci["draft"]
    g = inputs.rng(705, seed)
    x = inputs.normal(g, (n, w.d), dtype=torch.float32)
    depth = g.integers(0, 6, n).astype(np.int32)
    cyc = DraftVerifyCycle(w, ci, dev)
    kt = torch.zeros((w.hkv, Tk, w.hd), dtype=torch.bfloat16, device=dev)
    vt = torch.zeros_like(kt)
    prev = np.setdiff1d(np.arange(Tk), slots)            # K/V of earlier slots
    kprev = inputs.normal(g, (w.hkv, len(prev), w.hd))
    vprev = inputs.normal(g, (w.hkv, len(prev), w.hd))
    kt[:, prev] = kprev.to(dev)
    vt[:, prev] = vprev.to(dev)
    mask, _ = _lib.eagle_build_tree_mask(torch.from_numpy(slot_par).to(dev))
    out = torch.zeros((n, w.d), dtype=torch.float32, device=dev)
    sl = torch.from_numpy(slots.astype(np.int32)).to(dev)
    lwd = {k: v.to(dev) for k, v in lw.items()}
    _lib.eagle_rmsnorm(x.to(dev), lwd["norm1"], w.rms_eps, out=cyc.n1[:n])
    cyc._layer(lwd, n, cyc.n1[:n], None, x.to(dev), torch.from_numpy(depth).to(dev), sl, cyc.dkc,
               cyc.dvc, kt, vt, Tk, mask, out, sl, cyc.draft_norm)
    torch.cuda.synchronize()
    assert int(cyc.status.item()) == 0
    nq = w.hq * w.hd
    ow = LayerWeights(norm1=lw["norm1"], wq=lw["wqkv"][:nq], wk=lw["wqkv"][nq:nq + w.hkv * w.hd],
                      wv=lw["wqkv"][nq + w.hkv * w.hd:], wo=lw["wo"], norm2=lw["norm2"],
                      wgate=lw["wgate"], wup=lw["wup"], wdown=lw["wdown"])
    kt0 = np.zeros((w.hkv, Tk, w.hd))
    vt0 = np.zeros((w.hkv, Tk, w.hd))
    kt0[:, prev] = kprev.float().numpy()
    vt0[:, prev] = vprev.float().numpy()
    ref_mask, _ = oracle.build_tree_mask(slot_par)
    ref, _, _ = oracle.decoder_layer(x, ow, w.L + depth, w.hq, w.hkv, w.hd, ci["draft_k_cache"],
                                     ci["draft_v_cache"], w.L, kt0, vt0, list(slots), ref_mask,
                                     list(slots))
    got = out.cpu().numpy()
    e2 = rel_l2(got - x.numpy(), ref - x.numpy())        # error relative to the layer's update
    em = np.abs(got - ref).max() / np.abs(ref - x.numpy()).max()
    print(f"  layer rel L2 {e2:.3e} max {em:.3e}", flush=True)
    assert e2 <= 8 * U and em <= 16 * U


def test_layer_small(dev):
    w = inputs.SMALL_CYCLE
    slot_par = np.array([-1, 0, 0, 0, 1, 1, 2, 3, 4, 4], np.int32)
    layer_case(dev, w, 0, 4, 10, np.array([6, 7, 8, 9]), slot_par)


def test_layer_llama3_8b_shape(dev):
    """The Llama-3-8B draft layer at full width on one round's 10 rows."""
    w = inputs.LLAMA3_8B_CYCLE
    g = inputs.rng(706, 0)
    slot_par = np.concatenate([[-1], np.zeros(10), 1 + g.integers(0, 10, 10)]).astype(np.int32)
    layer_case(dev, w, 1, 10, 21, np.arange(11, 21), slot_par)


def test_verify_layer_llama3_8b_shape(dev):
    """The verify pass's layer at full width on all 64 tree rows: the many-row
    projections (M > 16) composed with the wide-group attention kernel, under
    a 64-node tree mask, against the oracle's layer."""
    w = inputs.LLAMA3_8B_CYCLE
    slot_par = inputs.random_tree(inputs.rng(707, 0), 64, 7, 4).astype(np.int32)
    layer_case(dev, w, 2, 64, 64, np.arange(64), slot_par)


def test_split_k_hand_off_is_deterministic(dev):
    """The split-K few-row projections hand fp32 tiles between workgroups
    (device-coherent stores, then an arrival count; the last arrival sums the
    tiles in range order).  If an arrival were counted before its tiles had
    landed, the summing workgroup would read a partial tile on some calls.
    Every one of 200 back-to-back calls must be bit-identical to the first,
    at the draft's down projection (14336 -> 4096, deferred norm) and gate/up
    (4096 -> 14336) shapes."""
    g = inputs.rng(720, 0)
    M = 10
    x = inputs.normal(g, (M, 14336)).to(dev)
    W = inputs.normal(g, (4096, 14336), std=float(1 / np.sqrt(14336))).to(dev)
    gamma = (1 + 0.1 * inputs.normal(g, (4096,), dtype=torch.float32)).to(dev)
    res = inputs.normal(g, (M, 4096), dtype=torch.float32).to(dev)
    h = inputs.normal(g, (M, 4096)).to(dev)
    wg = inputs.normal(g, (14336, 4096), std=float(1 / np.sqrt(4096))).to(dev)
    wu = inputs.normal(g, (14336, 4096), std=float(1 / np.sqrt(4096))).to(dev)
    o0, xg0, s0 = [t.clone() for t in _lib.eagle_linear_rmsnorm_deferred(x, W, gamma, residual=res)]
    y0 = _lib.eagle_linear_swiglu(h, wg, wu).clone()
    o, xg, s = torch.empty_like(o0), torch.empty_like(xg0), torch.empty_like(s0)
    y = torch.empty_like(y0)
    for rep in range(200):
        _lib.eagle_linear_rmsnorm_deferred(x, W, gamma, residual=res, out=o, xg_out=xg, ssq_out=s)
        _lib.eagle_linear_swiglu(h, wg, wu, out=y)
        assert torch.equal(o, o0) and torch.equal(xg, xg0) and torch.equal(s, s0), f"deferred, call {rep}"
        assert torch.equal(y, y0), f"swiglu, call {rep}"
    print("200 calls bit-identical", flush=True)
