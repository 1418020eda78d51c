"""Pins of the backward oracle (``oracle/backward.py``) to things other than
itself: torch autograd in float64 on an independent dense-mask formulation
of the layer, central finite differences of the (separately pinned) forward
oracle, closed forms and sum rules. Each pin takes the oracle module pair
(forward, backward) so that planted mistakes can be run through them."""
import math

import numpy as np
import torch

SEL_EPS = 1e-3     # gates are drawn at least this far apart (no tie, no swap under FD)


def _inputs(seed, B=2, Hq=4, Hkv=2, n=19, d=8, zero_q=False, const_v=False):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, n, d))
    k = r.standard_normal((B, Hkv, n, d))
    v = r.standard_normal((B, Hkv, n, d))
    if zero_q:
        q[:] = 0.0
    if const_v:
        v[:] = r.standard_normal((B, Hkv, 1, d))
    # distinct, well separated gate logits
    gate = np.stack([r.permutation(n) * 0.25 + r.uniform(-0.05, 0.05, n) for _ in range(B)])
    gate = gate.astype(np.float32)
    do = r.standard_normal((B, Hq, n, d))
    return q, k, v, gate, do


def _dense_autograd(q, k, v, gate, do, window, rho, scale):
    """torch float64 autograd of the layer written with explicit n x n masks:
    band mask for the local branch, causal mask for the global branch, the
    top-k of the gate by torch.topk, GQA by repeating K/V heads."""
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    tg = torch.tensor(gate.astype(np.float64), requires_grad=True)
    kk = min(max(math.ceil(rho * n), 0), n)
    sel = torch.zeros((B, n), dtype=torch.float64)
    if kk:
        top = torch.topk(tg.detach(), kk, dim=1).indices
        sel.scatter_(1, top, 1.0)
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    band = (j <= i) & (j >= i - window + 1)
    causal = j <= i
    kr = tk.repeat_interleave(Hq // Hkv, dim=1)
    vr = tv.repeat_interleave(Hq // Hkv, dim=1)
    s = scale * (tq @ kr.transpose(-1, -2))
    pl = torch.softmax(s.masked_fill(~band, float("-inf")), dim=-1)
    pg = torch.softmax(s.masked_fill(~causal, float("-inf")), dim=-1)
    o = pl @ vr + (sel * torch.sigmoid(tg))[:, None, :, None] * (pg @ vr)
    (o * torch.tensor(do)).sum().backward()
    return (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), tg.grad.numpy(),
            o.detach().numpy())


def pin_bwd_autograd_dense(F, BW):
    cases = [
        dict(seed=1, B=2, Hq=4, Hkv=2, n=19, d=8, window=5, rho=0.3),
        dict(seed=2, B=1, Hq=6, Hkv=2, n=23, d=4, window=7, rho=0.5),   # group of 3
        dict(seed=3, B=2, Hq=2, Hkv=2, n=11, d=8, window=40, rho=0.2),  # W >= n
        dict(seed=4, B=1, Hq=2, Hkv=1, n=17, d=8, window=4, rho=0.0),
        dict(seed=5, B=1, Hq=2, Hkv=1, n=13, d=8, window=3, rho=1.0),
    ]
    for c in cases:
        w, rho = c.pop("window"), c.pop("rho")
        q, k, v, gate, do = _inputs(**c)
        scale = F.default_scale(q.shape[3])
        got = BW.backward(q, k, v, gate, do, w, rho)
        ref = _dense_autograd(q, k, v, gate, do, w, rho, scale)
        for name, a, b in zip(("dq", "dk", "dv", "dgate", "o"),
                              (got["dq"], got["dk"], got["dv"], got["dgate"], got["o"]), ref):
            assert np.allclose(a, b, rtol=1e-9, atol=1e-10), (name, c, np.abs(a - b).max())


def pin_bwd_finite_differences(F, BW):
    """Central differences of L = sum(o * do) through the forward oracle."""
    q, k, v, gate, do = _inputs(7, B=1, Hq=2, Hkv=1, n=9, d=4)
    window, rho = 3, 0.4
    got = BW.backward(q, k, v, gate, do, window, rho)

    def loss(q_, k_, v_, g_):
        return float((F.forward(q_, k_, v_, g_, window, rho)["o"] * do).sum())

    r = np.random.default_rng(8)
    eps = 1e-6
    for name, arr in (("dq", q), ("dk", k), ("dv", v)):
        for _ in range(6):
            at = tuple(int(r.integers(0, s)) for s in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[at] += eps
            minus[at] -= eps
            args = {"dq": (plus, k, v), "dk": (q, plus, v), "dv": (q, k, plus)}[name]
            argm = {"dq": (minus, k, v), "dk": (q, minus, v), "dv": (q, k, minus)}[name]
            fd = (loss(*args, gate) - loss(*argm, gate)) / (2 * eps)
            assert abs(fd - got[name][at]) <= 1e-6 * max(1.0, abs(fd)), (name, at, fd,
                                                                          got[name][at])
    # gate: float32 logits; a step small against SEL_EPS keeps the selection
    g64 = gate.astype(np.float64)
    for i in range(gate.shape[1]):
        h = 1e-4
        gp, gm = g64.copy(), g64.copy()
        gp[0, i] += h
        gm[0, i] -= h
        fd = (loss(q, k, v, gp) - loss(q, k, v, gm)) / (2 * h)
        assert abs(fd - got["dgate"][0, i]) <= 1e-6 * max(1.0, abs(fd)), (i, fd,
                                                                          got["dgate"][0, i])


def pin_bwd_constant_values(F, BW):
    """v_j = c: every score gradient vanishes (dq = dk = 0) and
    dgate_i = g(1-g) sum_h <do_{h,i}, c>."""
    q, k, v, gate, do = _inputs(9, B=2, Hq=4, Hkv=2, n=15, d=8, const_v=True)
    got = BW.backward(q, k, v, gate, do, 4, 0.4)
    assert np.abs(got["dq"]).max() < 1e-12 and np.abs(got["dk"]).max() < 1e-12
    g = 1.0 / (1.0 + np.exp(-gate.astype(np.float64)))
    mask = got["mask"]
    for b in range(2):
        for i in range(15):
            want = 0.0
            if mask[b, i]:
                want = g[b, i] * (1 - g[b, i]) * sum(float(do[b, h, i] @ v[b, h // 2, 0])
                                                     for h in range(4))
            assert abs(got["dgate"][b, i] - want) < 1e-12


def pin_bwd_sum_rules(F, BW):
    """Per (b, kv head): sum_j dk_j = 0 (each row's ds sums to zero) and
    sum_j dv_j = sum over the group's rows of do_i (1 + [i in S] g_i) (each
    row's probabilities sum to one)."""
    q, k, v, gate, do = _inputs(10, B=2, Hq=6, Hkv=2, n=21, d=8)
    got = BW.backward(q, k, v, gate, do, 6, 0.3)
    g = 1.0 / (1.0 + np.exp(-gate.astype(np.float64)))
    w = 1.0 + got["mask"] * g                      # [B, n]
    for b in range(2):
        for hk in range(2):
            assert np.abs(got["dk"][b, hk].sum(axis=0)).max() < 1e-12
            grp = do[b, 3 * hk:3 * hk + 3]         # [3, n, d]
            want = (grp * w[b][None, :, None]).sum(axis=(0, 1))
            assert np.allclose(got["dv"][b, hk].sum(axis=0), want, atol=1e-12)


def pin_bwd_window_one(F, BW):
    """W = 1, rho = 0: each row reads only itself with weight one, so dq = dk = 0,
    dv_j = sum over the group of do_j, dgate = 0."""
    q, k, v, gate, do = _inputs(11, B=1, Hq=4, Hkv=2, n=12, d=8)
    got = BW.backward(q, k, v, gate, do, 1, 0.0)
    assert np.abs(got["dq"]).max() < 1e-14 and np.abs(got["dk"]).max() < 1e-14
    assert np.abs(got["dgate"]).max() == 0.0
    for hk in range(2):
        assert np.allclose(got["dv"][0, hk], do[0, 2 * hk] + do[0, 2 * hk + 1], atol=1e-14)


def pin_bwd_zero_query(F, BW):
    """q = 0, rho = 0: uniform weights over L(i), so dk = 0 and
    dv_j = sum_{i = j}^{j+W-1} do_i / min(W, i+1)."""
    n, W = 14, 4
    q, k, v, gate, do = _inputs(12, B=1, Hq=1, Hkv=1, n=n, d=8, zero_q=True)
    got = BW.backward(q, k, v, gate, do, W, 0.0)
    assert np.abs(got["dk"]).max() < 1e-14
    for j in range(n):
        want = sum(do[0, 0, i] / min(W, i + 1) for i in range(j, min(n, j + W)))
        assert np.allclose(got["dv"][0, 0, j], want, atol=1e-14)


def pin_bwd_rows_match(F, BW):
    q, k, v, gate, do = _inputs(13, B=2, Hq=4, Hkv=2, n=25, d=8)
    full = BW.backward(q, k, v, gate, do, 5, 0.35)
    rows = [(0, 0, 0), (0, 3, 24), (1, 1, 7), (1, 2, 13), (0, 1, 5)]
    dq = BW.dq_rows(q, k, v, gate, do, 5, 0.35, rows)
    for t, (b, h, i) in enumerate(rows):
        assert np.allclose(dq[t], full["dq"][b, h, i], atol=1e-13)
    for b, hk, j_from in ((0, 0, 20), (1, 1, 0), (1, 0, 24)):
        dk, dv = BW.dkdv_tail(q, k, v, gate, do, 5, 0.35, b, hk, j_from)
        assert np.allclose(dk, full["dk"][b, hk, j_from:], atol=1e-13)
        assert np.allclose(dv, full["dv"][b, hk, j_from:], atol=1e-13)
    # any key range, from all rows at once or summed over a partition of them
    for b, hk, j_lo, j_hi in ((0, 0, 0, 4), (1, 1, 3, 11), (0, 1, 0, 25), (1, 0, 24, 25)):
        dk, dv = BW.dkdv_keys(q, k, v, gate, do, 5, 0.35, b, hk, j_lo, j_hi)
        assert np.allclose(dk, full["dk"][b, hk, j_lo:j_hi], atol=1e-13)
        assert np.allclose(dv, full["dv"][b, hk, j_lo:j_hi], atol=1e-13)
        parts = [BW.dkdv_keys(q, k, v, gate, do, 5, 0.35, b, hk, j_lo, j_hi, rows=r)
                 for r in (range(0, 9), range(9, 17), range(17, 25))]
        assert np.allclose(sum(p[0] for p in parts), dk, atol=1e-13)
        assert np.allclose(sum(p[1] for p in parts), dv, atol=1e-13)
    pos = [(b, i) for b in range(2) for i in range(25)]
    dg = BW.dgate_at(q, k, v, gate, do, 0.35, pos)
    assert np.allclose(dg, full["dgate"].reshape(-1), atol=1e-13)


def pin_forward_stats(F, BW):
    """lse equals torch.logsumexp of the masked scaled scores; q = 0 gives
    log |R|; the saved branch outputs are the forward oracle's."""
    q, k, v, gate, do = _inputs(14, B=2, Hq=4, Hkv=2, n=17, d=8)
    W, rho = 5, 0.3
    st = BW.forward_stats(q, k, v, gate, W, rho)
    scale = F.default_scale(8)
    s = scale * torch.tensor(q) @ torch.tensor(k).repeat_interleave(2, dim=1).transpose(-1, -2)
    i = torch.arange(17)[:, None]
    j = torch.arange(17)[None, :]
    band = (j <= i) & (j >= i - W + 1)
    lse_l = torch.logsumexp(s.masked_fill(~band, float("-inf")), dim=-1).numpy()
    lse_c = torch.logsumexp(s.masked_fill(~(j <= i), float("-inf")), dim=-1).numpy()
    assert np.allclose(st["lse_local"], lse_l, atol=1e-12)
    idx = st["idx"]
    for b in range(2):
        assert np.allclose(st["lse_global"][b], lse_c[b][:, idx[b]], atol=1e-12)
    fw = F.forward(q, k, v, gate, W, rho)
    for b in range(2):
        assert np.allclose(st["o_local_sel"][b], fw["o_local"][b][:, idx[b]], atol=1e-13)
    assert np.allclose(st["o_global"], fw["o_global"], atol=1e-13)
    q0, k0, v0, g0, _ = _inputs(15, B=1, Hq=1, Hkv=1, n=9, d=4, zero_q=True)
    st0 = BW.forward_stats(q0, k0, v0, g0, 3, 1.0)
    for i in range(9):
        assert abs(st0["lse_local"][0, 0, i] - math.log(min(3, i + 1))) < 1e-14
        assert abs(st0["lse_global"][0, 0, i] - math.log(i + 1)) < 1e-14


ALL_BWD_PINS = [
    pin_bwd_autograd_dense,
    pin_bwd_finite_differences,
    pin_bwd_constant_values,
    pin_bwd_sum_rules,
    pin_bwd_window_one,
    pin_bwd_zero_query,
    pin_bwd_rows_match,
    pin_forward_stats,
]
