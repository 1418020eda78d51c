"""Pins for the CPU oracle: checks against facts fixed outside the oracle.

Each pin takes the oracle module ``O`` (``oracle.logo``) and raises
AssertionError when the oracle disagrees with a closed form, a library
routine computing a special case, a brute-force count, an invariant, or a
hand-derived fixture under ``tests/golden/``. The same pins run against
copies of the oracle with planted mistakes (``test_oracle_mutants.py``) to
show that a plausible mistake anywhere in it is caught.

Definitions pinned (pages: LoGo abstract; "Local-global attention",
attention-mask sketch and Gemma 2 variant; "Learning When to Attend",
"The Architecture of Conditional Attention"):
  L(i) = [max(0, i-W+1), i]   (last W keys, causal)
  G(i) = [0, i]               (full causal context)
  S    = ceil(rho*n) largest gate logits per sequence, ties to lower position
  o    = o_local + sigmoid(gate) * o_global on S, o_local elsewhere
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, B=1, Hq=2, Hkv=1, n=24, d=8):
    r = _rng(seed)
    q = r.standard_normal((B, Hq, n, d))
    k = r.standard_normal((B, Hkv, n, d))
    v = r.standard_normal((B, Hkv, n, d))
    return q, k, v


def _sdpa(q, k, v, scale, mask=None, causal=False):
    """torch CPU scaled_dot_product_attention in float64 (library routine)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    kt = torch.from_numpy(np.ascontiguousarray(k)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(np.ascontiguousarray(v)).repeat_interleave(G, dim=1)
    qt = torch.from_numpy(np.ascontiguousarray(q))
    m = None if mask is None else torch.from_numpy(mask)
    with torch.no_grad():
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=m, is_causal=causal, scale=scale)
    return o.numpy()


# --------------------------------------------------------------------------
# target count
# --------------------------------------------------------------------------

def pin_target_count(O):
    # closed forms: ceil(rho*n) on the workload sizes (rho*n exact there)
    cases = {(0.25, 256): 64, (0.2, 4096): 820, (0.2, 32768): 6554,
             (0.2, 131072): 26215, (0.0, 65536): 0, (0.05, 65536): 3277,
             (0.2, 65536): 13108, (0.5, 65536): 32768, (1.0, 65536): 65536,
             (0.1, 10): 1, (0.11, 10): 2, (1e-9, 7): 1, (1.0, 0): 0}
    for (rho, n), k in cases.items():
        assert O.target_count(rho, n) == k, (rho, n, O.target_count(rho, n), k)
    assert O.target_count(1.5, 10) == 10
    assert O.target_count(-0.5, 10) == 0


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def _brute_selected(g, k):
    """i is selected iff fewer than k tokens beat it; a token j beats i when
    its logit is larger, or equal with a lower position. NaN loses to every
    number; two NaNs are equal. -0.0 == +0.0."""
    n = len(g)

    def beats(j, i):
        a, b = g[j], g[i]
        an, bn = math.isnan(a), math.isnan(b)
        if an and bn:
            return j < i
        if an:
            return False
        if bn:
            return True
        return a > b or (a == b and j < i)

    return np.array([sum(beats(j, i) for j in range(n) if j != i) < k for i in range(n)])


def pin_selection_bruteforce(O):
    r = _rng(11)
    for trial in range(40):
        n = int(r.integers(1, 40))
        B = int(r.integers(1, 3))
        # small integer logits force many exact ties; sprinkle specials
        g = r.integers(-3, 4, size=(B, n)).astype(np.float32)
        specials = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0], np.float32)
        sel = r.random((B, n)) < 0.25
        g[sel] = specials[r.integers(0, len(specials), size=int(sel.sum()))]
        rho = float(r.choice([0.0, 0.1, 0.25, 0.33, 0.5, 0.9, 1.0, r.random()]))
        mask, idx, rank = O.select_queries(g, rho)
        k = O.target_count(rho, n)
        assert idx.shape == (B, k)
        for b in range(B):
            want = _brute_selected([float(x) for x in g[b]], k)
            assert np.array_equal(mask[b].astype(bool), want), (g[b], rho)
            assert int(mask[b].sum()) == k
            assert np.array_equal(idx[b], np.flatnonzero(want))
            assert np.all(np.diff(idx[b]) > 0)
            rr = np.full(n, -1)
            rr[idx[b]] = np.arange(k)
            assert np.array_equal(rank[b], rr)


def pin_selection_invariants(O):
    r = _rng(12)
    B, n = 2, 300
    g = r.standard_normal((B, n)).astype(np.float32)
    rhos = [0.0, 0.05, 0.2, 0.5, 0.77, 1.0]
    prev = None
    for rho in rhos:
        mask, _, _ = O.select_queries(g, rho)
        # threshold separation: every selected logit >= every unselected one
        for b in range(B):
            s = g[b][mask[b] == 1]
            u = g[b][mask[b] == 0]
            if len(s) and len(u):
                assert s.min() >= u.max()
        # nesting: a larger budget keeps every token a smaller one chose
        if prev is not None:
            assert np.all(mask >= prev)
        prev = mask
    # strictly increasing maps of the logits leave the choice unchanged
    m0, i0, _ = O.select_queries(g, 0.3)
    m1, i1, _ = O.select_queries(g * np.float32(4.0), 0.3)   # exact in float32
    assert np.array_equal(m0, m1) and np.array_equal(i0, i1)
    gi = r.integers(-4, 5, size=(B, n)).astype(np.float32)      # many ties
    a = O.select_queries(gi, 0.3)
    b = O.select_queries(gi + np.float32(1000.0), 0.3)          # exact shift
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    # all logits equal -> the first k positions
    mask, idx, _ = O.select_queries(np.zeros((1, 50), np.float32), 0.3)
    assert np.array_equal(idx[0], np.arange(15))


def pin_selection_golden(O):
    with open(os.path.join(GOLDEN, "selection_ties.json")) as f:
        fx = json.load(f)
    g = np.array([[float(x) for x in fx["gate"]]], dtype=np.float32)
    for case in fx["cases"]:
        mask, idx, rank = O.select_queries(g, case["rho"])
        assert idx[0].tolist() == case["idx"], (case, idx)
        assert rank[0].tolist() == case["rank"], (case, rank)


# --------------------------------------------------------------------------
# local branch
# --------------------------------------------------------------------------

def pin_local_zero_query(O):
    """q = 0 gives uniform weights over L(i); with v_j[0] = j the output is the
    mean position of the window, (max(0, i-W+1) + i) / 2: pins the window's
    width and its causal end."""
    for n, W in ((20, 1), (20, 4), (20, 7), (9, 30)):
        B, H, d = 1, 1, 4
        q = np.zeros((B, H, n, d))
        k = _rng(5).standard_normal((B, H, n, d))
        v = _rng(6).standard_normal((B, H, n, d))
        v[0, 0, :, 0] = np.arange(n)
        o = O.local_attention(q, k, v, W, 0.7)
        want = np.array([(max(0, i - W + 1) + i) / 2 for i in range(n)])
        assert np.allclose(o[0, 0, :, 0], want, atol=1e-12, rtol=0), (n, W)


def pin_local_special_cases(O):
    q, k, v = _qkv(21, B=2, Hq=4, Hkv=2, n=17, d=8)
    # W = 1: each query reads only itself
    o = O.local_attention(q, k, v, 1, 0.4)
    assert np.allclose(o, np.repeat(v, 2, axis=1), atol=1e-12)
    # constant values: any weights give the constant
    vc = np.full_like(v, 3.25)
    o = O.local_attention(q, k, vc, 5, 0.4)
    assert np.allclose(o, 3.25, atol=1e-12)


def pin_local_dense_when_window_covers(O):
    """W >= n: the local branch is dense causal attention (torch SDPA)."""
    q, k, v = _qkv(22, B=2, Hq=4, Hkv=2, n=19, d=8)
    for W in (19, 40):
        o = O.local_attention(q, k, v, W, 0.3)
        ref = _sdpa(q, k, v, 0.3, causal=True)
        assert np.allclose(o, ref, atol=1e-12, rtol=0)


def pin_local_band_mask(O):
    """Any W: equals SDPA with an explicit boolean band mask, built both as
    (i-W < j <= i) and, as the Gemma 2 note observes, as a two-sided bound
    |i-j| < W intersected with the causal mask."""
    q, k, v = _qkv(23, B=1, Hq=3, Hkv=3, n=29, d=16)
    n = q.shape[2]
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    for W in (1, 2, 5, 13, 28):
        one_sided = (j <= i) & (j > i - W)
        two_sided = (np.abs(i - j) < W) & (j <= i)
        assert np.array_equal(one_sided, two_sided)
        ref = _sdpa(q, k, v, 0.25, mask=one_sided)
        o = O.local_attention(q, k, v, W, 0.25)
        assert np.allclose(o, ref, atol=1e-12, rtol=0), W


def pin_local_bruteforce_matrix(O):
    """Tiny inputs: the full n x n score matrix, masked entries set to -inf,
    row-wise softmax by explicit exponentials; each weight row sums to 1."""
    q, k, v = _qkv(24, B=1, Hq=1, Hkv=1, n=12, d=3)
    n, W, sc = 12, 4, 0.9
    S = sc * (q[0, 0] @ k[0, 0].T)
    keep = np.array([[(i - W < j <= i) for j in range(n)] for i in range(n)])
    S = np.where(keep, S, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P = P / P.sum(axis=1, keepdims=True)
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(P[~keep] == 0)
    o = O.local_attention(q, k, v, W, sc)
    assert np.allclose(o[0, 0], P @ v[0, 0], atol=1e-12)
    # the oracle's own weights on one row sum to one too
    w = O.softmax_weights(S[7][keep[7]])
    assert abs(w.sum() - 1.0) < 1e-12


def pin_pow2_golden(O):
    with open(os.path.join(GOLDEN, "pow2_window.json")) as f:
        fx = json.load(f)
    n, W = fx["n"], fx["window"]
    q = np.ones((1, 1, n, 1))
    k = (np.arange(n) * math.log(2.0)).reshape(1, 1, n, 1)
    v = np.arange(n, dtype=np.float64).reshape(1, 1, n, 1)
    want_local = np.array([float(Fraction(x)) for x in fx["o_local"]])
    want_global = np.array([float(Fraction(x)) for x in fx["o_global"]])
    o = O.local_attention(q, k, v, W, 1.0)
    assert np.allclose(o[0, 0, :, 0], want_local, atol=1e-12, rtol=0)
    idx = np.arange(n, dtype=np.int32).reshape(1, n)
    og = O.global_attention(q, k, v, idx, 1.0)
    assert np.allclose(og[0, 0, :, 0], want_global, atol=1e-12, rtol=0)
    gate = np.array([[math.log(float(Fraction(x))) if x not in ("-inf",) else -np.inf
                      for x in fx["gate_exp"]]], dtype=np.float64)
    res = O.forward(q, k, v, gate.astype(np.float32), W, fx["rho"], 1.0)
    want_o = np.array([float(Fraction(x)) for x in fx["o"]])
    assert res["idx"][0].tolist() == fx["idx"]
    assert np.allclose(res["o"][0, 0, :, 0], want_o, atol=1e-6, rtol=0)


# --------------------------------------------------------------------------
# global branch
# --------------------------------------------------------------------------

def pin_global_equals_dense_causal(O):
    q, k, v = _qkv(31, B=2, Hq=4, Hkv=2, n=21, d=8)
    ref = _sdpa(q, k, v, 0.35, causal=True)
    idx = np.array([[0, 3, 4, 20], [1, 2, 11, 19]], dtype=np.int32)
    og = O.global_attention(q, k, v, idx, 0.35)
    for b in range(2):
        for r, i in enumerate(idx[b]):
            assert np.allclose(og[b, :, r], ref[b, :, i], atol=1e-12, rtol=0)


def pin_global_long_rows(O):
    """Rows far from the start read their whole causal prefix (dense causal
    attention by torch SDPA on a 300-token sequence)."""
    q, k, v = _qkv(32, B=1, Hq=2, Hkv=1, n=300, d=4)
    ref = _sdpa(q, k, v, 0.5, causal=True)
    idx = np.array([[0, 63, 64, 150, 299]], dtype=np.int32)
    og = O.global_attention(q, k, v, idx, 0.5)
    for r, i in enumerate(idx[0]):
        assert np.allclose(og[0, :, r], ref[0, :, i], atol=1e-12, rtol=0)


def pin_global_zero_query(O):
    n = 15
    q = np.zeros((1, 1, n, 2))
    k = _rng(7).standard_normal((1, 1, n, 2))
    v = np.zeros((1, 1, n, 2))
    v[0, 0, :, 0] = np.arange(n)
    idx = np.array([[0, 5, 14]], dtype=np.int32)
    og = O.global_attention(q, k, v, idx, 1.0)
    assert np.allclose(og[0, 0, :, 0], [0.0, 2.5, 7.0], atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------

def pin_forward_rho_extremes(O):
    q, k, v = _qkv(41, B=2, Hq=4, Hkv=2, n=23, d=8)
    gate = _rng(42).standard_normal((2, 23)).astype(np.float32)
    W, sc = 6, 0.3
    i = np.arange(23)[:, None]
    j = np.arange(23)[None, :]
    band = _sdpa(q, k, v, sc, mask=(j <= i) & (j > i - W))
    dense = _sdpa(q, k, v, sc, causal=True)
    # rho = 0: pure sliding-window attention
    r0 = O.forward(q, k, v, gate, W, 0.0, sc)
    assert r0["idx"].shape == (2, 0)
    assert np.allclose(r0["o"], band, atol=1e-12, rtol=0)
    # rho = 1: every row adds sigmoid(gate) times dense causal attention
    r1 = O.forward(q, k, v, gate, W, 1.0, sc)
    sg = 1.0 / (1.0 + np.exp(-gate.astype(np.float64)))
    want = band + sg[:, None, :, None] * dense
    assert np.allclose(r1["o"], want, atol=1e-12, rtol=0)


def pin_combine_constant_values(O):
    """v = c: o_local = o_global = c, so o = c (1 + sigmoid(gate)) on S and c
    elsewhere."""
    q, k, _ = _qkv(43, B=2, Hq=2, Hkv=1, n=31, d=8)
    c = 1.75
    v = np.full(k.shape, c)
    gate = _rng(44).standard_normal((2, 31)).astype(np.float32)
    res = O.forward(q, k, v, gate, 4, 0.3, 0.5)
    sg = 1.0 / (1.0 + np.exp(-gate.astype(np.float64)))
    want = np.where(res["mask"].astype(bool), c * (1.0 + sg), c)
    assert np.allclose(res["o"], want[:, None, :, None], atol=1e-12, rtol=0)
    assert int(res["mask"].sum()) == 2 * math.ceil(0.3 * 31)


def pin_gqa_equals_repeated_heads(O):
    q, k, v = _qkv(45, B=1, Hq=6, Hkv=2, n=13, d=4)
    gate = _rng(46).standard_normal((1, 13)).astype(np.float32)
    a = O.forward(q, k, v, gate, 3, 0.4, 0.5)
    b = O.forward(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), gate, 3, 0.4, 0.5)
    assert np.allclose(a["o"], b["o"], atol=1e-14, rtol=0)
    # head h reads key/value head h // 3: changing kv head 1 moves heads 3..5 only
    k2 = k.copy()
    k2[:, 1] += _rng(51).standard_normal(k2[:, 1].shape)
    c = O.forward(q, k2, v, gate, 3, 0.4, 0.5)
    assert np.allclose(a["o"][:, :3], c["o"][:, :3], atol=1e-14)
    assert not np.allclose(a["o"][:, 3:], c["o"][:, 3:])


def pin_batch_permutation(O):
    q, k, v = _qkv(47, B=3, Hq=2, Hkv=2, n=11, d=4)
    gate = _rng(48).standard_normal((3, 11)).astype(np.float32)
    a = O.forward(q, k, v, gate, 3, 0.5, 0.5)
    p = [2, 0, 1]
    b = O.forward(q[p], k[p], v[p], gate[p], 3, 0.5, 0.5)
    assert np.allclose(a["o"][p], b["o"], atol=1e-14)
    assert np.array_equal(a["idx"][p], b["idx"])


def pin_forward_rows_match(O):
    q, k, v = _qkv(49, B=2, Hq=4, Hkv=2, n=37, d=8)
    gate = _rng(50).standard_normal((2, 37)).astype(np.float32)
    full = O.forward(q, k, v, gate, 9, 0.3, 0.4)
    rows = [(0, 0, 0), (1, 3, 36), (0, 2, 17), (1, 1, 8)] + \
        [(b, 1, int(i)) for b in range(2) for i in full["idx"][b]]
    part = O.forward_rows(q, k, v, gate, 9, 0.3, rows, 0.4)
    for t, (b, h, i) in enumerate(rows):
        assert np.allclose(part["o_rows"][t], full["o"][b, h, i], atol=1e-14)


ALL_PINS = [
    pin_target_count,
    pin_selection_bruteforce,
    pin_selection_invariants,
    pin_selection_golden,
    pin_local_zero_query,
    pin_local_special_cases,
    pin_local_dense_when_window_covers,
    pin_local_band_mask,
    pin_local_bruteforce_matrix,
    pin_pow2_golden,
    pin_global_equals_dense_causal,
    pin_global_long_rows,
    pin_global_zero_query,
    pin_forward_rho_extremes,
    pin_combine_constant_values,
    pin_gqa_equals_repeated_heads,
    pin_batch_permutation,
    pin_forward_rows_match,
]
