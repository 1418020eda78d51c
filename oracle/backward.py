"""CPU fp64 oracle for the backward of token-level dynamic local-global attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP kernels, their headers
or their binding.

What is computed, and from which passage
-----------------------------------------
The gate is learned (LoGo abstract: a learned gate activates global attention
for some tokens) and the method is trained ("Learning When to Attend",
section "Empirical Validation and System Optimization": its speedup is quoted
for training throughput), but no page prints a backward pass. This module is
the chain rule of the forward in ``oracle/logo.py``:

    o_i = o_local_i + [i in S] g_i o_global_i,        g_i = sigmoid(gate_i)

Readings taken where the pages are silent:

* The selection S is a constant of the backward. Picking the top-k logits
  has no derivative and the pages say nothing of how a gradient would cross
  it (no straight-through rule is given), so the gate receives gradient only
  through sigmoid(gate_i) on selected tokens, and zero elsewhere.
* One gate per (batch, token) is shared by every query head, so its gradient
  sums over the heads. The key/value heads of grouped-query attention sum
  the gradients of their query heads.

For one attention row with query q, keys k_j and values v_j over its key
range R and upstream gradient e (the gradient of the loss with respect to
the row's output):

    s_j = scale <q, k_j>,  p = softmax(s),  o = sum_j p_j v_j
    dv_j += p_j e
    t_j   = <e, v_j>,   ds_j = p_j (t_j - sum_l p_l t_l)
    dq   += scale sum_j ds_j k_j
    dk_j += scale ds_j q

Local rows use e = do_i over L(i) = [max(0, i-W+1), i]; selected rows also
run a global row with e = g_i do_i over G(i) = [0, i]; and

    dgate_i = g_i (1 - g_i) sum_h <do_{h,i}, o_global_{h,i}>   for i in S.

Every function is the definition written out row by row in float64, with no
tiling and no reordering. The log-sum-exp of a row (``row_lse``) is what a
forward saves so that a backward can rebuild p without a second pass over
the row: lse = log sum_j exp(s_j), natural log of the scaled scores.

Parity: pinned in ``tests/test_oracle_backward.py`` against torch autograd
in float64 on an independent dense-mask formulation, central finite
differences, closed forms (constant values, a window of one, a zero query)
and sum rules that hold at any size.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

from . import logo as F

__all__ = ["row_grad", "row_lse", "backward", "dq_rows", "dgate_at", "forward_stats",
           "dkdv_tail", "dkdv_keys"]


def row_lse(qrow, keys, scale: float) -> float:
    """log sum_j exp(scale <q, k_j>) over one row's keys (natural log)."""
    s = scale * (np.asarray(keys, np.float64) @ np.asarray(qrow, np.float64))
    m = s.max()
    return float(m + math.log(np.exp(s - m).sum()))


def row_grad(qrow, keys, vals, e, scale: float):
    """Output and gradients of one softmax-attention row.

    Returns (o [d], dq [d], dkeys [len, d], dvals [len, d]) for upstream
    gradient e [d] (see the module docstring for the formulas)."""
    q = np.asarray(qrow, np.float64)
    K = np.asarray(keys, np.float64)
    V = np.asarray(vals, np.float64)
    e = np.asarray(e, np.float64)
    p = F.softmax_weights(scale * (K @ q))
    o = p @ V
    dvals = np.outer(p, e)
    t = V @ e
    ds = p * (t - p @ t)
    dq = scale * (ds @ K)
    dkeys = scale * np.outer(ds, q)
    return o, dq, dkeys, dvals


def backward(q, k, v, gate, do, window: int, rho: float,
             scale: Optional[float] = None) -> dict:
    """Gradients of the whole layer for upstream gradient do [B, Hq, n, d].

    Returns dq [B,Hq,n,d], dk, dv [B,Hkv,n,d], dgate [B,n] (float64), the
    selection (mask, idx, rank) and the forward output o."""
    F._check_shapes(q, k, v)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    scale = F.default_scale(d) if scale is None else scale
    do = np.asarray(do, np.float64)
    if do.shape != q.shape:
        raise ValueError("do must have q's shape")
    mask, idx, rank = F.select_queries(gate, rho)
    g = F.sigmoid(gate)
    dq = np.zeros((B, Hq, n, d))
    dk = np.zeros((B, Hkv, n, d))
    dv = np.zeros((B, Hkv, n, d))
    dgate = np.zeros((B, n))
    o = np.zeros((B, Hq, n, d))
    for b in range(B):
        for h in range(Hq):
            hk = F._kv_head(h, Hq, Hkv)
            for i in range(n):
                lo = max(0, i - window + 1)
                ol, gq, gk, gv = row_grad(q[b, h, i], k[b, hk, lo:i + 1], v[b, hk, lo:i + 1],
                                          do[b, h, i], scale)
                dq[b, h, i] += gq
                dk[b, hk, lo:i + 1] += gk
                dv[b, hk, lo:i + 1] += gv
                o[b, h, i] = ol
                if mask[b, i]:
                    og, gq, gk, gv = row_grad(q[b, h, i], k[b, hk, :i + 1], v[b, hk, :i + 1],
                                              g[b, i] * do[b, h, i], scale)
                    dq[b, h, i] += gq
                    dk[b, hk, :i + 1] += gk
                    dv[b, hk, :i + 1] += gv
                    o[b, h, i] += g[b, i] * og
                    dgate[b, i] += g[b, i] * (1.0 - g[b, i]) * float(do[b, h, i] @ og)
    return {"dq": dq, "dk": dk, "dv": dv, "dgate": dgate, "o": o,
            "mask": mask, "idx": idx, "rank": rank}


def forward_stats(q, k, v, gate, window: int, rho: float,
                  scale: Optional[float] = None) -> dict:
    """What a training forward saves: lse_local [B,Hq,n], lse_global [B,Hq,k]
    (idx order), and the two branch outputs of the selected rows,
    o_local_sel and o_global [B,Hq,k,d]."""
    F._check_shapes(q, k, v)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    scale = F.default_scale(d) if scale is None else scale
    mask, idx, rank = F.select_queries(gate, rho)
    kk = idx.shape[1]
    lse_l = np.zeros((B, Hq, n))
    lse_g = np.zeros((B, Hq, kk))
    o_ls = np.zeros((B, Hq, kk, d))
    o_g = np.zeros((B, Hq, kk, d))
    for b in range(B):
        for h in range(Hq):
            hk = F._kv_head(h, Hq, Hkv)
            for i in range(n):
                lse_l[b, h, i] = row_lse(q[b, h, i], k[b, hk, max(0, i - window + 1):i + 1],
                                         scale)
            for r in range(kk):
                i = int(idx[b, r])
                lse_g[b, h, r] = row_lse(q[b, h, i], k[b, hk, :i + 1], scale)
                o_ls[b, h, r] = F.local_row(q, k, v, b, h, i, window, scale)
                o_g[b, h, r] = F.global_row(q, k, v, b, h, i, scale)
    return {"lse_local": lse_l, "lse_global": lse_g, "o_local_sel": o_ls, "o_global": o_g,
            "mask": mask, "idx": idx, "rank": rank}


def dq_rows(q, k, v, gate, do, window: int, rho: float, rows: Iterable[Sequence[int]],
            scale: Optional[float] = None) -> np.ndarray:
    """dq on chosen (b, h, i) rows only, for inputs too large to do whole: a
    row's dq depends only on its own attention rows. [len(rows), d]."""
    F._check_shapes(q, k, v)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    scale = F.default_scale(d) if scale is None else scale
    mask, _, _ = F.select_queries(gate, rho)
    g = F.sigmoid(gate)
    rows = [tuple(int(x) for x in r) for r in rows]
    out = np.zeros((len(rows), d))
    for t, (b, h, i) in enumerate(rows):
        hk = F._kv_head(h, Hq, Hkv)
        lo = max(0, i - window + 1)
        out[t] = row_grad(q[b, h, i], k[b, hk, lo:i + 1], v[b, hk, lo:i + 1], do[b, h, i],
                          scale)[1]
        if mask[b, i]:
            out[t] += row_grad(q[b, h, i], k[b, hk, :i + 1], v[b, hk, :i + 1],
                               g[b, i] * np.asarray(do[b, h, i], np.float64), scale)[1]
    return out


def dgate_at(q, k, v, gate, do, rho: float, positions: Iterable[Sequence[int]],
             scale: Optional[float] = None) -> np.ndarray:
    """dgate on chosen (b, i) positions only. [len(positions)]."""
    F._check_shapes(q, k, v)
    B, Hq, n, d = q.shape
    scale = F.default_scale(d) if scale is None else scale
    mask, _, _ = F.select_queries(gate, rho)
    g = F.sigmoid(gate)
    positions = [tuple(int(x) for x in r) for r in positions]
    out = np.zeros(len(positions))
    for t, (b, i) in enumerate(positions):
        if not mask[b, i]:
            continue
        acc = 0.0
        for h in range(Hq):
            og = F.global_row(q, k, v, b, h, i, scale)
            acc += float(np.asarray(do[b, h, i], np.float64) @ og)
        out[t] = g[b, i] * (1.0 - g[b, i]) * acc
    return out


def dkdv_tail(q, k, v, gate, do, window: int, rho: float, b: int, hk: int, j_from: int,
              scale: Optional[float] = None):
    """dk, dv [n - j_from, d] of keys j_from..n-1 of (b, kv head hk), for
    inputs too large to do whole: only rows at or after j_from read those
    keys, so the rows i >= j_from of the kv head's query heads, both
    branches, give their gradients exactly."""
    F._check_shapes(q, k, v)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    scale = F.default_scale(d) if scale is None else scale
    mask, _, _ = F.select_queries(gate, rho)
    g = F.sigmoid(gate)
    G = Hq // Hkv
    dk = np.zeros((n - j_from, d))
    dv = np.zeros((n - j_from, d))
    for h in range(hk * G, hk * G + G):
        for i in range(j_from, n):
            e = np.asarray(do[b, h, i], np.float64)
            lo = max(0, i - window + 1)
            _, _, gk, gv = row_grad(q[b, h, i], k[b, hk, lo:i + 1], v[b, hk, lo:i + 1], e, scale)
            a = max(lo, j_from)
            dk[a - j_from:i + 1 - j_from] += gk[a - lo:]
            dv[a - j_from:i + 1 - j_from] += gv[a - lo:]
            if mask[b, i]:
                _, _, gk, gv = row_grad(q[b, h, i], k[b, hk, :i + 1], v[b, hk, :i + 1],
                                        g[b, i] * e, scale)
                dk[:i + 1 - j_from] += gk[j_from:]
                dv[:i + 1 - j_from] += gv[j_from:]
    return dk, dv


def dkdv_keys(q, k, v, gate, do, window: int, rho: float, b: int, hk: int, j_lo: int,
              j_hi: int, rows: Optional[Iterable[int]] = None,
              scale: Optional[float] = None):
    """dk, dv [j_hi - j_lo, d] of keys j_lo..j_hi-1 of (b, kv head hk): the
    sum over the kv head's query heads and over query positions ``rows``
    (default: every position) of each row's gradient on those keys, both
    branches. A row's local branch reads L(i), its global branch (selected
    rows only) [0, i]; rows that read none of the keys add nothing. Summing
    the results over a partition of the positions gives the keys' full
    gradients, so the earliest keys, which every selected row reads, can be
    computed in parts."""
    F._check_shapes(q, k, v)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    scale = F.default_scale(d) if scale is None else scale
    mask, _, _ = F.select_queries(gate, rho)
    g = F.sigmoid(gate)
    G = Hq // Hkv
    dk = np.zeros((j_hi - j_lo, d))
    dv = np.zeros((j_hi - j_lo, d))
    positions = range(n) if rows is None else [int(i) for i in rows]
    for i in positions:
        if i < j_lo:
            continue                       # a row reads no key after it
        lo = max(0, i - window + 1)
        local_hits = lo < j_hi              # the window reaches the range
        if not local_hits and not mask[b, i]:
            continue
        for h in range(hk * G, hk * G + G):
            e = np.asarray(do[b, h, i], np.float64)
            if local_hits:
                _, _, gk, gv = row_grad(q[b, h, i], k[b, hk, lo:i + 1], v[b, hk, lo:i + 1], e,
                                        scale)
                a, z = max(lo, j_lo), min(i + 1, j_hi)
                dk[a - j_lo:z - j_lo] += gk[a - lo:z - lo]
                dv[a - j_lo:z - j_lo] += gv[a - lo:z - lo]
            if mask[b, i]:
                _, _, gk, gv = row_grad(q[b, h, i], k[b, hk, :i + 1], v[b, hk, :i + 1],
                                        g[b, i] * e, scale)
                z = min(i + 1, j_hi)
                dk[:z - j_lo] += gk[j_lo:z]
                dv[:z - j_lo] += gv[j_lo:z]
    return dk, dv
