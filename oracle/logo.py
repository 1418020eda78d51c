"""CPU fp64 oracle for token-level dynamic local-global attention (forward).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP kernels, their
headers or their binding; the only module both sides use is the seeded input
generator in ``workloads``, which holds no attention arithmetic.

What is computed, and from which passage
-----------------------------------------
Pages: "LoGo: Token-Level Dynamic Local-Global Attention" (abstract),
"Local-global attention" (sections "Variants / Alternating sliding-window and
global layers (Gemma 2)" and "Implementation sketch", the attention-mask
pseudocode), "Learning When to Attend" (section "The Architecture of
Conditional Attention").

* Every query attends locally over a restricted recent window (LoGo
  abstract; L2A "Architecture": local attention over a fixed recent window).
  The mask is causal AND within-window (local-global attention page, the
  attention-mask sketch). Reading taken: the window holds the query's last W
  keys, itself included: L(i) = [max(0, i-W+1), i].
* A gate score per token and a budget controller that holds a target global
  ratio pick the tokens that also get global attention (LoGo abstract; L2A
  "Architecture": one binary decision per token). Reading taken: exactly
  k = ceil(rho * n) tokens per sequence, the k largest gate logits, ties to
  the lower position, one gate per (batch, token) shared by all heads.
* The selected tokens get exact attention over the full causal context
  G(i) = [0, i] (L2A "Architecture": exact attention over the full context
  for a sparse subset of query tokens only; Gemma 2 variant: a query never
  reads a later position).
* Combine: o_i = o_local_i + sigmoid(gate_i) * o_global_i for selected i,
  o_local_i otherwise (the pages print no combine rule; this one is the
  problem statement's).

Every function below is the definition written out row by row, in float64,
with no tiling, no online softmax and no reordering. Each softmax is the
textbook one with the row maximum subtracted before exponentiation (an exact
identity that only avoids overflow).

Parity: k, the selection, both branches and the combine are pinned by
closed forms, library routines and brute force in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "target_count",
    "select_queries",
    "softmax_weights",
    "local_row",
    "global_row",
    "local_attention",
    "global_attention",
    "combine",
    "forward",
    "forward_rows",
    "default_scale",
]


def default_scale(d: int) -> float:
    """Softmax scale 1/sqrt(d) (the pages leave the scale unstated; the
    standard scaled-dot-product one is taken)."""
    return 1.0 / math.sqrt(d)


def target_count(rho: float, n: int) -> int:
    """Size of the selected set per sequence: ceil(rho * n), clamped to [0, n].

    LoGo abstract: the budget controller keeps a target global ratio; the
    ratio is turned into a count by rounding up, in float64."""
    if not (rho == rho) or n < 0:
        raise ValueError("rho must be a number and n >= 0")
    k = math.ceil(float(rho) * float(n))
    return int(min(max(k, 0), n))


def select_queries(gate: np.ndarray, rho: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per sequence, the k = ceil(rho*n) tokens with the largest gate logits.

    Ties go to the lower position; -0.0 equals +0.0; a NaN logit ranks below
    every number (-inf included). Returns
      mask [B, n] uint8  (1 = selected),
      idx  [B, k] int32  (selected positions, ascending),
      rank [B, n] int32  (position of the token in idx, -1 if not selected).
    A stable sort of the negated logits puts larger logits first and keeps
    equal logits in position order; numpy sorts NaN last."""
    gate = np.asarray(gate, dtype=np.float32)
    if gate.ndim != 2:
        raise ValueError("gate must be [B, n]")
    B, n = gate.shape
    k = target_count(rho, n)
    mask = np.zeros((B, n), dtype=np.uint8)
    idx = np.zeros((B, k), dtype=np.int32)
    rank = np.full((B, n), -1, dtype=np.int32)
    for b in range(B):
        order = np.argsort(-gate[b].astype(np.float64), kind="stable")
        chosen = np.sort(order[:k])
        mask[b, chosen] = 1
        idx[b] = chosen
        rank[b, chosen] = np.arange(k, dtype=np.int32)
    return mask, idx, rank


def softmax_weights(s: np.ndarray) -> np.ndarray:
    """Textbook softmax of one score row (float64)."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max())
    return e / e.sum()


def _attend(qrow: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float) -> np.ndarray:
    s = scale * (keys.astype(np.float64) @ qrow.astype(np.float64))
    p = softmax_weights(s)
    return p @ vals.astype(np.float64)


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    # grouped-query heads: contiguous groups of Hq/Hkv query heads share one
    # key/value head
    return h // (Hq // Hkv)


def local_row(q, k, v, b: int, h: int, i: int, window: int, scale: float) -> np.ndarray:
    """o_local for one query: softmax over its last `window` keys (itself
    included), times the values."""
    Hq, Hkv = q.shape[1], k.shape[1]
    hk = _kv_head(h, Hq, Hkv)
    lo = max(0, i - window + 1)
    return _attend(q[b, h, i], k[b, hk, lo:i + 1], v[b, hk, lo:i + 1], scale)


def global_row(q, k, v, b: int, h: int, i: int, scale: float) -> np.ndarray:
    """o_global for one query: softmax over every key at or before it."""
    Hq, Hkv = q.shape[1], k.shape[1]
    hk = _kv_head(h, Hq, Hkv)
    return _attend(q[b, h, i], k[b, hk, :i + 1], v[b, hk, :i + 1], scale)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, n, d]")
    B, Hq, n, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != n or k.shape[3] != d:
        raise ValueError("k, v must be [B, Hkv, n, d] matching q")
    if Hq % k.shape[1] != 0:
        raise ValueError("Hq must be a multiple of Hkv")


def local_attention(q, k, v, window: int, scale: Optional[float] = None) -> np.ndarray:
    """o_local [B, Hq, n, d] float64 for every query."""
    _check_shapes(q, k, v)
    if window < 1:
        raise ValueError("window must be >= 1")
    B, Hq, n, d = q.shape
    scale = default_scale(d) if scale is None else scale
    o = np.empty((B, Hq, n, d), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            for i in range(n):
                o[b, h, i] = local_row(q, k, v, b, h, i, window, scale)
    return o


def global_attention(q, k, v, idx: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """o_global [B, Hq, k, d] float64 for the selected rows, in idx order."""
    _check_shapes(q, k, v)
    B, Hq, n, d = q.shape
    scale = default_scale(d) if scale is None else scale
    kk = idx.shape[1]
    o = np.empty((B, Hq, kk, d), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            for r in range(kk):
                o[b, h, r] = global_row(q, k, v, b, h, int(idx[b, r]), scale)
    return o


def sigmoid(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def combine(o_local: np.ndarray, o_global: np.ndarray, rank: np.ndarray,
            gate: np.ndarray) -> np.ndarray:
    """o = o_local + sigmoid(gate) * o_global on selected rows, o_local elsewhere.

    o_local [B,Hq,n,d], o_global [B,Hq,k,d] (idx order), rank [B,n], gate [B,n]."""
    o = np.array(o_local, dtype=np.float64, copy=True)
    B, Hq, n, d = o.shape
    g = sigmoid(gate)
    for b in range(B):
        for i in range(n):
            r = int(rank[b, i])
            if r >= 0:
                o[b, :, i, :] += g[b, i] * np.asarray(o_global[b, :, r, :], dtype=np.float64)
    return o


def forward(q, k, v, gate, window: int, rho: float, scale: Optional[float] = None) -> dict:
    """The whole layer: selection, local branch, global branch, combine."""
    _check_shapes(q, k, v)
    d = q.shape[3]
    scale = default_scale(d) if scale is None else scale
    mask, idx, rank = select_queries(gate, rho)
    o_local = local_attention(q, k, v, window, scale)
    o_global = global_attention(q, k, v, idx, scale)
    o = combine(o_local, o_global, rank, gate)
    return {"o": o, "mask": mask, "idx": idx, "rank": rank,
            "o_local": o_local, "o_global": o_global}


def forward_rows(q, k, v, gate, window: int, rho: float,
                 rows: Iterable[Sequence[int]], scale: Optional[float] = None,
                 selection: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]] = None) -> dict:
    """The layer's output on chosen rows only, for inputs too large to do whole.

    Rows are independent given the keys and values, so each (b, h, i) in
    `rows` is computed exactly as in `forward`. The selection is computed for
    the whole sequence, or passed in as `selection` (the (mask, idx, rank)
    that ``select_queries(gate, rho)`` returned, when many row sets share
    it). Returns the selection and an array o_rows [len(rows), d] float64 in
    the order given."""
    _check_shapes(q, k, v)
    d = q.shape[3]
    scale = default_scale(d) if scale is None else scale
    mask, idx, rank = select_queries(gate, rho) if selection is None else selection
    g = sigmoid(gate)
    rows = [tuple(int(x) for x in r) for r in rows]
    out = np.empty((len(rows), d), dtype=np.float64)
    for t, (b, h, i) in enumerate(rows):
        o = local_row(q, k, v, b, h, i, window, scale)
        if mask[b, i]:
            o = o + g[b, i] * global_row(q, k, v, b, h, i, scale)
        out[t] = o
    return {"o_rows": out, "mask": mask, "idx": idx, "rank": rank}
