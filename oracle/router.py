"""CPU fp64 oracle for the routed forward: the gate computed from the local
branch's output, then selection, global branch and combine.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP kernels.

What is computed, and from which passage
-----------------------------------------
"Learning When to Attend", section "The Architecture of Conditional
Attention": every token first gets local attention; a router then makes one
binary decision per token, and only the chosen tokens get exact attention
over the full context. LoGo (abstract): a learned gate activates global
attention per token, a budget controller holds the target ratio.

Readings taken where the pages are silent:

* The router is a linear map of the token's local-branch output, all query
  heads concatenated, to one logit: gate_{b,i} = sum_h <w_h, o_local_{b,h,i}>
  + bias, with w [Hq, d] and a scalar bias (the pages give no router
  architecture; a linear layer is the plainest reading, and its weights
  here are synthetic).
* The budget controller, ties, combine and both branches are those of
  ``oracle/logo.py``.
* The logits are computed in float64; the selection, an integer decision
  taken by floating point, is made on those logits rounded to float32 (the
  precision the logits have on the device, where gates are float32), and the
  combine uses the sigmoid of the float64 logits. The oracle never takes a
  logit from anywhere else.

Parity: pinned in ``tests/test_oracle_router.py`` (closed forms, an
independent torch formulation, consistency with the pinned forward).
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

from . import logo as F

__all__ = ["router_logits", "forward_routed", "router_logits_at"]


def router_logits(o_local: np.ndarray, w: np.ndarray, bias: float) -> np.ndarray:
    """gate [B, n] = sum over heads and d of w[h, d] o_local[b, h, i, d] + bias."""
    o_local = np.asarray(o_local, np.float64)
    w = np.asarray(w, np.float64)
    B, Hq, n, d = o_local.shape
    if w.shape != (Hq, d):
        raise ValueError("w must be [Hq, d]")
    gate = np.full((B, n), float(bias))
    for h in range(Hq):
        gate += o_local[:, h] @ w[h]
    return gate


def forward_routed(q, k, v, w, bias: float, window: int, rho: float,
                   scale: Optional[float] = None) -> dict:
    """Local branch for every row, router logits from it (float64), the
    selection on those logits rounded to float32, global branch on the
    selected rows, combine with the sigmoid of the float64 logits. Returns o,
    gate (float64 logits), gate32 (the float32 logits the selection used),
    the selection, o_local and o_global."""
    F._check_shapes(q, k, v)
    d = q.shape[3]
    scale = F.default_scale(d) if scale is None else scale
    o_local = F.local_attention(q, k, v, window, scale)
    gate = router_logits(o_local, w, bias)
    gate32 = gate.astype(np.float32)
    mask, idx, rank = F.select_queries(gate32, rho)
    o_global = F.global_attention(q, k, v, idx, scale)
    o = F.combine(o_local, o_global, rank, gate)
    return {"o": o, "gate": gate, "gate32": gate32, "mask": mask, "idx": idx, "rank": rank,
            "o_local": o_local, "o_global": o_global}


def router_logits_at(q, k, v, w, bias: float, window: int,
                     positions: Iterable[Sequence[int]],
                     scale: Optional[float] = None) -> np.ndarray:
    """The logits of chosen (b, i) only (each needs the local rows of every
    head at that position), for inputs too large to do whole."""
    F._check_shapes(q, k, v)
    B, Hq, n, d = q.shape
    scale = F.default_scale(d) if scale is None else scale
    w = np.asarray(w, np.float64)
    positions = [tuple(int(x) for x in p) for p in positions]
    out = np.full(len(positions), float(bias))
    for t, (b, i) in enumerate(positions):
        for h in range(Hq):
            out[t] += float(F.local_row(q, k, v, b, h, i, window, scale) @ w[h])
    return out
