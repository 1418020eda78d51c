"""CPU fp64 oracle for the threshold budget controller and the decode step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP kernels.

What is computed, and from which passage
-----------------------------------------
LoGo (abstract): a learned gate activates global attention per token and a
threshold-based budget controller keeps a target global ratio. "Learning
When to Attend" (section "Empirical Validation and System Optimization"):
decoding reads the full context only for the tokens that are routed to it.

Readings taken where the pages are silent:

* Threshold rule: a token is selected iff its logit is strictly above the
  sequence's threshold tau (a NaN logit never is).
* Running controller: after each decision, tau <- tau + eta (selected - rho).
  This is the stochastic-approximation quantile tracker: its fixed point is
  the threshold the logits exceed with probability rho, so the selected
  fraction settles at the target ratio using only past tokens (causal).
* Calibrated threshold: from a prefill's exact top-k selection, tau is the
  largest logit that was not selected (-inf when every token was), so that
  "logit > tau" reproduces that selection when the logits are distinct.
* Decode step: the cache of sequence b holds positions 0 .. lens[b]-1, the
  newest (the query's own token) included; the query is at i = lens[b]-1 and
  attends over L(i) = [max(0, i-W+1), i] and, when selected, G(i) = [0, i];
  o = o_local + sigmoid(gate) o_global on selection, o_local otherwise (the
  forward's combine, ``oracle/logo.py``).

Parity: pinned in ``tests/test_oracle_decode.py`` (the decode row equals the
pinned forward's row, the controller's fixed point against the normal
quantile function, the calibration against the top-k selection).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import logo as F

__all__ = ["controller_step", "calibrate_threshold", "decode_step", "select_threshold"]


def controller_step(gate, tau, rho: float, eta: float):
    """One decision per sequence: sel = gate > tau; tau_new = tau + eta (sel - rho)."""
    gate = np.asarray(gate, np.float32).astype(np.float64)
    tau = np.asarray(tau, np.float32).astype(np.float64)
    sel = gate > tau                      # NaN compares false
    tau_new = tau + eta * (sel.astype(np.float64) - rho)
    return sel, tau_new


def select_threshold(gate, tau):
    """Threshold selection of a whole sequence: mask [B, n] (gate > tau_b),
    idx [B, n] (ascending positions, -1 after the count), count [B]."""
    gate = np.asarray(gate, np.float32)
    tau = np.asarray(tau, np.float32).reshape(-1)
    B, n = gate.shape
    mask = (gate > tau[:, None]).astype(np.uint8)
    idx = np.full((B, n), -1, np.int32)
    count = np.zeros(B, np.int32)
    for b in range(B):
        sel = np.nonzero(mask[b])[0]
        idx[b, :len(sel)] = sel
        count[b] = len(sel)
    return mask, idx, count


def calibrate_threshold(gate, rho: float):
    """tau_b = the largest logit the exact top-k selection left out."""
    gate = np.asarray(gate, np.float32)
    mask, _, _ = F.select_queries(gate, rho)
    B, n = gate.shape
    tau = np.full(B, -np.inf)
    for b in range(B):
        rest = gate[b][(mask[b] == 0) & ~np.isnan(gate[b])]
        if rest.size:
            tau[b] = float(rest.max())
    return tau.astype(np.float32)


def decode_step(q, k_cache, v_cache, lens, gate, tau, window: int, rho: float, eta: float,
                scale: Optional[float] = None) -> dict:
    """q [B, Hq, d]; k_cache, v_cache [B, Hkv, cap, d]; lens [B] (>= 1);
    gate, tau [B]. Returns o [B, Hq, d], selected [B], tau_new [B]."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    scale = F.default_scale(d) if scale is None else scale
    sel, tau_new = controller_step(gate, tau, rho, eta)
    g = F.sigmoid(np.asarray(gate, np.float32).astype(np.float64))
    o = np.zeros((B, Hq, d))
    for b in range(B):
        i = int(lens[b]) - 1
        lo = max(0, i - window + 1)
        for h in range(Hq):
            hk = F._kv_head(h, Hq, Hkv)
            o[b, h] = F._attend(q[b, h], k_cache[b, hk, lo:i + 1], v_cache[b, hk, lo:i + 1],
                                scale)
            if sel[b]:
                o[b, h] += g[b] * F._attend(q[b, h], k_cache[b, hk, :i + 1],
                                            v_cache[b, hk, :i + 1], scale)
    return {"o": o, "selected": sel.astype(np.uint8), "tau": tau_new}


def normal_quantile(p: float) -> float:
    """Inverse of the standard normal distribution function, by bisection on
    the error function (for the controller's fixed-point pin)."""
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * (1.0 + math.erf(mid / math.sqrt(2.0))) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)
