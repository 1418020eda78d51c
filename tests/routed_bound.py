"""Error scales of the routed forward's logits, for the GPU test's tolerance.

Not part of the oracle: this computes how far a logit computed in floating
point can sit from the exact one, from the exact softmax weights of each
local row (float64, NumPy only, so the oracle's worker processes can run it).

A logit is g_i = bias + sum_h <w_h, o_h,i>, o_h,i = sum_{j in L(i)} p_hij v_j.
The device rounds each (unnormalised) weight to bf16 before the P V product,
a relative error eta_hij with |eta| <= 2^-8, and accumulates in float32. In
the probabilistic model of rounding errors (Higham and Mary, "A New Approach
to Probabilistic Rounding Error Analysis", SIAM J. Sci. Comput. 2019:
independent, mean-zero errors), Hoeffding's inequality bounds
|sum_j a_j eta_j| by lam u sqrt(sum_j a_j^2) except with probability
2 exp(-lam^2 / 2). The weight rounding moves g_i by
sum_h sum_j p_hij eta_hij <w_h, v_j>, so its scale is
    s_i = sqrt(sum_h sum_j (p_hij <w_h, v_j>)^2),
and the float32 sums (the P V products over the window, the dot product over
Hq d terms) have scales sqrt(W) sum_h ||w_h|| max_j ||v_j|| and
sqrt(Hq d + 2) sum_h ||w_h|| ||o_h,i||.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np


def logit_error_scales(q, k, v, w, window: int, positions: Iterable[Sequence[int]],
                       scale: Optional[float] = None) -> np.ndarray:
    """[len(positions), 3]: s_i (weight rounding), the P V accumulation
    scale and the dot-product accumulation scale of each (b, i)."""
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    w = np.asarray(w, np.float64)
    wn = np.linalg.norm(w, axis=1)
    out = np.zeros((0, 3))
    rows = []
    for b, i in positions:
        lo = max(0, i - window + 1)
        s2 = 0.0
        pv = 0.0
        dot = 0.0
        for h in range(Hq):
            hk = h // G
            K = np.asarray(k[b, hk, lo:i + 1], np.float64)
            V = np.asarray(v[b, hk, lo:i + 1], np.float64)
            s = scale * (K @ np.asarray(q[b, h, i], np.float64))
            p = np.exp(s - s.max())
            p /= p.sum()
            u = V @ w[h]
            s2 += float(((p * u) ** 2).sum())
            pv += wn[h] * float(np.sqrt((V ** 2).sum(axis=1)).max())
            dot += wn[h] * float(np.linalg.norm(p @ V))
        rows.append((math.sqrt(s2), math.sqrt(i + 1 - lo) * pv, math.sqrt(Hq * d + 2) * dot))
    return np.asarray(rows, np.float64).reshape(-1, 3) if rows else out


def logit_bound(scales: np.ndarray, dtype: str, lam: float = 8.0) -> np.ndarray:
    """The tolerance m_i on |device logit - float64 logit| from the scales
    (lam = 8: each term fails with probability below 2e-14)."""
    u_p = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -22
    u32 = 2.0 ** -24
    return lam * (u_p * scales[:, 0] + u32 * (scales[:, 1] + scales[:, 2])) + 1e-7
