"""CPU fp64 oracle for packed variable-length batches.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP kernels.

What is computed, and from which passage
-----------------------------------------
"Local-global attention" (section "Implementation sketch", its notes on
packing): when several examples are packed into one row, a token must not
attend across an example boundary, so the mask needs per-example
boundaries. LoGo (abstract): the budget controller holds a target ratio per
sequence.

Readings taken where the pages are silent:

* A packed batch is one token stream of T tokens split by cu_seqlens
  (example e holds tokens cu[e] .. cu[e+1]-1). Every example is a sequence
  of its own: the local window and the global prefix are clipped at the
  example's first token, and the selection is the top ceil(rho * n_e) of the
  example's own logits (ties to the lower position).
* Outputs are laid out like the inputs (q, o [Hq, T, d]); idx concatenates
  the examples' selections (absolute token positions, ascending), and rank
  is a token's index in that concatenation (-1 if not selected).

The function below is that definition: each example runs through the pinned
forward of ``oracle/logo.py`` on its own slice, and the results are placed
back. Parity: pinned in ``tests/test_oracle_varlen.py`` against torch float64
attention with one block-diagonal (same-example), causal and banded mask
over the whole packed stream, and against brute-force selection.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import logo as F

__all__ = ["forward_varlen", "check_cu"]


def check_cu(cu, T: int) -> np.ndarray:
    cu = np.asarray(cu, np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at T and not decrease")
    return cu


def forward_varlen(q, k, v, gate, cu, window: int, rho: float,
                   scale: Optional[float] = None) -> dict:
    """q [Hq, T, d], k, v [Hkv, T, d], gate [T], cu [E+1]. Returns o [Hq, T, d],
    mask [T], idx [K] (absolute positions), rank [T], ks [E] (per-example
    counts) and koff [E+1] (offsets of each example's selection in idx)."""
    q = np.asarray(q, np.float64)
    Hq, T, d = q.shape
    cu = check_cu(cu, T)
    E = cu.size - 1
    o = np.zeros((Hq, T, d))
    mask = np.zeros(T, np.uint8)
    rank = np.full(T, -1, np.int32)
    idx_parts = []
    ks = np.zeros(E, np.int64)
    for e in range(E):
        a, b = int(cu[e]), int(cu[e + 1])
        if b == a:
            continue
        fw = F.forward(q[None, :, a:b], np.asarray(k)[None, :, a:b], np.asarray(v)[None, :, a:b],
                       np.asarray(gate, np.float32)[None, a:b], window, rho, scale)
        o[:, a:b] = fw["o"][0]
        mask[a:b] = fw["mask"][0]
        idx_parts.append(fw["idx"][0].astype(np.int64) + a)
        ks[e] = fw["idx"].shape[1]
    idx = np.concatenate(idx_parts).astype(np.int32) if idx_parts else np.zeros(0, np.int32)
    rank[idx] = np.arange(idx.size, dtype=np.int32)
    koff = np.concatenate([[0], np.cumsum(ks)]).astype(np.int64)
    return {"o": o, "mask": mask, "idx": idx, "rank": rank, "ks": ks, "koff": koff}
