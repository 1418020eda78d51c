"""GPU budget controller + compaction against the oracle: mask, idx and rank
bit-exact, on ties, signed zeros, NaN, infinities, ragged lengths, every
workload length, and the extreme budgets."""
import numpy as np
import pytest
import torch

import oracle
import token_level_dynamic_amd as T
from gpu_util import dev, ensure_built, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _gpu_select(gate, rho):
    B, n = gate.shape
    p = T.make_problem(B, 1, 1, n, 64, 1, rho, dtype="bf16")
    k = T.logo_target_count(rho, n)
    g = torch.from_numpy(np.ascontiguousarray(gate, dtype=np.float32)).to(dev())
    mask = torch.full((B, n), 7, dtype=torch.uint8, device=dev())
    idx = torch.full((B, k), -7, dtype=torch.int32, device=dev())
    rank = torch.full((B, n), -7, dtype=torch.int32, device=dev())
    T.logo_select_queries(p, g, mask, idx, rank)
    torch.cuda.synchronize()
    return mask.cpu().numpy(), idx.cpu().numpy(), rank.cpu().numpy()


def _check(gate, rho, label):
    say(f"[select] {label} B={gate.shape[0]} n={gate.shape[1]} rho={rho}")
    m, i, r = _gpu_select(gate, rho)
    rm, ri, rr = oracle.select_queries(gate, rho)
    assert np.array_equal(m, rm), label
    assert np.array_equal(i, ri), label
    assert np.array_equal(r, rr), label


def _gates(kind, B, n, seed):
    r = np.random.default_rng(seed)
    if kind == "normal":
        return r.standard_normal((B, n)).astype(np.float32)
    if kind == "int_ties":
        return r.integers(-3, 4, size=(B, n)).astype(np.float32)
    if kind == "all_equal":
        return np.full((B, n), 0.5, np.float32)
    if kind == "specials":
        g = r.integers(-2, 3, size=(B, n)).astype(np.float32)
        sp = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0], np.float32)
        sel = r.random((B, n)) < 0.3
        g[sel] = sp[r.integers(0, len(sp), size=int(sel.sum()))]
        return g
    if kind == "near_ties":
        base = r.standard_normal((B, n)).astype(np.float32)
        return np.nextafter(base, np.float32(np.inf) * np.sign(r.random((B, n)) - 0.5)) \
            .astype(np.float32)
    if kind == "ascending":
        return np.tile(np.arange(n, dtype=np.float32), (B, 1))
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "int_ties", "all_equal", "specials", "near_ties",
                                  "ascending"])
@pytest.mark.parametrize("n", [1, 7, 64, 1000, 8192, 8193, 20001])
def test_select_matches_oracle(kind, n):
    for rho in (0.0, 0.05, 0.2, 0.5, 1.0, 0.37):
        _check(_gates(kind, 2, n, n), rho, f"{kind}")


@pytest.mark.parametrize("n", [4096, 32768, 65536, 131072])
def test_select_workload_lengths(n):
    g = _gates("normal", 2, n, 11)
    for rho in (0.05, 0.2, 0.25, 0.5):
        _check(g, rho, "normal")
    _check(_gates("int_ties", 1, n, 12), 0.2, "int_ties")


def test_select_count_property_large():
    n = 131072
    g = _gates("normal", 3, n, 13)
    m, i, r = _gpu_select(g, 0.2)
    k = T.logo_target_count(0.2, n)
    assert (m.sum(axis=1) == k).all()
    for b in range(3):
        assert np.all(np.diff(i[b]) > 0)
        assert np.array_equal(r[b][i[b]], np.arange(k))
        # every unselected logit is <= every selected one
        assert g[b][m[b] == 0].max() <= g[b][m[b] == 1].min()
