"""Pins of the packed variable-length oracle (``oracle/varlen.py``) to
things other than itself, and planted mistakes that must trip them. No GPU."""
import math

import numpy as np
import pytest
import torch

import oracle.logo as F
import oracle.varlen as VL


def _inputs(seed, lens, Hq=4, Hkv=2, d=8):
    r = np.random.default_rng(seed)
    T = int(sum(lens))
    q = r.standard_normal((Hq, T, d))
    k = r.standard_normal((Hkv, T, d))
    v = r.standard_normal((Hkv, T, d))
    gate = r.standard_normal(T).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, gate, cu


def _brute_select(g, k):
    """i is selected iff fewer than k tokens of its example beat it (a larger
    logit, or an equal one at a lower position)."""
    n = g.size
    sel = np.zeros(n, bool)
    for i in range(n):
        beats = sum(1 for j in range(n) if g[j] > g[i] or (g[j] == g[i] and j < i))
        sel[i] = beats < k
    return sel


def pin_varlen_dense_block_mask(VM):
    """Whole packed stream at once in torch float64: softmax with a mask that is
    same-example AND causal AND (banded | selected-and-global), combined with
    sigmoid of the logit on selected rows."""
    for seed, lens, W, rho in ((1, [5, 1, 9, 13, 2], 4, 0.3), (2, [17, 17], 40, 0.5),
                               (3, [3, 0, 11, 6], 2, 0.0), (4, [7, 8], 3, 1.0)):
        q, k, v, gate, cu = _inputs(seed, lens)
        out = VM.forward_varlen(q, k, v, gate, cu, W, rho)
        Hq, T, d = q.shape
        seg = np.repeat(np.arange(len(lens)), lens)
        same = torch.tensor(seg[:, None] == seg[None, :])
        i = torch.arange(T)[:, None]
        j = torch.arange(T)[None, :]
        causal = j <= i
        band = causal & (j >= i - W + 1) & same
        full = causal & same
        tq = torch.tensor(q)
        kr = torch.tensor(k).repeat_interleave(Hq // k.shape[0], dim=0)
        vr = torch.tensor(v).repeat_interleave(Hq // k.shape[0], dim=0)
        ol = torch.nn.functional.scaled_dot_product_attention(tq, kr, vr, attn_mask=band)
        og = torch.nn.functional.scaled_dot_product_attention(tq, kr, vr, attn_mask=full)
        sel = torch.tensor(out["mask"].astype(bool))
        g = torch.sigmoid(torch.tensor(gate.astype(np.float64)))
        want = ol + (sel * g)[None, :, None] * og
        assert np.allclose(out["o"], want.numpy(), atol=1e-12), (seed, lens)


def pin_varlen_selection_bruteforce(VM):
    r = np.random.default_rng(5)
    lens = [6, 1, 10, 4]
    q, k, v, _, cu = _inputs(6, lens)
    gate = r.integers(-2, 3, size=sum(lens)).astype(np.float32)   # many ties
    for rho in (0.0, 0.25, 0.5, 1.0):
        out = VM.forward_varlen(q, k, v, gate, cu, 3, rho)
        want = np.concatenate([_brute_select(gate[cu[e]:cu[e + 1]],
                                             min(lens[e], math.ceil(rho * lens[e])))
                               for e in range(len(lens))])
        assert np.array_equal(out["mask"].astype(bool), want), rho
        assert np.all(np.diff(out["idx"]) > 0)
        assert np.array_equal(out["rank"][out["idx"]], np.arange(out["idx"].size))
        assert np.array_equal(out["ks"], [math.ceil(rho * n) for n in lens])


def pin_varlen_single_example(VM):
    """One example is the plain forward."""
    q, k, v, gate, cu = _inputs(7, [21])
    out = VM.forward_varlen(q, k, v, gate, cu, 5, 0.3)
    ref = F.forward(q[None], k[None], v[None], gate[None], 5, 0.3)
    assert np.allclose(out["o"], ref["o"][0], atol=1e-13)
    assert np.array_equal(out["idx"], ref["idx"][0])


PINS = [pin_varlen_dense_block_mask, pin_varlen_selection_bruteforce, pin_varlen_single_example]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_varlen_pin(pin):
    pin(VL)


def test_bad_cu_rejected():
    q, k, v, gate, cu = _inputs(8, [4, 4])
    for bad in ([0, 4], [1, 4, 8], [0, 5, 4, 8]):
        with pytest.raises(ValueError):
            VL.forward_varlen(q, k, v, gate, np.array(bad), 3, 0.5)


def _some_pin_fails():
    for pin in PINS:
        try:
            pin(VL)
        except AssertionError:
            return True
    return False


def test_cross_boundary_mutant_is_caught(monkeypatch):
    """Treating the packed stream as one sequence (attention and selection
    across boundaries) must fail a pin."""
    def whole(q, k, v, gate, cu, window, rho, scale=None):
        T = q.shape[1]
        return VL.__dict__["_real"](q, k, v, gate, np.array([0, T]), window, rho, scale)
    monkeypatch.setitem(VL.__dict__, "_real", VL.forward_varlen)
    monkeypatch.setattr(VL, "forward_varlen", whole)
    assert _some_pin_fails()


def test_global_selection_mutant_is_caught(monkeypatch):
    """Per-example attention but one budget over the whole stream."""
    real = VL.forward_varlen

    def pooled(q, k, v, gate, cu, window, rho, scale=None):
        out = real(q, k, v, gate, cu, window, rho, scale)
        T = q.shape[1]
        m, idx, rank = F.select_queries(np.asarray(gate, np.float32)[None], rho)
        out["mask"], out["idx"] = m[0], idx[0]
        return out
    monkeypatch.setattr(VL, "forward_varlen", pooled)
    assert _some_pin_fails()
