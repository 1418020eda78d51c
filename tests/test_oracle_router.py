"""Pins of the routed-forward oracle (``oracle/router.py``) to things other
than itself, and planted mistakes that must trip them. No GPU."""
import math

import numpy as np
import pytest
import torch

import oracle.logo as F
import oracle.router as R


def _inputs(seed, B=2, Hq=4, Hkv=2, n=19, d=8):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, n, d))
    k = r.standard_normal((B, Hkv, n, d))
    v = r.standard_normal((B, Hkv, n, d))
    w = r.standard_normal((Hq, d))
    return q, k, v, w, float(r.standard_normal())


def pin_router_torch(RM):
    """The logits equal an independent torch float64 formulation: band-masked
    softmax attention for every head, then one einsum with the weights."""
    for seed, W in ((1, 5), (2, 40)):
        q, k, v, w, bias = _inputs(seed)
        B, Hq, n, d = q.shape
        tq, tk, tv = (torch.tensor(x) for x in (q, k, v))
        kr, vr = tk.repeat_interleave(2, dim=1), tv.repeat_interleave(2, dim=1)
        i = torch.arange(n)[:, None]
        j = torch.arange(n)[None, :]
        band = (j <= i) & (j >= i - W + 1)
        o = torch.nn.functional.scaled_dot_product_attention(tq, kr, vr, attn_mask=band)
        want = torch.einsum("bhid,hd->bi", o, torch.tensor(w)).numpy() + bias
        got = RM.forward_routed(q, k, v, w, bias, W, 0.3)["gate"]
        assert np.allclose(got, want, atol=1e-12), np.abs(got - want).max()


def pin_router_zero_weights(RM):
    """w = 0: every logit is the bias, so the selection is the first k
    positions (ties to the lower position) and every selected row gets
    sigmoid(bias) of its global output."""
    q, k, v, w, bias = _inputs(3)
    w[:] = 0.0
    out = RM.forward_routed(q, k, v, w, 0.75, 4, 0.3)
    n = q.shape[2]
    kk = math.ceil(0.3 * n)
    assert np.all(out["gate"] == 0.75)
    assert np.array_equal(out["idx"], np.tile(np.arange(kk), (2, 1)))


def pin_router_constant_values(RM):
    """v_j = c per kv head: o_local = c, so gate = sum_h <w_h, c_kv(h)> + bias,
    the same for every token."""
    q, k, v, w, bias = _inputs(4)
    v[:] = v[:, :, :1, :]
    out = RM.forward_routed(q, k, v, w, bias, 3, 0.25)
    want = bias + sum(float(w[h] @ v[0, h // 2, 0]) for h in range(4))
    assert np.allclose(out["gate"][0], want, atol=1e-12)


def pin_router_consistent_with_forward(RM):
    """Given its own logits, the routed forward is the pinned forward (which
    selects on the float32 rounding of the logits it is given and squashes
    them as given)."""
    q, k, v, w, bias = _inputs(5)
    out = RM.forward_routed(q, k, v, w, bias, 6, 0.4)
    assert np.array_equal(out["gate32"], out["gate"].astype(np.float32))
    ref = F.forward(q, k, v, out["gate"], 6, 0.4)
    assert np.array_equal(out["idx"], ref["idx"])
    assert np.allclose(out["o"], ref["o"], atol=1e-12)
    g = RM.router_logits_at(q, k, v, w, bias, 6, [(0, 0), (1, 18), (1, 7)])
    assert np.allclose(g, [out["gate"][0, 0], out["gate"][1, 18], out["gate"][1, 7]],
                       atol=1e-12)


def pin_router_decides_in_float32(RM):
    """Values that differ from a constant per kv head by amounts far below
    float32 resolution give float64 logits that differ only there: rounded to
    float32 they tie, so the selection is the first k positions (ties to the
    lower position), whatever order the float64 logits have."""
    q, k, v, w, bias = _inputs(8, B=1)
    n = q.shape[2]
    v[:] = v[:, :, :1, :]
    v[0, :, :, 0] += 1e-13 * np.arange(n)[::-1][None, :]   # later tokens: smaller
    w[:] = np.abs(w)
    out = RM.forward_routed(q, k, v, w, bias, n, 0.25)
    g = out["gate"][0]
    assert np.unique(out["gate32"][0]).size == 1      # one float32 value
    assert np.unique(g).size > 1                      # distinct float64 values
    kk = math.ceil(0.25 * n)
    assert np.array_equal(out["idx"][0], np.arange(kk))


def pin_router_linear(RM):
    """The logits are affine in (w, bias)."""
    q, k, v, w, bias = _inputs(6)
    w2 = np.random.default_rng(7).standard_normal(w.shape)
    a = RM.forward_routed(q, k, v, w, bias, 5, 0.2)["gate"]
    b = RM.forward_routed(q, k, v, w2, 0.0, 5, 0.2)["gate"]
    c = RM.forward_routed(q, k, v, w + w2, bias, 5, 0.2)["gate"]
    assert np.allclose(a + b, c, atol=1e-12)


PINS = [pin_router_torch, pin_router_zero_weights, pin_router_constant_values,
        pin_router_consistent_with_forward, pin_router_decides_in_float32, pin_router_linear]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_router_pin(pin):
    pin(R)


def _some_pin_fails():
    for pin in PINS:
        try:
            pin(R)
        except AssertionError:
            return True
    return False


_real_logits = R.router_logits


def _logits_first_head_only(o_local, w, bias):
    return np.asarray(o_local, np.float64)[:, 0] @ np.asarray(w, np.float64)[0] + bias


def _logits_no_bias(o_local, w, bias):
    return _real_logits(o_local, w, 0.0)


def _logits_transposed_weights(o_local, w, bias):
    w = np.asarray(w, np.float64)
    return _real_logits(o_local, w[::-1], bias)


@pytest.mark.parametrize("mut", [_logits_first_head_only, _logits_no_bias,
                                 _logits_transposed_weights], ids=lambda f: f.__name__)
def test_router_mutant_is_caught(mut, monkeypatch):
    monkeypatch.setattr(R, "router_logits", mut)
    assert _some_pin_fails()


def test_router_float64_decision_is_caught():
    """A routed oracle that selected on the float64 logits (ordering them in
    float64) would pick the largest float64 values instead of the float32
    ties' lower positions."""
    import types

    def forward_routed_f64(q, k, v, w, bias, window, rho, scale=None):
        out = R.forward_routed(q, k, v, w, bias, window, rho, scale)
        g = out["gate"]
        B, n = g.shape
        kk = F.target_count(rho, n)
        idx = np.stack([np.sort(np.argsort(-g[b], kind="stable")[:kk]) for b in range(B)])
        return dict(out, idx=idx.astype(np.int32))

    mutant = types.SimpleNamespace(forward_routed=forward_routed_f64,
                                   router_logits_at=R.router_logits_at)
    with pytest.raises(AssertionError):
        pin_router_decides_in_float32(mutant)
