"""Pins of the controller / decode oracle (``oracle/decode.py``) to things
other than itself, and planted mistakes that must trip them. No GPU."""
import numpy as np
import pytest
from scipy.stats import norm

import oracle.decode as DC
import oracle.logo as F


def pin_decode_equals_forward_row(DM):
    """The decode row of the newest token equals the pinned forward's row of
    that position, selected or not (same window, same logit)."""
    r = np.random.default_rng(1)
    B, Hq, Hkv, n, d, W = 2, 4, 2, 23, 8, 5
    q = r.standard_normal((B, Hq, n, d))
    k = r.standard_normal((B, Hkv, n, d))
    v = r.standard_normal((B, Hkv, n, d))
    gate = r.standard_normal((B, n)).astype(np.float32)
    fw = F.forward(q, k, v, gate, W, 0.4)
    for i in (0, 3, 11, 22):
        lens = np.array([i + 1, i + 1])
        # tau just below / above the token's logit reproduces its selection
        sel = fw["mask"][:, i].astype(bool)
        tau = np.where(sel, np.nextafter(gate[:, i], -np.inf), gate[:, i]).astype(np.float32)
        out = DM.decode_step(q[:, :, i], k, v, lens, gate[:, i], tau, W, 0.4, 0.0)
        assert np.array_equal(out["selected"].astype(bool), sel)
        assert np.allclose(out["o"], fw["o"][:, :, i], atol=1e-12)


def pin_controller_steps(DM):
    """Closed forms: a selected token moves tau up by eta (1 - rho), an
    unselected one down by eta rho; NaN is never selected; ties stay out."""
    sel, tau = DM.controller_step([2.0, -1.0, np.nan, 0.5], [0.0, 0.0, 0.0, 0.5], 0.2, 0.1)
    assert list(sel) == [True, False, False, False]
    assert np.allclose(tau, [0.08, -0.02, -0.02, 0.48])


def pin_controller_fixed_point(DM):
    """On N(0,1) logits the running threshold settles at the normal quantile
    of 1 - rho and the selected fraction at rho."""
    r = np.random.default_rng(2)
    for rho in (0.2, 0.05):
        tau = np.zeros(1, np.float32)
        hits = 0
        N = 60000
        g = r.standard_normal(N).astype(np.float32)
        taus = []
        for t in range(N):
            eta = 0.05 if t < N // 2 else 0.01
            sel, tau_new = DM.controller_step(g[t:t + 1], tau, rho, eta)
            tau = tau_new.astype(np.float32)
            if t >= N // 2:
                hits += int(sel[0])
                taus.append(float(tau[0]))
        assert abs(np.mean(taus) - norm.ppf(1 - rho)) < 0.05, (rho, np.mean(taus))
        assert abs(hits / (N // 2) - rho) < 0.01
    assert abs(DM.normal_quantile(0.8) - norm.ppf(0.8)) < 1e-9


def pin_calibrated_threshold(DM):
    """'logit > tau' with the calibrated tau reproduces the exact top-k
    selection on distinct logits; all selected gives -inf."""
    r = np.random.default_rng(3)
    g = r.standard_normal((3, 101)).astype(np.float32)
    for rho in (0.0, 0.1, 0.37, 1.0):
        tau = DM.calibrate_threshold(g, rho)
        mask, idx, count = DM.select_threshold(g, tau)
        ref, ridx, _ = F.select_queries(g, rho)
        assert np.array_equal(mask, ref), rho
        for b in range(3):
            assert count[b] == ridx.shape[1]
            assert np.array_equal(idx[b, :count[b]], ridx[b])
            assert np.all(idx[b, count[b]:] == -1)
    assert np.all(DM.calibrate_threshold(g, 1.0) == -np.inf)


PINS = [pin_decode_equals_forward_row, pin_controller_steps, pin_controller_fixed_point,
        pin_calibrated_threshold]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_decode_pin(pin):
    pin(DC)


def _some_pin_fails():
    for pin in PINS:
        try:
            pin(DC)
        except AssertionError:
            return True
    return False


_real_step = DC.controller_step


def _step_ge(gate, tau, rho, eta):
    gate = np.asarray(gate, np.float32).astype(np.float64)
    tau = np.asarray(tau, np.float32).astype(np.float64)
    sel = gate >= tau
    return sel, tau + eta * (sel - rho)


def _step_sign(gate, tau, rho, eta):
    sel, t = _real_step(gate, tau, rho, eta)
    tau = np.asarray(tau, np.float32).astype(np.float64)
    return sel, tau - (t - tau)


def _step_no_rho(gate, tau, rho, eta):
    sel, _ = _real_step(gate, tau, rho, eta)
    return sel, np.asarray(tau, np.float32) + eta * sel


@pytest.mark.parametrize("mut", [_step_ge, _step_sign, _step_no_rho], ids=lambda f: f.__name__)
def test_controller_mutant_is_caught(mut, monkeypatch):
    monkeypatch.setattr(DC, "controller_step", mut)
    assert _some_pin_fails()


def test_decode_window_mutant_is_caught(monkeypatch):
    real = DC.decode_step

    def wide(q, k_cache, v_cache, lens, gate, tau, window, rho, eta, scale=None):
        return real(q, k_cache, v_cache, lens, gate, tau, window + 1, rho, eta, scale)
    monkeypatch.setattr(DC, "decode_step", wide)
    assert _some_pin_fails()
