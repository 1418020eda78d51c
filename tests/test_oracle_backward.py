"""The backward oracle against its pins, and planted mistakes in it (on the
CPU) that must each trip at least one pin. No GPU."""
import numpy as np
import pytest

import oracle.backward as BW
import oracle.logo as F
import pins_backward as P


@pytest.mark.parametrize("pin", P.ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin(F, BW)


_real_row_grad = BW.row_grad
_real_backward = BW.backward


def _rg_no_centering(qrow, keys, vals, e, scale):
    q, K, V, e = (np.asarray(x, np.float64) for x in (qrow, keys, vals, e))
    p = F.softmax_weights(scale * (K @ q))
    t = V @ e
    ds = p * t                                   # the -sum p t term dropped
    return p @ V, scale * (ds @ K), scale * np.outer(ds, q), np.outer(p, e)


def _rg_dq_unscaled(qrow, keys, vals, e, scale):
    o, dq, dk, dv = _real_row_grad(qrow, keys, vals, e, scale)
    return o, dq / scale, dk, dv


def _rg_dk_sign(qrow, keys, vals, e, scale):
    o, dq, dk, dv = _real_row_grad(qrow, keys, vals, e, scale)
    return o, dq, -dk, dv


def _rg_dv_uniform(qrow, keys, vals, e, scale):
    o, dq, dk, dv = _real_row_grad(qrow, keys, vals, e, scale)
    n = len(keys)
    return o, dq, dk, np.outer(np.full(n, 1.0 / n), np.asarray(e, np.float64))


def _rg_dk_uses_query_of_keys(qrow, keys, vals, e, scale):
    # dk_j = scale ds_j k_j instead of scale ds_j q
    o, dq, dk, dv = _real_row_grad(qrow, keys, vals, e, scale)
    q, K, V, ee = (np.asarray(x, np.float64) for x in (qrow, keys, vals, e))
    p = F.softmax_weights(scale * (K @ q))
    t = V @ ee
    ds = p * (t - p @ t)
    return o, dq, scale * ds[:, None] * K, dv


def _rg_t_from_keys(qrow, keys, vals, e, scale):
    # t_j = <e, k_j>: keys and values swapped in the score gradient
    q, K, V, ee = (np.asarray(x, np.float64) for x in (qrow, keys, vals, e))
    p = F.softmax_weights(scale * (K @ q))
    t = K @ ee
    ds = p * (t - p @ t)
    return p @ V, scale * (ds @ K), scale * np.outer(ds, q), np.outer(p, ee)


def _mutated_backward(kind):
    def run(q, k, v, gate, do, window, rho, scale=None):
        B, Hq, n, d = q.shape
        Hkv = k.shape[1]
        scale = F.default_scale(d) if scale is None else scale
        do = np.asarray(do, np.float64)
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
                    ol, gq, gk, gv = _real_row_grad(q[b, h, i], k[b, hk, lo:i + 1],
                                                    v[b, hk, lo:i + 1], do[b, h, i], scale)
                    dq[b, h, i] += gq
                    dk[b, hk, lo:i + 1] += gk
                    dv[b, hk, lo:i + 1] += gv
                    o[b, h, i] = ol
                    if not mask[b, i]:
                        continue
                    e = do[b, h, i] if kind == "global_no_gate" else g[b, i] * do[b, h, i]
                    glo = lo if kind == "global_windowed" else 0
                    og, gq, gk, gv = _real_row_grad(q[b, h, i], k[b, hk, glo:i + 1],
                                                    v[b, hk, glo:i + 1], e, scale)
                    if kind != "global_dq_dropped":
                        dq[b, h, i] += gq
                    dk[b, hk, glo:i + 1] += gk
                    dv[b, hk, glo:i + 1] += gv
                    o[b, h, i] += g[b, i] * og
                    deriv = g[b, i] if kind == "sigmoid_deriv" else g[b, i] * (1 - g[b, i])
                    if kind == "dgate_head0" and h != 0:
                        continue
                    dgate[b, i] += deriv * float(do[b, h, i] @ og)
        return {"dq": dq, "dk": dk, "dv": dv, "dgate": dgate, "o": o,
                "mask": mask, "idx": idx, "rank": rank}
    return run


ROW_MUTANTS = {
    "no_centering": _rg_no_centering,
    "dq_unscaled": _rg_dq_unscaled,
    "dk_sign": _rg_dk_sign,
    "dv_uniform": _rg_dv_uniform,
    "dk_uses_keys": _rg_dk_uses_query_of_keys,
    "t_from_keys": _rg_t_from_keys,
}
BACKWARD_MUTANTS = ["global_no_gate", "global_windowed", "global_dq_dropped", "sigmoid_deriv",
                    "dgate_head0"]


def _some_pin_fails():
    for pin in P.ALL_BWD_PINS:
        try:
            pin(F, BW)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(ROW_MUTANTS))
def test_row_grad_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(BW, "row_grad", ROW_MUTANTS[name])
    assert _some_pin_fails(), name


@pytest.mark.parametrize("kind", BACKWARD_MUTANTS)
def test_backward_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(BW, "backward", _mutated_backward(kind))
    assert _some_pin_fails(), kind


def test_unmutated_mirror_passes(monkeypatch):
    """The mutant harness itself, with no mutation, passes every pin."""
    monkeypatch.setattr(BW, "backward", _mutated_backward("none"))
    assert not _some_pin_fails()


def test_lse_mutant_is_caught(monkeypatch):
    real = BW.row_lse
    monkeypatch.setattr(BW, "row_lse", lambda q, k, s: real(q, k, s) / np.log(2.0))
    assert _some_pin_fails()
