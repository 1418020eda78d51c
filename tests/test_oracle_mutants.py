"""Planted mistakes in the oracle (on the CPU) must each trip at least one pin.

Each mutant replaces one function of ``oracle.logo`` with a plausibly wrong
version (a window off by one, a dropped term, a wrong sign or index, a
transposed operand, a wrong tie rule) for the duration of one test. The test
passes when at least one pin fails on the mutant: evidence that the pins pin
the oracle, not just restate it. No GPU."""
import math

import numpy as np
import pytest

import oracle.logo as O
import pins

_real = {name: getattr(O, name) for name in
         ("local_row", "global_row", "_attend", "_kv_head", "select_queries",
          "target_count", "sigmoid", "softmax_weights", "combine")}


def _local_row_wide(q, k, v, b, h, i, window, scale):
    hk = O._kv_head(h, q.shape[1], k.shape[1])
    lo = max(0, i - window)                      # W+1 keys
    return O._attend(q[b, h, i], k[b, hk, lo:i + 1], v[b, hk, lo:i + 1], scale)


def _local_row_no_self(q, k, v, b, h, i, window, scale):
    hk = O._kv_head(h, q.shape[1], k.shape[1])
    lo = max(0, i - window)
    if i == 0:
        return np.zeros(q.shape[3])
    return O._attend(q[b, h, i], k[b, hk, lo:i], v[b, hk, lo:i], scale)   # self dropped


def _local_row_wrong_query(q, k, v, b, h, i, window, scale):
    hk = O._kv_head(h, q.shape[1], k.shape[1])
    lo = max(0, i - window + 1)
    return O._attend(q[b, h, lo], k[b, hk, lo:i + 1], v[b, hk, lo:i + 1], scale)  # wrong row


def _global_row_no_diag(q, k, v, b, h, i, scale):
    hk = O._kv_head(h, q.shape[1], k.shape[1])
    if i == 0:
        return np.zeros(q.shape[3])
    return O._attend(q[b, h, i], k[b, hk, :i], v[b, hk, :i], scale)


def _global_row_windowed(q, k, v, b, h, i, scale):
    return _real["local_row"](q, k, v, b, h, i, 64, scale)   # not the full context


def _attend_no_scale(qrow, keys, vals, scale):
    return _real["_attend"](qrow, keys, vals, 1.0)


def _attend_kv_swapped(qrow, keys, vals, scale):
    return _real["_attend"](qrow, vals, keys, scale)


def _attend_exp_sign(qrow, keys, vals, scale):
    return _real["_attend"](qrow, keys, vals, -scale)


def _kv_head_modulo(h, Hq, Hkv):
    return h % Hkv


def _select_ties_high(gate, rho):
    gate = np.asarray(gate, dtype=np.float32)
    B, n = gate.shape
    k = O.target_count(rho, n)
    mask = np.zeros((B, n), np.uint8)
    idx = np.zeros((B, k), np.int32)
    rank = np.full((B, n), -1, np.int32)
    for b in range(B):
        g = gate[b].astype(np.float64)[::-1]
        order = (n - 1) - np.argsort(-g, kind="stable")   # ties to the higher position
        ch = np.sort(order[:k])
        mask[b, ch] = 1
        idx[b] = ch
        rank[b, ch] = np.arange(k)
    return mask, idx, rank


def _select_nan_high(gate, rho):
    g = np.array(gate, dtype=np.float32, copy=True)
    g[np.isnan(g)] = np.inf                      # NaN treated as the largest
    return _real["select_queries"](g, rho)


def _select_negzero_low(gate, rho):
    g = np.array(gate, dtype=np.float32, copy=True)
    neg0 = (g == 0) & np.signbit(g)
    g[neg0] = -1e-30                             # -0.0 ranked below +0.0
    return _real["select_queries"](g, rho)


def _target_floor(rho, n):
    return int(min(max(math.floor(float(rho) * float(n)), 0), n))


def _sigmoid_identity(x):
    return np.asarray(x, dtype=np.float64)


def _softmax_unnormalised(s):
    s = np.asarray(s, dtype=np.float64)
    return np.exp(s - s.max())


def _combine_minus(o_local, o_global, rank, gate):
    neg = -np.asarray(o_global, dtype=np.float64)
    return _real["combine"](o_local, neg, rank, gate)


MUTANTS = {
    "window_plus_one": ("local_row", _local_row_wide),
    "window_drops_self": ("local_row", _local_row_no_self),
    "local_wrong_query_row": ("local_row", _local_row_wrong_query),
    "global_drops_diagonal": ("global_row", _global_row_no_diag),
    "global_windowed": ("global_row", _global_row_windowed),
    "scale_dropped": ("_attend", _attend_no_scale),
    "keys_values_swapped": ("_attend", _attend_kv_swapped),
    "score_sign_flipped": ("_attend", _attend_exp_sign),
    "gqa_modulo_head_map": ("_kv_head", _kv_head_modulo),
    "ties_to_higher_position": ("select_queries", _select_ties_high),
    "nan_ranked_highest": ("select_queries", _select_nan_high),
    "negative_zero_below_zero": ("select_queries", _select_negzero_low),
    "count_floor": ("target_count", _target_floor),
    "gate_not_squashed": ("sigmoid", _sigmoid_identity),
    "softmax_unnormalised": ("softmax_weights", _softmax_unnormalised),
    "combine_sign_flipped": ("combine", _combine_minus),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
