"""Seeded input generators: determinism, bf16 rounding, bursty gate runs. No GPU."""
import numpy as np
import torch

from workloads import (WORKLOADS, bf16_bits, bursty_gate_runs, get_workload,
                       make_inputs, round_to_bf16)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 37,
                        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf,
                                  3.3895314e38, 1e-40, -1e-42], np.float32)])
    ours = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(round_to_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_inputs_deterministic_and_rounded():
    w = get_workload("mha4k", n=256, Hq=2, Hkv=2)
    a = make_inputs(w, 3)
    b = make_inputs(w, 3)
    assert a.sha256() == b.sha256()
    assert np.array_equal(round_to_bf16(a.q), a.q)
    assert np.all(np.abs(a.q) < 2.0)        # N(0,1)/sqrt(d) entries
    c = make_inputs(w, 4)
    assert a.sha256() != c.sha256()
    g = make_inputs(w, 3, gate_only=True)
    assert np.array_equal(g.gate, a.gate)


def test_bursty_runs():
    r = np.random.default_rng(1)
    s = bursty_gate_runs(r, 65536)
    assert np.all(np.diff(s) >= 64) and s[0] >= 64 and s[-1] < 65536
    assert 40 < len(s) < 100
    w = get_workload("sweep64k", n=8192, Hq=1, Hkv=1)
    inp = make_inputs(w, 0)
    assert (inp.gate > 2.5).mean() > 0.03


def test_workload_table():
    assert WORKLOADS["gqa32k"].Hq == 16 and WORKLOADS["gqa32k"].Hkv == 4
    assert WORKLOADS["tiny"].dtype == "f32"
