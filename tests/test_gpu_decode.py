"""GPU threshold controller, calibration, threshold selection and decode step
against the oracle (``oracle/decode.py``). Decisions (selected, mask, idx,
count) bit-exact; tau within float32 rounding of its one update; outputs
within 2e-2 (bf16) or 1e-4 (float32), the forward's bounds."""
import numpy as np
import pytest
import torch

import oracle
import oracle.decode as DC
import token_level_dynamic_amd as T
from gpu_util import dev, ensure_built, say
from workloads import DECODE_WORKLOADS, make_decode_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _dev_io(x, bits, dtype):
    if dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev())


def run_decode(cfg, inp, eta):
    p = T.make_decode_problem(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["cap"], cfg["d"],
                              cfg["window"], cfg["rho"], eta=eta, dtype=cfg["dtype"])
    dt = cfg["dtype"]
    q = _dev_io(inp.q, inp.bits.get("q"), dt)
    k = _dev_io(inp.k, inp.bits.get("k"), dt)
    v = _dev_io(inp.v, inp.bits.get("v"), dt)
    lens = torch.from_numpy(inp.lens).to(dev())
    gate = torch.from_numpy(inp.gate).to(dev())
    tau = torch.from_numpy(inp.tau.copy()).to(dev())
    o = torch.empty((cfg["B"], cfg["Hq"], cfg["d"]), dtype=T.io_dtype(p), device=dev())
    sel = torch.empty(cfg["B"], dtype=torch.uint8, device=dev())
    ws = torch.empty(T.logo_decode_workspace_size(p), dtype=torch.uint8, device=dev())
    T.logo_decode_step(p, q, k, v, lens, gate, tau, o, sel, ws)
    torch.cuda.synchronize()
    return {"o": o.float().cpu().numpy(), "selected": sel.cpu().numpy(),
            "tau": tau.cpu().numpy()}


CASES = {
    "bf16_g2_chunks": dict(B=6, Hq=4, Hkv=2, cap=5000, d=128, window=300, rho=0.2,
                           dtype="bf16"),
    "bf16_g1_d64": dict(B=4, Hq=3, Hkv=3, cap=2100, d=64, window=2047, rho=0.5, dtype="bf16"),
    "bf16_g4": dict(B=5, Hq=8, Hkv=2, cap=4500, d=128, window=2049, rho=0.3, dtype="bf16"),
    "bf16_g7": dict(B=3, Hq=14, Hkv=2, cap=3000, d=128, window=100, rho=0.2, dtype="bf16"),
    "bf16_g8_window1": dict(B=4, Hq=8, Hkv=1, cap=700, d=64, window=1, rho=0.2, dtype="bf16"),
    "bf16_g3_d64": dict(B=3, Hq=6, Hkv=2, cap=3100, d=64, window=1500, rho=0.3, dtype="bf16"),
    "bf16_g16": dict(B=2, Hq=16, Hkv=1, cap=2500, d=128, window=700, rho=0.5, dtype="bf16"),
    "f32_g2": dict(B=4, Hq=4, Hkv=2, cap=2500, d=128, window=64, rho=0.25, dtype="f32"),
    "f32_g1_d64": dict(B=3, Hq=2, Hkv=2, cap=600, d=64, window=600, rho=0.1, dtype="f32"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_matches_oracle(name):
    cfg = CASES[name]
    B, cap = cfg["B"], cfg["cap"]
    r = np.random.default_rng(7)
    # lengths: 1, around the window and the chunk edge (2048), the full cache
    pool = [1, 2, cfg["window"], cfg["window"] + 1, 2047, 2048, 2049, cap - 1, cap]
    lens = np.array([min(cap, max(1, int(r.choice(pool)))) for _ in range(B)], np.int32)
    lens[0], lens[-1] = 1, cap
    inp = make_decode_inputs(B, cfg["Hq"], cfg["Hkv"], cap, cfg["d"], cfg["dtype"], seed=3,
                             lens=lens)
    # thresholds that select about half the sequences, one tie (not selected)
    tau = inp.gate + np.where(r.random(B) < 0.5, -0.5, 0.5).astype(np.float32)
    tau[1] = inp.gate[1]
    inp.tau = tau.astype(np.float32)
    say(f"[decode] {name}: lens={lens.tolist()}")
    got = run_decode(cfg, inp, eta=0.05)
    ref = DC.decode_step(inp.q, inp.k, inp.v, inp.lens, inp.gate, inp.tau, cfg["window"],
                         cfg["rho"], 0.05)
    assert np.array_equal(got["selected"], ref["selected"])
    assert got["selected"][1] == 0
    assert np.allclose(got["tau"], ref["tau"], rtol=0, atol=1e-6)
    err = float(np.abs(got["o"] - ref["o"]).max())
    say(f"  selected={got['selected'].tolist()} o max_abs={err:.3e}")
    assert err <= TOL[cfg["dtype"]]


def test_decode_many_sequences():
    """More sequences than the streaming kernel's item table holds: the
    chunked kernel serves the step (bf16), with the same results."""
    cfg = dict(B=1030, Hq=2, Hkv=1, cap=300, d=64, window=40, rho=0.3, dtype="bf16")
    r = np.random.default_rng(11)
    lens = r.integers(1, cfg["cap"] + 1, size=cfg["B"]).astype(np.int32)
    inp = make_decode_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["cap"], cfg["d"], "bf16",
                             seed=5, lens=lens)
    inp.tau = (inp.gate + np.where(r.random(cfg["B"]) < 0.3, -0.5, 0.5)).astype(np.float32)
    say(f"[decode] many sequences B={cfg['B']}")
    got = run_decode(cfg, inp, eta=0.0)
    ref = DC.decode_step(inp.q, inp.k, inp.v, inp.lens, inp.gate, inp.tau, cfg["window"],
                         cfg["rho"], 0.0)
    assert np.array_equal(got["selected"], ref["selected"])
    err = float(np.abs(got["o"] - ref["o"]).max())
    say(f"  o max_abs={err:.3e}")
    assert err <= TOL["bf16"]


def test_decode_is_deterministic_and_tau_accumulates():
    cfg = CASES["bf16_g2_chunks"]
    inp = make_decode_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["cap"], cfg["d"], "bf16",
                             seed=4)
    a = run_decode(cfg, inp, eta=0.1)
    b = run_decode(cfg, inp, eta=0.1)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["tau"], b["tau"])
    want = inp.tau + np.float32(0.1) * (a["selected"].astype(np.float32) - np.float32(0.2))
    assert np.allclose(a["tau"], want, atol=1e-7)


def test_calibrate_and_select_threshold():
    r = np.random.default_rng(8)
    for n in (1, 100, 5000, 40000):
        B = 3
        g = r.standard_normal((B, n)).astype(np.float32)
        if n > 10:
            g[0, :5] = np.nan
            g[1, 3:9] = 0.25                     # ties
        for rho in (0.0, 0.2, 1.0):
            p = T.make_problem(B, 1, 1, n, 64, 1, rho)
            mask, idx, _ = oracle.select_queries(g, rho)
            gt = torch.from_numpy(g).to(dev())
            tau = torch.empty(B, dtype=torch.float32, device=dev())
            T.logo_calibrate_threshold(p, gt, torch.from_numpy(mask).to(dev()), tau)
            torch.cuda.synchronize()
            want = DC.calibrate_threshold(g, rho)
            assert np.array_equal(tau.cpu().numpy(), want), (n, rho)
            m2 = torch.empty((B, n), dtype=torch.uint8, device=dev())
            i2 = torch.empty((B, n), dtype=torch.int32, device=dev())
            c2 = torch.empty(B, dtype=torch.int32, device=dev())
            T.logo_select_threshold(p, gt, tau, m2, i2, c2)
            torch.cuda.synchronize()
            rm, ri, rc = DC.select_threshold(g, want)
            assert np.array_equal(m2.cpu().numpy(), rm), (n, rho)
            assert np.array_equal(i2.cpu().numpy(), ri), (n, rho)
            assert np.array_equal(c2.cpu().numpy(), rc), (n, rho)


def test_decode_full_decode128k():
    cfg = dict(DECODE_WORKLOADS["decode128k"])
    cfg["B"] = 4   # half the benchmark's batch keeps the oracle to seconds
    inp = make_decode_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["cap"], cfg["d"], "bf16",
                             seed=0)
    inp.tau = np.full(cfg["B"], 0.0, np.float32)
    got = run_decode(cfg, inp, eta=0.0)
    ref = DC.decode_step(inp.q, inp.k, inp.v, inp.lens, inp.gate, inp.tau, cfg["window"],
                         cfg["rho"], 0.0)
    assert np.array_equal(got["selected"], ref["selected"])
    err = float(np.abs(got["o"] - ref["o"]).max())
    say(f"[decode full] selected={got['selected'].tolist()} o max_abs={err:.3e}")
    assert err <= TOL["bf16"]
