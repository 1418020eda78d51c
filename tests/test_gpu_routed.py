"""GPU routed forward (logo_forward_routed: local branch, router logits from
its output, selection, global branch, combine) against the oracle.

The selection is decided by float32 logits on both sides: the oracle selects
on the GPU's logits (bit-exact mask/idx/rank), and the logits themselves are
compared with the oracle's fp64 ones, within 2e-2 (bf16 inputs) or 1e-4
(float32) times max(1, max |logit|): each logit is a sum of Hq*d products
of the local output, whose own error bound is the forward's."""
import numpy as np
import pytest
import torch

import oracle
import oracle.router as RO
import token_level_dynamic_amd as T
from gpu_util import dev, ensure_built, host, problem, say, to_dev
from workloads import get_workload, make_inputs, make_router

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
CASES = {
    "bf16_d128_gqa": ("gqa32k", dict(B=2, Hq=4, Hkv=2, n=700, window=150, rho=0.2)),
    "bf16_d64_mha": ("sweep64k", dict(B=1, Hq=3, Hkv=3, n=555, window=100, rho=0.3)),
    "bf16_group7": ("gqa128k", dict(B=1, Hq=14, Hkv=2, n=300, window=70, rho=0.2)),
    "bf16_rho_zero": ("gqa32k", dict(B=1, Hq=2, Hkv=1, n=257, window=64, rho=0.0)),
    "bf16_rho_one": ("sweep64k", dict(B=1, Hq=2, Hkv=2, n=200, window=33, rho=1.0)),
    "bf16_single_token": ("gqa32k", dict(B=2, Hq=4, Hkv=2, n=1, window=8, rho=1.0)),
    "f32_tiny": ("tiny", {}),
    "f32_d128_gqa": ("tiny", dict(B=2, Hq=4, Hkv=2, n=301, d=128, window=45, rho=0.3)),
}


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def run_routed(w, inp, rw, rb):
    p = problem(w)
    q, k, v, _ = to_dev(inp)
    buf = T.alloc_routed_buffers(p, dev())
    wt = torch.from_numpy(rw).to(dev())
    T.logo_forward_routed(p, q, k, v, wt, rb, buf["gate"], buf["o"], buf["mask"], buf["idx"],
                          buf["rank"], buf["workspace"])
    torch.cuda.synchronize()
    return buf


@pytest.mark.parametrize("name", sorted(CASES))
def test_routed_matches_oracle(name):
    base, over = CASES[name]
    w = get_workload(base, **over)
    inp = make_inputs(w, 0)
    rw, rb = make_router(w, 0)
    say(f"[routed] {name}: {w}")
    got = run_routed(w, inp, rw, rb)
    gate = host(got["gate"])
    ref = RO.forward_routed(inp.q, inp.k, inp.v, rw, rb, w.window, w.rho, gate_used=gate)
    gerr = float(np.abs(gate - ref["gate"]).max())
    gbound = TOL[w.dtype] * max(1.0, float(np.abs(ref["gate"]).max()))
    say(f"  gate max_abs={gerr:.3e} bound={gbound:.3e}")
    assert gerr <= gbound
    assert np.array_equal(host(got["mask"]), ref["mask"])
    assert np.array_equal(host(got["idx"]), ref["idx"])
    assert np.array_equal(host(got["rank"]), ref["rank"])
    err = float(np.abs(host(got["o"]) - ref["o"]).max())
    say(f"  o max_abs={err:.3e}")
    assert err <= TOL[w.dtype]


def test_routed_is_deterministic():
    w = get_workload("gqa32k", B=2, Hq=4, Hkv=2, n=900, window=128, rho=0.25)
    inp = make_inputs(w, 2)
    rw, rb = make_router(w, 2)
    a = run_routed(w, inp, rw, rb)
    b = run_routed(w, inp, rw, rb)
    for key in ("gate", "o", "idx"):
        assert torch.equal(a[key], b[key]), key


def test_routed_full_gqa32k():
    w = get_workload("gqa32k")
    inp = make_inputs(w, 0)
    rw, rb = make_router(w, 0)
    say(f"[routed full] {w}")
    got = run_routed(w, inp, rw, rb)
    gate = host(got["gate"])
    assert np.all(np.isfinite(gate))
    # selection: the oracle's on the GPU logits, bit for bit
    rm, ri, rr = oracle.select_queries(gate, w.rho)
    assert np.array_equal(host(got["mask"]), rm) and np.array_equal(host(got["idx"]), ri)
    assert np.array_equal(host(got["rank"]), rr)
    r = np.random.default_rng(5)
    pos = [(b, int(i)) for b in range(w.B) for i in (0, 1, w.window - 1, w.n - 1)]
    pos += [(b, int(ri[b, j])) for b in range(w.B) for j in r.choice(ri.shape[1], 3, False)]
    pos += [(int(r.integers(0, w.B)), int(r.integers(0, w.n))) for _ in range(4)]
    refg = RO.router_logits_at(inp.q, inp.k, inp.v, rw, rb, w.window, pos)
    gotg = np.array([gate[b, i] for b, i in pos])
    gerr = float(np.abs(gotg - refg).max())
    gbound = TOL[w.dtype] * max(1.0, float(np.abs(refg).max()))
    say(f"  gate ({len(pos)} positions) max_abs={gerr:.3e} bound={gbound:.3e}")
    assert gerr <= gbound
    rows = []
    for b in range(w.B):
        rows += [(b, 0, i) for i in (0, 1, w.window - 1, w.window, w.n - 1)]
        rows += [(b, int(r.integers(0, w.Hq)), int(ri[b, j]))
                 for j in r.choice(ri.shape[1], 8, False)]
        rows += [(b, w.Hq - 1, int(ri[b, -1]))]
    rows = sorted(set(rows))
    ref = oracle.forward_rows(inp.q, inp.k, inp.v, gate, w.window, w.rho, rows)
    o = got["o"]
    vals = np.stack([o[b, h, i].float().cpu().numpy() for b, h, i in rows])
    err = float(np.abs(vals - ref["o_rows"]).max())
    say(f"  o ({len(rows)} rows) max_abs={err:.3e}")
    assert err <= TOL[w.dtype]
