"""Full-size workloads, in the launch configuration the benchmark times
(logo_forward). The oracle recomputes the whole selection (bit-exact
mask/idx/rank) and the output rows of a fixed subset one by one, in a
process pool: every position of the band edge (0 .. W + 64), the last 256
positions, every selected position in three 2048-position windows (start,
middle, end), a seeded 1 % of positions, for all query heads of kv group 0,
plus the 1 % sample on random heads of the whole layer. The 4K multi-head
workload is compared in full."""
import numpy as np
import pytest
import torch

import oracle
import token_level_dynamic_amd as T
import oracle_pool as OP
from gpu_util import ensure_built, gather_rows, host, parity_rows, problem, run_forward, say, to_dev
from workloads import SWEEP_RHOS, get_workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _check_full(w, inp, label):
    say(f"[full] {label}: {w}")
    p = problem(w)
    q, k, v, gate = to_dev(inp)
    got = run_forward(p, q, k, v, gate)
    del q, k, v
    kk = T.logo_target_count(w.rho, w.n)
    mask, idx, rank = host(got["mask"]), host(got["idx"]), host(got["rank"])
    # properties that hold at any size
    assert (mask.sum(axis=1) == kk).all()
    for b in range(w.B):
        assert np.all(np.diff(idx[b]) > 0)
        assert np.array_equal(rank[b][idx[b]], np.arange(kk))
    assert bool(torch.isfinite(got["o"]).all())
    # selection: the oracle's, bit for bit
    rm, ri, rr = oracle.select_queries(inp.gate, w.rho)
    assert np.array_equal(mask, rm) and np.array_equal(idx, ri) and np.array_equal(rank, rr)
    rows = parity_rows(w, ri, seed=7)
    with OP.SharedInputs(q=inp.q, k=inp.k, v=inp.v, gate=inp.gate) as sh:
        parts = OP.map_chunks(sh, "oracle.forward_rows",
                              lambda c: ("@q", "@k", "@v", "@gate", w.window, w.rho, list(c)),
                              rows, chunk=48)
    ref = np.concatenate([x["o_rows"] for x in parts])
    vals = gather_rows(got["o"], rows)
    err = np.abs(vals - ref)
    nsel = sum(int(mask[b, i]) for b, _, i in rows)
    say(f"  {len(rows)} rows ({nsel} selected), max_abs={err.max():.3e} "
        f"(max |o| {np.abs(ref).max():.3e}, rms err {np.sqrt((err ** 2).mean()):.2e})")
    assert err.max() <= TOL[w.dtype]


def test_mha4k_full_layer():
    w = get_workload("mha4k")
    inp = make_inputs(w, 0)
    say(f"[full] mha4k whole layer: {w}")
    q, k, v, gate = to_dev(inp)
    got = run_forward(problem(w), q, k, v, gate)
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.gate, w.window, w.rho)
    assert np.array_equal(host(got["idx"]), ref["idx"])
    o = host(got["o"])
    err = np.abs(o - ref["o"])
    say(f"  max_abs={err.max():.3e} rel={err.max() / np.abs(ref['o']).max():.3e}")
    assert err.max() <= TOL["bf16"]
    # the same shape with unscaled N(0,1) entries (outputs of order 0.1-1)
    w2 = w.with_(qkv_scale=False)
    inp2 = make_inputs(w2, 0)
    q, k, v, gate = to_dev(inp2)
    got2 = run_forward(problem(w2), q, k, v, gate)
    ref2 = oracle.forward(inp2.q, inp2.k, inp2.v, inp2.gate, w2.window, w2.rho)
    err2 = np.abs(host(got2["o"]) - ref2["o"])
    say(f"  unscaled: max_abs={err2.max():.3e}")
    assert err2.max() <= TOL["bf16"]


def test_tiny_full_layer():
    w = get_workload("tiny")
    for seed in range(4):
        inp = make_inputs(w, seed)
        q, k, v, gate = to_dev(inp)
        got = run_forward(problem(w), q, k, v, gate)
        ref = oracle.forward(inp.q, inp.k, inp.v, inp.gate, w.window, w.rho)
        assert np.array_equal(host(got["idx"]), ref["idx"])
        err = np.abs(host(got["o"]) - ref["o"]).max()
        say(f"[full] tiny seed {seed}: max_abs={err:.3e}")
        assert err <= TOL["f32"]


def test_gqa32k_headline():
    w = get_workload("gqa32k")
    _check_full(w, make_inputs(w, 0), "gqa32k")


def test_gqa128k():
    w = get_workload("gqa128k")
    _check_full(w, make_inputs(w, 0), "gqa128k")


@pytest.mark.parametrize("rho", SWEEP_RHOS)
def test_sweep64k(rho):
    w = get_workload("sweep64k", rho=rho)
    _check_full(w, make_inputs(w, 0), f"sweep64k rho={rho}")
