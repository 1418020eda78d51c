"""GPU forward over packed variable-length batches (logo_forward_varlen)
against the oracle (``oracle/varlen.py``): selection bit-exact per example,
outputs within 2e-2 (bf16) or 1e-4 (float32)."""
import numpy as np
import pytest
import torch

import oracle
import oracle.varlen as VL
import token_level_dynamic_amd as T
from gpu_util import dev, ensure_built, global_splits, say, single_launch
from workloads import VARLEN_WORKLOADS, make_varlen_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _io(x, bits, dtype):
    if dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev())


def run_varlen(inp, Hq, Hkv, d, window, rho, dtype, token_major=False):
    Tn = int(inp["cu"][-1])
    q = _io(inp["q"], inp["bits"].get("q"), dtype)[None]
    k = _io(inp["k"], inp["bits"].get("k"), dtype)[None]
    v = _io(inp["v"], inp["bits"].get("v"), dtype)[None]
    kw = {}
    if token_major:   # [T][H][d] storage seen as [1][H][T][d] views
        q = q[0].permute(1, 0, 2).contiguous().permute(1, 0, 2)[None]
        k = k[0].permute(1, 0, 2).contiguous().permute(1, 0, 2)[None]
        v = v[0].permute(1, 0, 2).contiguous().permute(1, 0, 2)[None]
        kw = dict(q_strides=T.view_strides(q), k_strides=T.view_strides(k),
                  v_strides=T.view_strides(v))
    p = T.make_problem(1, Hq, Hkv, Tn, d, window, rho, dtype=dtype, **kw)
    K = T.logo_varlen_selected_count(rho, inp["cu"])
    cu = torch.from_numpy(inp["cu"]).to(dev())
    gate = torch.from_numpy(inp["gate"]).to(dev())
    o = torch.empty((1, Hq, Tn, d), dtype=T.io_dtype(p), device=dev())
    mask = torch.empty(Tn, dtype=torch.uint8, device=dev())
    idx = torch.full((K,), -5, dtype=torch.int32, device=dev())
    rank = torch.empty(Tn, dtype=torch.int32, device=dev())
    ws = torch.empty(T.logo_varlen_workspace_size(p, cu.numel() - 1, K), dtype=torch.uint8,
                     device=dev())
    T.logo_forward_varlen(p, cu, K, q, k, v, gate, o, mask, idx, rank, ws)
    torch.cuda.synchronize()
    return {"o": o[0].float().cpu().numpy(), "mask": mask.cpu().numpy(),
            "idx": idx.cpu().numpy(), "rank": rank.cpu().numpy(), "o_dev": o}


CASES = {
    "bf16_mix": (dict(lens=[1, 31, 32, 33, 500, 64, 2, 200], Hq=4, Hkv=2, d=128, window=100,
                      rho=0.25, dtype="bf16"), False),
    "bf16_empty_and_long": (dict(lens=[0, 700, 0, 65, 1], Hq=2, Hkv=1, d=64, window=64, rho=0.5,
                                 dtype="bf16"), False),
    "bf16_token_major": (dict(lens=[120, 7, 300], Hq=4, Hkv=2, d=128, window=40, rho=0.3,
                              dtype="bf16"), True),
    "bf16_window_covers": (dict(lens=[90, 150, 33], Hq=3, Hkv=3, d=64, window=1000, rho=0.2,
                                dtype="bf16"), False),
    "f32_mix": (dict(lens=[5, 250, 1, 64], Hq=2, Hkv=1, d=64, window=32, rho=0.25,
                     dtype="f32"), False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_varlen_matches_oracle(name):
    cfg, tm = CASES[name]
    inp = make_varlen_inputs(cfg["lens"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["dtype"], seed=1)
    say(f"[varlen] {name}: lens={cfg['lens']}")
    got = run_varlen(inp, cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["window"], cfg["rho"],
                     cfg["dtype"], token_major=tm)
    ref = VL.forward_varlen(inp["q"], inp["k"], inp["v"], inp["gate"], inp["cu"], cfg["window"],
                            cfg["rho"])
    assert np.array_equal(got["mask"], ref["mask"])
    assert np.array_equal(got["idx"], ref["idx"])
    assert np.array_equal(got["rank"], ref["rank"])
    err = float(np.abs(got["o"] - ref["o"]).max())
    say(f"  K={ref['idx'].size} o max_abs={err:.3e}")
    assert err <= TOL[cfg["dtype"]]


def test_single_example_equals_forward():
    """One example: the same arithmetic as logo_forward, bit for bit, except
    where logo_forward splits a small problem's global branch into key
    ranges (probabilities rounded against each range's maximum): then the
    two agree to the parity tolerance."""
    Hq, Hkv, d, n, W, rho = 4, 2, 128, 777, 90, 0.2
    inp = make_varlen_inputs([n], Hq, Hkv, d, "bf16", seed=2)
    got = run_varlen(inp, Hq, Hkv, d, W, rho, "bf16")
    p = T.make_problem(1, Hq, Hkv, n, d, W, rho)
    buf = T.alloc_forward_buffers(p, dev())
    q = _io(None, inp["bits"]["q"], "bf16")[None]
    k = _io(None, inp["bits"]["k"], "bf16")[None]
    v = _io(None, inp["bits"]["v"], "bf16")[None]
    g = torch.from_numpy(inp["gate"]).to(dev())[None]
    T.logo_forward(p, q, k, v, g, buf["o"], buf["mask"], buf["idx"], buf["rank"],
                   buf["workspace"])
    torch.cuda.synchronize()
    if global_splits(p) or single_launch(p):
        err = float((got["o_dev"].float() - buf["o"].float()).abs().max())
        say(f"  split or single-launch forward vs packed max_abs={err:.3e}")
        assert err <= TOL["bf16"]
    else:
        assert torch.equal(got["o_dev"].view(torch.int16), buf["o"].view(torch.int16))
    assert np.array_equal(got["idx"], buf["idx"][0].cpu().numpy())


def test_varlen_full_64k():
    cfg = VARLEN_WORKLOADS["varlen64k"]
    inp = make_varlen_inputs(cfg["lens"], cfg["Hq"], cfg["Hkv"], cfg["d"], "bf16", seed=0)
    say(f"[varlen full] lens={cfg['lens']}")
    got = run_varlen(inp, cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["window"], cfg["rho"], "bf16")
    cu = inp["cu"]
    r = np.random.default_rng(3)
    worst = 0.0
    for e in range(len(cfg["lens"])):
        a, b = int(cu[e]), int(cu[e + 1])
        g = inp["gate"][a:b][None]
        rm, ri, rr = oracle.select_queries(g, cfg["rho"])
        assert np.array_equal(got["mask"][a:b], rm[0]), e
        sel = got["idx"][(got["idx"] >= a) & (got["idx"] < b)] - a
        assert np.array_equal(sel, ri[0]), e
        rows = [(0, h, i) for h in (0, cfg["Hq"] - 1)
                for i in sorted({0, 1, min(b - a - 1, cfg["window"]), b - a - 1})]
        if ri.shape[1]:
            rows += [(0, int(r.integers(0, cfg["Hq"])), int(ri[0, j]))
                     for j in r.choice(ri.shape[1], min(4, ri.shape[1]), replace=False)]
        rows = sorted(set(rows))
        ref = oracle.forward_rows(inp["q"][None, :, a:b], inp["k"][None, :, a:b],
                                  inp["v"][None, :, a:b], g, cfg["window"], cfg["rho"], rows)
        vals = np.stack([got["o"][h, a + i] for _, h, i in rows])
        worst = max(worst, float(np.abs(vals - ref["o_rows"]).max()))
    say(f"  sampled rows max_abs={worst:.3e}")
    assert worst <= TOL["bf16"]
