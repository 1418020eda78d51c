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


def _takes_single_launch(Hq, Hkv, d, Tn, K, dtype):
    """logo_forward_varlen's single launch applies as logo_forward's does
    (include/logo.h): bf16, d in {64, 128}, something selected, no key-range
    split (512 or more row-block workgroups, or too few keys to split), and
    Hkv a multiple or a divisor of 8."""
    if dtype != "bf16" or K == 0 or d not in (64, 128):
        return False
    wg = Hkv * -(-(-(-K // 32) * (Hq // Hkv)) // 4)
    if wg < 512 and min(8, -(-512 // wg), (-(-Tn // 64)) // 4) >= 2:
        return False
    return Hkv % 8 == 0 or 8 % Hkv == 0


# Packed streams that take the single launch: every row of three query heads
# of every example is compared with the oracle (run per example, as the
# sequences they are), so example starts inside row blocks, inside tiles and
# inside a selected row's window all occur, with empty and one-token examples.
SINGLE = {
    "single_d128": dict(lens=[3001, 1, 700, 0, 64, 2500, 33, 1900, 2, 1999], Hq=32, Hkv=8,
                        d=128, window=500, rho=0.2),
    "single_d64": dict(lens=[4095, 7, 1, 2100, 1, 129, 1800], Hq=16, Hkv=16, d=64,
                       window=300, rho=0.5),
}


@pytest.mark.parametrize("name", sorted(SINGLE))
def test_varlen_single_launch_matches_oracle(name):
    import oracle_pool as OP
    cfg = SINGLE[name]
    inp = make_varlen_inputs(cfg["lens"], cfg["Hq"], cfg["Hkv"], cfg["d"], "bf16", seed=4)
    cu = inp["cu"]
    Tn = int(cu[-1])
    K = T.logo_varlen_selected_count(cfg["rho"], cu)
    assert _takes_single_launch(cfg["Hq"], cfg["Hkv"], cfg["d"], Tn, K, "bf16")
    say(f"[varlen single] {name}: lens={cfg['lens']} K={K}")
    got = run_varlen(inp, cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["window"], cfg["rho"], "bf16")
    G = cfg["Hq"] // cfg["Hkv"]
    heads = sorted({0, G - 1, cfg["Hq"] - 1})
    worst = 0.0
    for e in range(len(cfg["lens"])):
        a, b = int(cu[e]), int(cu[e + 1])
        if b == a:
            continue
        g = np.ascontiguousarray(inp["gate"][a:b][None])
        rm, ri, _ = oracle.select_queries(g, cfg["rho"])
        assert np.array_equal(got["mask"][a:b], rm[0]), e
        sel = got["idx"][(got["idx"] >= a) & (got["idx"] < b)] - a
        assert np.array_equal(sel, ri[0]), e
        rows = [(0, h, i) for h in heads for i in range(b - a)]
        with OP.SharedInputs(q=np.ascontiguousarray(inp["q"][None, :, a:b]),
                             k=np.ascontiguousarray(inp["k"][None, :, a:b]),
                             v=np.ascontiguousarray(inp["v"][None, :, a:b]), gate=g) as sh:
            parts = OP.map_chunks(sh, "oracle.forward_rows",
                                  lambda c: ("@q", "@k", "@v", "@gate", cfg["window"],
                                             cfg["rho"], list(c)), rows, chunk=256)
        ref = np.concatenate([x["o_rows"] for x in parts])
        vals = np.stack([got["o"][h, a + i] for _, h, i in rows])
        worst = max(worst, float(np.abs(vals - ref).max()))
    say(f"  {len(heads)} heads x {Tn} tokens, max_abs={worst:.3e}")
    assert worst <= TOL["bf16"]
