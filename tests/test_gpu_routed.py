"""GPU routed forward (logo_forward_routed: local branch, router logits from
its output, selection, global branch, combine) against the oracle, which
computes everything from the inputs on its own: float64 logits, a selection
on their float32 rounding, and the combine with the sigmoid of the float64
logits ("Learning When to Attend", The Architecture of Conditional Attention:
local attention first, then one routing decision per token).

A logit is a sum over heads of <w_h, o_local row>; the device rounds the
softmax weights to bf16 before the P V product and accumulates in float32.
``routed_bound`` turns the exact weights of each local row into a tolerance
m_i on |device logit - float64 logit| (probabilistic rounding-error model,
lam = 8: a correct device exceeds it with probability below 1e-13 per
position), and the rounding of the float64 logit to float32.

Selection: with the oracle's float32 logits g, its selected set O,
U = max over i outside O of g_i + m_i and L = min over i in O of g_i - m_i,
a correct device selection on logits within m_i of g contains every i with
g_i - m_i > U (its (k+1)-th largest logit is at most U) and no i with
g_i + m_i < L (its k-th largest is at least L). Those positions are compared
bit for bit;
the device's choice in the band between them is checked for validity (the k
largest of its own logits, ties to the lower position). Outputs are compared
on the rows where both selections agree, at 2e-2 (bf16) or 1e-4 (float32),
plus, on selected rows, the sigmoid's share of the logit tolerance:
0.25 m_i max|o_global row| (the sigmoid's slope is at most 1/4)."""
import numpy as np
import pytest
import torch

import oracle.router as RO
import oracle_pool as OP
import routed_bound as RB
import token_level_dynamic_amd as T
from gpu_util import dev, ensure_built, gather_rows, host, parity_rows, problem, say, to_dev
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


def logit_bound(w, inp, rw):
    """Tolerance m [B, n] on |device logit - oracle logit| (routed_bound)."""
    pos = [(b, i) for b in range(w.B) for i in range(w.n)]
    sc = RB.logit_error_scales(inp.q, inp.k, inp.v, rw, w.window, pos)
    return RB.logit_bound(sc, w.dtype).reshape(w.B, w.n)


def band_bound(m, g):
    """|device logit - oracle float32 logit| <= m + the float32 rounding."""
    return m + 2.0 ** -24 * np.abs(g)


def check_selection(gdev, mask, idx, rank, g32, rmask, m, k):
    """The device selection is valid for its own logits and equals the
    oracle's outside the band the logit bound leaves open. Returns the number
    of positions where the two differ."""
    B, n = g32.shape
    ndiff = 0
    for b in range(B):
        sel = mask[b].astype(bool)
        assert sel.sum() == k
        assert np.array_equal(idx[b], np.flatnonzero(sel))
        assert np.array_equal(rank[b][idx[b]], np.arange(k))
        assert np.all(rank[b][~sel] == -1)
        if 0 < k < n:
            # the k largest device logits, ties to the lower position
            lo_in = gdev[b][sel].min()
            assert not np.any(gdev[b][~sel] > lo_in)
            ties_out = np.flatnonzero(~sel & (gdev[b] == lo_in))
            ties_in = np.flatnonzero(sel & (gdev[b] == lo_in))
            assert ties_out.size == 0 or ties_in.max() < ties_out.min()
            # U bounds the device's (k+1)-th largest logit from above: some
            # position of its top k+1 lies outside the oracle's top k; L
            # bounds its k-th largest from below (the oracle's top k)
            gb, mb = g32[b].astype(np.float64), m[b]
            top = rmask[b].astype(bool)
            U = (gb + mb)[~top].max()
            L = (gb - mb)[top].min()
            must_in = gb - mb > U
            must_out = gb + mb < L
            assert np.all(sel[must_in]) and not np.any(sel[must_out])
            assert np.all(top[must_in]) and not np.any(top[must_out])
            band = ~(must_in | must_out)
            assert np.array_equal(sel[~band], rmask[b][~band].astype(bool))
            ndiff += int((sel != rmask[b].astype(bool)).sum())
        else:
            assert np.array_equal(sel, rmask[b].astype(bool))
    return ndiff


@pytest.mark.parametrize("name", sorted(CASES))
def test_routed_matches_oracle(name):
    base, over = CASES[name]
    w = get_workload(base, **over)
    inp = make_inputs(w, 0)
    rw, rb = make_router(w, 0)
    say(f"[routed] {name}: {w}")
    got = run_routed(w, inp, rw, rb)
    ref = RO.forward_routed(inp.q, inp.k, inp.v, rw, rb, w.window, w.rho)
    gdev = host(got["gate"])
    m = logit_bound(w, inp, rw)
    gerr = np.abs(gdev.astype(np.float64) - ref["gate"])
    say(f"  gate max_abs={gerr.max():.3e} max bound={m.max():.3e} "
        f"worst err/bound={(gerr / m).max():.3f}")
    assert np.all(gerr <= m)
    k = T.logo_target_count(w.rho, w.n)
    mask, idx, rank = host(got["mask"]), host(got["idx"]), host(got["rank"])
    ndiff = check_selection(gdev, mask, idx, rank, ref["gate32"], ref["mask"],
                            band_bound(m, ref["gate"]), k)
    say(f"  selection: {ndiff} positions differ from the oracle's, all inside the bound's band")
    o = host(got["o"]).astype(np.float64)
    agree = mask == ref["mask"]                                     # [B, n]
    err = np.abs(o - ref["o"])                                      # [B, Hq, n, d]
    tol = np.full((w.B, w.Hq, w.n), TOL[w.dtype])
    for b in range(w.B):
        for r, i in enumerate(ref["idx"][b]):
            og = np.abs(ref["o_global"][b, :, r]).max(axis=-1)      # [Hq]
            tol[b, :, i] += 0.25 * m[b, i] * og
    ok = err.max(axis=-1) <= tol
    assert np.all(ok[np.broadcast_to(agree[:, None, :], ok.shape)])
    say(f"  o max_abs={err.max(axis=-1)[np.broadcast_to(agree[:, None, :], ok.shape)].max():.3e} "
        f"on the rows both selections agree on")


def test_routed_is_deterministic():
    w = get_workload("gqa32k", B=2, Hq=4, Hkv=2, n=900, window=128, rho=0.25)
    inp = make_inputs(w, 2)
    rw, rb = make_router(w, 2)
    a = run_routed(w, inp, rw, rb)
    b = run_routed(w, inp, rw, rb)
    for key in ("gate", "o", "idx"):
        assert torch.equal(a[key], b[key]), key


def test_routed_full_gqa32k():
    """The headline layer: the oracle's logits and their tolerances for every
    position (a process pool), the selection checked as above, and the output
    rows of the parity subset on which both selections agree."""
    w = get_workload("gqa32k")
    inp = make_inputs(w, 0)
    rw, rb = make_router(w, 0)
    say(f"[routed full] {w}")
    got = run_routed(w, inp, rw, rb)
    gdev = host(got["gate"])
    mask, idx, rank = host(got["mask"]), host(got["idx"]), host(got["rank"])
    o_dev = got["o"]
    del got
    assert np.all(np.isfinite(gdev))
    import oracle
    positions = [(b, i) for b in range(w.B) for i in range(w.n)]
    with OP.SharedInputs(q=inp.q, k=inp.k, v=inp.v, w=rw) as sh:
        parts = OP.map_chunks(sh, "router.router_logits_at",
                              lambda c: ("@q", "@k", "@v", "@w", rb, w.window, list(c)),
                              positions, chunk=512)
        g = np.concatenate(parts).reshape(w.B, w.n)
        parts = OP.map_chunks(sh, "routed_bound.logit_error_scales",
                              lambda c: ("@q", "@k", "@v", "@w", w.window, list(c)),
                              positions, chunk=512)
        m = RB.logit_bound(np.concatenate(parts), w.dtype).reshape(w.B, w.n)
        g32 = g.astype(np.float32)
        rmask, ridx, _ = oracle.select_queries(g32, w.rho)
        gerr = np.abs(gdev.astype(np.float64) - g)
        say(f"  gate max_abs={gerr.max():.3e} max bound={m.max():.3e} "
            f"worst err/bound={(gerr / m).max():.3f}")
        assert np.all(gerr <= m)
        k = T.logo_target_count(w.rho, w.n)
        ndiff = check_selection(gdev, mask, idx, rank, g32, rmask, band_bound(m, g), k)
        say(f"  selection: {ndiff} of {w.B * w.n} positions differ, all inside the band")
        rows = [r for r in parity_rows(w, ridx, seed=5) if mask[r[0], r[2]] == rmask[r[0], r[2]]]
        sh.add(gate=g)
        # oracle.forward_rows selects on the float32 rounding of the logits
        # it is given and squashes them as given: the routed oracle's rows
        parts = OP.map_chunks(sh, "oracle.forward_rows",
                              lambda c: ("@q", "@k", "@v", "@gate", w.window, w.rho, list(c)),
                              rows, chunk=64)
    ref = np.concatenate([p["o_rows"] for p in parts])
    vals = gather_rows(o_dev, rows)
    err = np.abs(vals - ref).max(axis=-1)
    # the sigmoid's share: |o_global| is at most the largest |v| of the head
    vmax = np.abs(inp.v).max(axis=(2, 3))                       # [B, Hkv]
    G = w.Hq // w.Hkv
    tol = np.array([TOL[w.dtype] + (0.25 * m[b, i] * vmax[b, h // G] if rmask[b, i] else 0.0)
                    for b, h, i in rows])
    say(f"  o ({len(rows)} rows) max_abs={err.max():.3e}")
    assert np.all(err <= tol)
