"""GPU backward (logo_forward_train + logo_backward) against the fp64 oracle.

Saved statistics (lse of both branches, the selected rows' branch outputs)
and the gradients dq, dk, dv, dgate on the same seeded inputs and upstream
gradient. Bound for the gradients (no page states one; derived from the
arithmetic): max |err| <= tol * max(1, max |ref|) per tensor, tol = 2e-2
with bf16 inputs (the forward's bf16 bound; the matrix-core operands P, dS
and g*dout are rounded to bf16, unit roundoff 2^-8 each) and 1e-4 with float32
inputs. Full-size cases check sampled dq rows, dgate at sampled positions,
exact dk/dv of the last keys of each sequence, exact dk/dv of the first 64
keys of one (batch, kv head) (read by every selected row's global branch:
the largest sums; the oracle's rows are spread over a process pool), and sum
rules over all keys."""
import numpy as np
import pytest
import torch

import oracle
import oracle.backward as BW
import token_level_dynamic_amd as T
import oracle_pool as OP
from gpu_util import dev, ensure_built, host, problem, say, to_dev
from workloads import get_workload, make_dout, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
LSE_TOL = {"bf16": 2e-3, "f32": 1e-5}

CASES = {
    "bf16_d128_gqa": ("gqa32k", dict(B=2, Hq=4, Hkv=2, n=700, window=150, rho=0.2)),
    "bf16_d64_mha": ("sweep64k", dict(B=1, Hq=3, Hkv=3, n=555, window=100, rho=0.3)),
    "bf16_group7": ("gqa128k", dict(B=1, Hq=14, Hkv=2, n=300, window=70, rho=0.2)),
    "bf16_window_covers_all": ("gqa32k", dict(B=1, Hq=2, Hkv=2, n=190, window=1000, rho=0.5)),
    "bf16_window_one": ("gqa32k", dict(B=1, Hq=2, Hkv=1, n=130, window=1, rho=0.25)),
    "bf16_rho_zero": ("gqa32k", dict(B=1, Hq=2, Hkv=1, n=257, window=64, rho=0.0)),
    "bf16_rho_one": ("sweep64k", dict(B=1, Hq=2, Hkv=2, n=200, window=33, rho=1.0)),
    "bf16_single_token": ("gqa32k", dict(B=2, Hq=4, Hkv=2, n=1, window=8, rho=1.0)),
    "bf16_unscaled": ("mha4k", dict(Hq=2, Hkv=2, n=400, window=64, qkv_scale=False)),
    "f32_tiny": ("tiny", {}),
    "f32_d128_gqa": ("tiny", dict(B=2, Hq=4, Hkv=2, n=301, d=128, window=45, rho=0.3)),
}


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _dout_dev(w, vals, bits):
    if bits is not None:
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(vals, np.float32)).to(dev())


def run_train(w, inp, dout):
    p = problem(w)
    q, k, v, gate = to_dev(inp)
    fw = T.alloc_train_buffers(p, dev())
    T.logo_forward_train(p, q, k, v, gate, fw["o"], fw["mask"], fw["idx"], fw["rank"],
                         fw["lse_local"], fw["lse_global"], fw["o_local_sel"], fw["o_global"])
    bw = T.alloc_backward_buffers(p, dev())
    T.logo_backward(p, q, k, v, gate, fw["o"], dout, fw["idx"], fw["rank"], fw["lse_local"],
                    fw["lse_global"], fw["o_local_sel"], fw["o_global"], bw["dq"], bw["dk"],
                    bw["dv"], bw["dgate"], bw["workspace"])
    torch.cuda.synchronize()
    return fw, bw


def _err(name, got, ref, tol):
    got = np.asarray(got, np.float64)
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    bound = tol * max(1.0, float(np.abs(ref).max()) if ref.size else 0.0)
    say(f"  {name}: max_abs={err:.3e} bound={bound:.3e} (max |ref| "
        f"{float(np.abs(ref).max()) if ref.size else 0.0:.3e})")
    return err, bound


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_matches_oracle(name):
    base, over = CASES[name]
    w = get_workload(base, **over)
    inp = make_inputs(w, 0)
    dvals, dbits = make_dout(w, 0)
    say(f"[backward] {name}: {w}")
    fw, bw = run_train(w, inp, _dout_dev(w, dvals, dbits))
    st = BW.forward_stats(inp.q, inp.k, inp.v, inp.gate, w.window, w.rho)
    assert np.array_equal(host(fw["idx"]), st["idx"])
    assert np.array_equal(host(fw["rank"]), st["rank"])
    for key in ("lse_local", "lse_global"):
        e, _ = _err(key, host(fw[key]), st[key], 1.0)
        assert e <= LSE_TOL[w.dtype], key
    for key in ("o_local_sel", "o_global"):
        e, _ = _err(key, host(fw[key]), st[key], 1.0)
        assert e <= TOL[w.dtype], key
    ref = BW.backward(inp.q, inp.k, inp.v, inp.gate, dvals, w.window, w.rho)
    e, _ = _err("o", host(fw["o"]), ref["o"], 1.0)
    assert e <= TOL[w.dtype]
    for key in ("dq", "dk", "dv", "dgate"):
        e, bound = _err(key, host(bw[key]), ref[key], TOL[w.dtype])
        assert e <= bound, key


def test_backward_is_deterministic():
    w = get_workload("gqa32k", B=2, Hq=4, Hkv=2, n=900, window=128, rho=0.25)
    inp = make_inputs(w, 3)
    dvals, dbits = make_dout(w, 3)
    dout = _dout_dev(w, dvals, dbits)
    _, a = run_train(w, inp, dout)
    _, b = run_train(w, inp, dout)
    for key in ("dq", "dk", "dv", "dgate"):
        assert torch.equal(a[key], b[key]), key


def test_backward_unselected_dgate_is_zero_and_rho_zero_has_no_global():
    w = get_workload("gqa32k", B=1, Hq=2, Hkv=1, n=333, window=50, rho=0.1)
    inp = make_inputs(w, 5)
    dvals, dbits = make_dout(w, 5)
    fw, bw = run_train(w, inp, _dout_dev(w, dvals, dbits))
    mask = host(fw["mask"]).astype(bool)
    dg = host(bw["dgate"])
    assert np.all(dg[~mask] == 0.0)
    assert np.all(np.isfinite(dg))


def _check_full(w, label):
    inp = make_inputs(w, 0)
    dvals, dbits = make_dout(w, 0)
    say(f"[backward full] {label}: {w}")
    fw, bw = run_train(w, inp, _dout_dev(w, dvals, dbits))
    mask, idx = host(fw["mask"]), host(fw["idx"])
    rm, ri, _ = oracle.select_queries(inp.gate, w.rho)
    assert np.array_equal(mask, rm) and np.array_equal(idx, ri)
    for key in ("dq", "dk", "dv", "dgate"):
        assert bool(torch.isfinite(bw[key]).all()), key
    r = np.random.default_rng(11)
    # dq on sampled rows: band edges, the last rows, selected rows
    rows = []
    for b in range(w.B):
        h0, h1 = 0, w.Hq - 1
        rows += [(b, h0, i) for i in (0, 1, w.window - 1, w.window, w.n - 1)]
        if idx.shape[1]:
            for j in r.choice(idx.shape[1], size=min(6, idx.shape[1]), replace=False):
                rows.append((b, int(r.choice([h0, h1])), int(idx[b, j])))
            rows.append((b, h1, int(idx[b, -1])))
        rows += [(b, int(r.integers(0, w.Hq)), int(r.integers(0, w.n))) for _ in range(4)]
    rows = sorted(set(rows))
    ref = BW.dq_rows(inp.q, inp.k, inp.v, inp.gate, dvals, w.window, w.rho, rows)
    dq = bw["dq"]
    got = np.stack([dq[b, h, i].cpu().numpy() for b, h, i in rows])
    e, bound = _err(f"dq ({len(rows)} rows)", got, ref, TOL[w.dtype])
    assert e <= bound
    # dgate at sampled selected positions (and zero elsewhere)
    pos = []
    for b in range(w.B):
        if idx.shape[1]:
            pos += [(b, int(idx[b, j])) for j in r.choice(idx.shape[1],
                                                          size=min(4, idx.shape[1]),
                                                          replace=False)]
    if pos:
        refg = BW.dgate_at(inp.q, inp.k, inp.v, inp.gate, dvals, w.rho, pos)
        gotg = np.array([float(bw["dgate"][b, i]) for b, i in pos])
        e, bound = _err(f"dgate ({len(pos)} positions)", gotg, refg, TOL[w.dtype])
        assert e <= bound
    dg = host(bw["dgate"])
    assert np.all(dg[mask == 0] == 0.0)
    # exact dk/dv of the last 40 keys of (b, kv head) 0 and the last
    tail = 40
    for b, hk in ((0, 0), (w.B - 1, w.Hkv - 1)):
        rk, rv = BW.dkdv_tail(inp.q, inp.k, inp.v, inp.gate, dvals, w.window, w.rho, b, hk,
                              w.n - tail)
        e, bound = _err(f"dk tail (b={b}, kv={hk})", host(bw["dk"][b, hk, w.n - tail:]), rk,
                        TOL[w.dtype])
        assert e <= bound
        e, bound = _err(f"dv tail (b={b}, kv={hk})", host(bw["dv"][b, hk, w.n - tail:]), rv,
                        TOL[w.dtype])
        assert e <= bound
    # exact dk/dv of the first keys of (b, kv head) 0: every local row whose
    # window reaches them and every selected row, in parts summed here
    head = 64
    b, hk = 0, 0
    pos = sorted(set(range(0, min(w.n, head + w.window - 1))) | {int(i) for i in idx[b]})
    with OP.SharedInputs(q=inp.q, k=inp.k, v=inp.v, gate=inp.gate, do=dvals) as sh:
        parts = OP.map_chunks(sh, "backward.dkdv_keys",
                              lambda c: ("@q", "@k", "@v", "@gate", "@do", w.window, w.rho, b,
                                         hk, 0, head, list(c)),
                              pos, chunk=64)
    rk = sum(x[0] for x in parts)
    rv = sum(x[1] for x in parts)
    e, bound = _err(f"dk first {head} keys (b={b}, kv={hk}, {len(pos)} rows)",
                    host(bw["dk"][b, hk, :head]), rk, TOL[w.dtype])
    assert e <= bound
    e, bound = _err(f"dv first {head} keys (b={b}, kv={hk})", host(bw["dv"][b, hk, :head]), rv,
                    TOL[w.dtype])
    assert e <= bound
    # sum rules over every key of each (b, kv head): sum_j dk_j = 0 and
    # sum_j dv_j = sum over the group's rows of dout_i (1 + [i in S] g_i)
    g = 1.0 / (1.0 + np.exp(-inp.gate.astype(np.float64)))
    wgt = 1.0 + mask * g
    G = w.Hq // w.Hkv
    dk_sum = bw["dk"].double().sum(dim=2).cpu().numpy()   # [B, Hkv, d]
    dv_sum = bw["dv"].double().sum(dim=2).cpu().numpy()
    dk_abs = bw["dk"].double().abs().sum(dim=2).cpu().numpy()
    for b in range(w.B):
        for hk in range(w.Hkv):
            grp = dvals[b, hk * G:(hk + 1) * G].astype(np.float64)       # [G, n, d]
            want = (grp * wgt[b][None, :, None]).sum(axis=(0, 1))
            mass = (np.abs(grp) * wgt[b][None, :, None]).sum(axis=(0, 1))
            assert np.all(np.abs(dv_sum[b, hk] - want) <= 1e-3 * mass), (b, hk)
            assert np.all(np.abs(dk_sum[b, hk]) <= 1e-3 * dk_abs[b, hk] + 1e-6), (b, hk)
    say(f"  sum rules: max |sum dv - want| / mass and |sum dk| / sum |dk| within 1e-3")


def test_backward_full_gqa32k():
    _check_full(get_workload("gqa32k"), "gqa32k")


def test_backward_full_sweep64k_rho02():
    _check_full(get_workload("sweep64k", rho=0.2), "sweep64k rho=0.2")
