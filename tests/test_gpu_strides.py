"""Strided q/k/v/o views through the C ABI: token-major [B][n][H][d] storage,
K and V as the two halves of one fused buffer, padded token rows, and K/V
broadcast over the batch (batch stride 0). Every strided run must equal the
contiguous run bit for bit (the kernels do the same arithmetic in the same
order) and the oracle within the usual tolerance, and must not write outside
the output view."""
import numpy as np
import pytest
import torch

import oracle
import token_level_dynamic_amd as T
from gpu_util import dev, ensure_built, host, problem, run_forward, run_unfused, say, to_dev
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
SENTINEL = 7.0

CASES = {
    "bf16_d128_gqa": ("gqa32k", dict(B=2, Hq=4, Hkv=2, n=1000, window=200, rho=0.2)),
    "bf16_d64_mha": ("sweep64k", dict(B=2, Hq=3, Hkv=3, n=777, window=100, rho=0.3)),
    "f32_d128_gqa": ("tiny", dict(B=2, Hq=4, Hkv=2, n=301, d=128, window=45, rho=0.3)),
}
LAYOUTS = ["token_major", "fused_kv", "padded", "kv_batch_broadcast"]


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _token_major(x):
    """[B][H][n][d] view of a [B][n][H][d] copy of x."""
    s = torch.empty((x.shape[0], x.shape[2], x.shape[1], x.shape[3]), dtype=x.dtype,
                    device=x.device)
    s.copy_(x.permute(0, 2, 1, 3))
    return s.permute(0, 2, 1, 3)


def _padded(x, pad):
    s = torch.full(x.shape[:3] + (x.shape[3] + pad,), SENTINEL, dtype=x.dtype, device=x.device)
    s[..., : x.shape[3]].copy_(x)
    return s[..., : x.shape[3]]


def _fused_kv(k, v):
    B, H, n, d = k.shape
    s = torch.empty((B, n, 2, H, d), dtype=k.dtype, device=k.device)
    s[:, :, 0].copy_(k.permute(0, 2, 1, 3))
    s[:, :, 1].copy_(v.permute(0, 2, 1, 3))
    return s[:, :, 0].permute(0, 2, 1, 3), s[:, :, 1].permute(0, 2, 1, 3)


def _views(layout, q, k, v, w):
    """Strided q, k, v and an output view o (filled with a sentinel), plus the
    storage that backs o so that the test can check what lies outside it."""
    pad = 8 if w.dtype == "bf16" else 4
    if layout == "token_major":
        qv, kv_, vv = _token_major(q), _token_major(k), _token_major(v)
        o_store = torch.full((w.B, w.n, w.Hq, w.d), SENTINEL, dtype=q.dtype, device=q.device)
        ov = o_store.permute(0, 2, 1, 3)
    elif layout == "fused_kv":
        qv = q
        kv_, vv = _fused_kv(k, v)
        o_store = torch.full((w.B, w.Hq, w.n, w.d + pad), SENTINEL, dtype=q.dtype,
                             device=q.device)
        ov = o_store[..., : w.d]
    elif layout == "padded":
        qv, kv_, vv = _padded(q, pad), _padded(k, 2 * pad), _padded(v, pad)
        o_store = torch.full((w.B, w.Hq, w.n, w.d + pad), SENTINEL, dtype=q.dtype,
                             device=q.device)
        ov = o_store[..., : w.d]
    elif layout == "kv_batch_broadcast":
        qv = q
        kv_ = k[:1].expand(w.B, -1, -1, -1)
        vv = v[:1].expand(w.B, -1, -1, -1)
        o_store = torch.full((w.B, w.n, w.Hq, w.d), SENTINEL, dtype=q.dtype, device=q.device)
        ov = o_store.permute(0, 2, 1, 3)
    else:
        raise ValueError(layout)
    return qv, kv_, vv, ov, o_store


def _strided_problem(w, qv, kv_, vv, ov):
    return T.make_problem(w.B, w.Hq, w.Hkv, w.n, w.d, w.window, w.rho, dtype=w.dtype,
                          q_strides=T.view_strides(qv), k_strides=T.view_strides(kv_),
                          v_strides=T.view_strides(vv), o_strides=T.view_strides(ov))


def _outside_untouched(o_store, ov):
    """Every element of the backing storage that the view does not cover
    still holds the sentinel."""
    inside = torch.zeros(o_store.shape, dtype=torch.bool, device=o_store.device)
    if ov.data_ptr() == o_store.data_ptr() and ov.shape != o_store.shape:
        inside[..., : ov.shape[3]] = True
    else:
        inside[...] = True
    out = o_store[~inside]
    return bool((out.float() == SENTINEL).all()) if out.numel() else True


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("name", sorted(CASES))
def test_strided_views(name, layout):
    base, over = CASES[name]
    w = get_workload(base, **over)
    inp = make_inputs(w, 0)
    q, k, v, gate = to_dev(inp)
    if layout == "kv_batch_broadcast":
        # every batch row reads batch 0's K and V
        k = k[:1].expand(w.B, -1, -1, -1).contiguous()
        v = v[:1].expand(w.B, -1, -1, -1).contiguous()
    say(f"[strides] {name} {layout}: {w}")
    ref_gpu = run_forward(problem(w), q, k, v, gate)
    qv, kv_, vv, ov, o_store = _views(layout, q, k, v, w)
    p = _strided_problem(w, qv, kv_, vv, ov)
    buf = T.alloc_forward_buffers(p, dev())
    T.logo_forward(p, qv, kv_, vv, gate, ov, buf["mask"], buf["idx"], buf["rank"],
                   buf["workspace"])
    torch.cuda.synchronize()
    got = ov.contiguous()
    assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                       ref_gpu["o"].view(torch.int16) if got.dtype == torch.bfloat16
                       else ref_gpu["o"]), "strided forward differs from contiguous"
    assert _outside_untouched(o_store, ov)

    # oracle on the values the kernels read
    kk = host(k).astype(np.float64)
    vv_ = host(v).astype(np.float64)
    ref = oracle.forward(inp.q, kk, vv_, inp.gate, w.window, w.rho)
    assert np.array_equal(host(buf["idx"]), ref["idx"])
    err = float(np.abs(host(got) - ref["o"]).max())
    say(f"  forward max_abs={err:.3e}")
    assert err <= TOL[w.dtype]

    # unfused path: combine writes the strided o
    un = run_unfused(problem(w), q, k, v, gate)
    o_store.fill_(SENTINEL)
    o_local = un["o_local"]
    o_global = un["o_global"]
    T.logo_select_queries(p, gate, buf["mask"], buf["idx"], buf["rank"])
    ol2 = torch.empty_like(o_local)
    og2 = torch.empty_like(o_global)
    T.logo_local_attn(p, qv, kv_, vv, ol2)
    T.logo_global_attn_sparse(p, qv, kv_, vv, buf["idx"], og2)
    T.logo_combine(p, ol2, og2, buf["rank"], gate, ov)
    torch.cuda.synchronize()
    assert torch.equal(ol2, o_local) and torch.equal(og2, o_global)
    got2 = ov.contiguous()
    assert torch.equal(got2.float(), un["o"].float())
    assert _outside_untouched(o_store, ov)


def test_strides_must_match_the_view():
    w = get_workload("gqa32k", B=1, Hq=2, Hkv=1, n=64, window=16, rho=0.25)
    q, k, v, gate = to_dev(make_inputs(w, 0))
    qv = _token_major(q)
    p = T.make_problem(w.B, w.Hq, w.Hkv, w.n, w.d, w.window, w.rho, dtype=w.dtype)
    buf = T.alloc_forward_buffers(p, dev())
    with pytest.raises(ValueError):      # strided view, contiguous problem
        T.logo_forward(p, qv, k, v, gate, buf["o"], buf["mask"], buf["idx"], buf["rank"],
                       buf["workspace"])
    p2 = T.make_problem(w.B, w.Hq, w.Hkv, w.n, w.d, w.window, w.rho, dtype=w.dtype,
                        q_strides=T.view_strides(qv))
    with pytest.raises(ValueError):      # declared strides, contiguous tensor
        T.logo_forward(p2, q.clone(), k, v, gate, buf["o"], buf["mask"], buf["idx"],
                       buf["rank"], buf["workspace"])
