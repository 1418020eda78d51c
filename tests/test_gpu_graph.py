"""The entry points under HIP graph capture: a captured forward, training pass
and decode step, replayed several times on new input contents written in
place, with eager work and synchronisations between the replays, must give
exactly (bit for bit) what the same call gives eagerly on those contents.

Nothing here involves the oracle: eager results of the same library calls
are the reference, and the kernels are deterministic (fixed reduction
orders, no atomics in any sum), so equality is exact. The library enqueues
no memset nodes (counters and queues are cleared by kernels), which is what
makes replays after the first safe."""
import numpy as np
import pytest
import torch

import token_level_dynamic_amd as T
from gpu_util import dev, ensure_built, global_splits, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _fill(gen, t):
    """Seeded N(0,1) contents written into t in place (its dtype)."""
    t.copy_(torch.randn(t.shape, generator=gen, device=dev(), dtype=torch.float32))


def _capture(fn):
    """fn() once on a side stream (first-call set-up stays out of the
    graph), then captured; returns the graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _same(name, a, b):
    if a is None and b is None:
        return
    assert torch.equal(a, b), f"{name}: replay differs from the eager call"


FWD_CASES = {
    # (B, Hq, Hkv, n, d, window, rho, dtype)
    "bf16_split": (1, 8, 8, 1500, 128, 200, 0.3, "bf16"),
    "bf16_queue": (1, 16, 1, 20000, 128, 512, 0.2, "bf16"),
    "bf16_static_d64": (2, 8, 4, 12000, 64, 700, 0.5, "bf16"),
    "f32": (2, 4, 2, 900, 128, 100, 0.25, "f32"),
}


@pytest.mark.parametrize("name", sorted(FWD_CASES))
def test_forward_graph_replays(name):
    B, Hq, Hkv, n, d, W, rho, dt = FWD_CASES[name]
    p = T.make_problem(B, Hq, Hkv, n, d, W, rho, 0.0, dtype=dt)
    io = T.io_dtype(p)
    say(f"[graph] forward {name}: B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} W={W} rho={rho} "
        f"split={global_splits(p) if dt == 'bf16' else '-'}")
    q = torch.empty((B, Hq, n, d), dtype=io, device=dev())
    k = torch.empty((B, Hkv, n, d), dtype=io, device=dev())
    v = torch.empty_like(k)
    gate = torch.empty((B, n), dtype=torch.float32, device=dev())
    gen = torch.Generator(device=dev())
    gen.manual_seed(11)
    for t in (q, k, v, gate):
        _fill(gen, t)
    cap = T.alloc_forward_buffers(p, dev())
    eag = T.alloc_forward_buffers(p, dev())

    def fwd(b):
        T.logo_forward(p, q, k, v, gate, b["o"], b["mask"], b["idx"], b["rank"],
                       b["workspace"])

    g = _capture(lambda: fwd(cap))
    for rep in range(REPLAYS):
        if rep:
            for t in (q, gate) if rep == 1 else (k, v, gate):
                _fill(gen, t)
        # stale results in both sets of outputs: nothing may survive
        for b in (cap, eag):
            b["o"].fill_(float("nan") if io == torch.float32 else 7.0)
            b["mask"].fill_(3)
            b["idx"].fill_(-5)
            b["rank"].fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        fwd(eag)
        torch.cuda.synchronize()
        for key in ("o", "mask", "idx", "rank"):
            _same(f"{name} replay {rep} {key}", cap[key], eag[key])
        assert int(cap["mask"].sum()) == B * T.logo_target_count(rho, n)
        say(f"  replay {rep}: o, mask, idx, rank identical")


def test_training_pass_graph_replays():
    B, Hq, Hkv, n, d, W, rho = 1, 4, 2, 2100, 128, 300, 0.3
    p = T.make_problem(B, Hq, Hkv, n, d, W, rho, 0.0, dtype="bf16")
    say(f"[graph] training pass: B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} W={W} rho={rho}")
    bf = torch.bfloat16
    q = torch.empty((B, Hq, n, d), dtype=bf, device=dev())
    k = torch.empty((B, Hkv, n, d), dtype=bf, device=dev())
    v = torch.empty_like(k)
    gate = torch.empty((B, n), dtype=torch.float32, device=dev())
    dout = torch.empty_like(q)
    gen = torch.Generator(device=dev())
    gen.manual_seed(12)
    for t in (q, k, v, gate, dout):
        _fill(gen, t)

    def alloc():
        b = T.alloc_train_buffers(p, dev())
        b.update(T.alloc_backward_buffers(p, dev()))
        return b

    cap, eag = alloc(), alloc()

    def step(b):
        T.logo_forward_train(p, q, k, v, gate, b["o"], b["mask"], b["idx"], b["rank"],
                             b["lse_local"], b["lse_global"], b["o_local_sel"], b["o_global"])
        T.logo_backward(p, q, k, v, gate, b["o"], dout, b["idx"], b["rank"], b["lse_local"],
                        b["lse_global"], b["o_local_sel"], b["o_global"], b["dq"], b["dk"],
                        b["dv"], b["dgate"], b["workspace"])

    g = _capture(lambda: step(cap))
    outs = ("o", "mask", "idx", "rank", "lse_local", "lse_global", "o_local_sel", "o_global",
            "dq", "dk", "dv", "dgate")
    for rep in range(REPLAYS):
        if rep:
            for t in (dout, gate) if rep == 1 else (q, k):
                _fill(gen, t)
        for b in (cap, eag):
            for key in outs:
                b[key].fill_(9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(eag)
        torch.cuda.synchronize()
        for key in outs:
            _same(f"training replay {rep} {key}", cap[key], eag[key])
        say(f"  replay {rep}: forward outputs, statistics and gradients identical")


def test_decode_graph_replays_carry_the_threshold():
    """A captured decode step replayed as a decode loop: each replay reads
    the threshold the previous one updated, exactly as eager steps do."""
    B, Hq, Hkv, cap_len, d, W, rho, eta = 6, 8, 2, 3000, 128, 500, 0.3, 0.1
    p = T.make_decode_problem(B, Hq, Hkv, cap_len, d, W, rho, eta=eta, dtype="bf16")
    say(f"[graph] decode: B={B} Hq={Hq} Hkv={Hkv} cap={cap_len} d={d} W={W} eta={eta}")
    gen = torch.Generator(device=dev())
    gen.manual_seed(13)
    bf = torch.bfloat16
    q = torch.empty((B, Hq, d), dtype=bf, device=dev())
    kc = torch.empty((B, Hkv, cap_len, d), dtype=bf, device=dev())
    vc = torch.empty_like(kc)
    for t in (q, kc, vc):
        _fill(gen, t)
    lens = torch.tensor(np.array([1, 499, 500, 1700, 2999, 3000], np.int32), device=dev())
    gate = torch.empty(B, dtype=torch.float32, device=dev())
    _fill(gen, gate)
    tau0 = torch.zeros(B, dtype=torch.float32, device=dev())
    ws_bytes = T.logo_decode_workspace_size(p)

    def bufs():
        return {"tau": tau0.clone(),
                "o": torch.empty((B, Hq, d), dtype=bf, device=dev()),
                "sel": torch.empty(B, dtype=torch.uint8, device=dev()),
                "ws": torch.empty(ws_bytes, dtype=torch.uint8, device=dev())}

    cap, eag = bufs(), bufs()

    def step(b):
        T.logo_decode_step(p, q, kc, vc, lens, gate, b["tau"], b["o"], b["sel"], b["ws"])

    g = _capture(lambda: step(cap))
    cap["tau"].copy_(tau0)  # the set-up call and the capture left it moved on
    for rep in range(4):
        if rep:
            _fill(gen, q)
            _fill(gen, gate)
            lens.add_(1).clamp_(max=cap_len)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(eag)
        torch.cuda.synchronize()
        for key in ("o", "sel", "tau"):
            _same(f"decode replay {rep} {key}", cap[key], eag[key])
        say(f"  replay {rep}: selected={cap['sel'].tolist()} tau identical")
    assert not torch.equal(cap["tau"], tau0)


def test_routed_forward_graph_replays():
    """The routed forward computes the gate itself (router on the local
    output), then selects: a replay must redo every stage."""
    B, Hq, Hkv, n, d, W, rho = 2, 8, 2, 3000, 128, 256, 0.25
    p = T.make_problem(B, Hq, Hkv, n, d, W, rho, 0.0, dtype="bf16")
    say(f"[graph] routed forward: B={B} Hq={Hq} Hkv={Hkv} n={n} d={d} W={W} rho={rho}")
    bf = torch.bfloat16
    q = torch.empty((B, Hq, n, d), dtype=bf, device=dev())
    k = torch.empty((B, Hkv, n, d), dtype=bf, device=dev())
    v = torch.empty_like(k)
    w = torch.empty((Hq, d), dtype=torch.float32, device=dev())
    gen = torch.Generator(device=dev())
    gen.manual_seed(14)
    for t in (q, k, v, w):
        _fill(gen, t)
    cap = T.alloc_routed_buffers(p, dev())
    eag = T.alloc_routed_buffers(p, dev())
    outs = ("gate", "o", "mask", "idx", "rank")

    def fwd(b):
        T.logo_forward_routed(p, q, k, v, w, 0.5, b["gate"], b["o"], b["mask"], b["idx"],
                              b["rank"], b["workspace"])

    g = _capture(lambda: fwd(cap))
    for rep in range(REPLAYS):
        if rep:
            for t in (q, w) if rep == 1 else (k, v):
                _fill(gen, t)
        for b in (cap, eag):
            for key in outs:
                b[key].fill_(9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        fwd(eag)
        torch.cuda.synchronize()
        for key in outs:
            _same(f"routed replay {rep} {key}", cap[key], eag[key])
        say(f"  replay {rep}: gate, o, mask, idx, rank identical")


def test_varlen_forward_graph_replays():
    """Packed examples: the per-example tables are rebuilt from the device
    offsets on every replay."""
    cu_host = np.array([0, 700, 701, 2500, 2564, 4000], np.int32)
    n, Hq, Hkv, d, W, rho = int(cu_host[-1]), 4, 2, 128, 300, 0.3
    p = T.make_problem(1, Hq, Hkv, n, d, W, rho, 0.0, dtype="bf16")
    K = T.logo_varlen_selected_count(rho, cu_host)
    E = cu_host.size - 1
    say(f"[graph] varlen forward: offsets={cu_host.tolist()} Hq={Hq} Hkv={Hkv} d={d} W={W} "
        f"rho={rho} K={K}")
    bf = torch.bfloat16
    cu = torch.from_numpy(cu_host).to(dev())
    q = torch.empty((1, Hq, n, d), dtype=bf, device=dev())
    k = torch.empty((1, Hkv, n, d), dtype=bf, device=dev())
    v = torch.empty_like(k)
    gate = torch.empty(n, dtype=torch.float32, device=dev())
    gen = torch.Generator(device=dev())
    gen.manual_seed(15)
    for t in (q, k, v, gate):
        _fill(gen, t)
    ws = T.logo_varlen_workspace_size(p, E, K)

    def bufs():
        return {"o": torch.empty_like(q),
                "mask": torch.empty(n, dtype=torch.uint8, device=dev()),
                "idx": torch.empty(K, dtype=torch.int32, device=dev()),
                "rank": torch.empty(n, dtype=torch.int32, device=dev()),
                "workspace": torch.empty(ws, dtype=torch.uint8, device=dev()) if ws else None}

    cap, eag = bufs(), bufs()
    outs = ("o", "mask", "idx", "rank")

    def fwd(b):
        T.logo_forward_varlen(p, cu, K, q, k, v, gate, b["o"], b["mask"], b["idx"], b["rank"],
                              b["workspace"])

    g = _capture(lambda: fwd(cap))
    for rep in range(REPLAYS):
        if rep:
            for t in (q, gate) if rep == 1 else (k, v, gate):
                _fill(gen, t)
        for b in (cap, eag):
            for key in outs:
                b[key].fill_(9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        fwd(eag)
        torch.cuda.synchronize()
        for key in outs:
            _same(f"varlen replay {rep} {key}", cap[key], eag[key])
        assert int(cap["mask"].sum()) == K
        say(f"  replay {rep}: o, mask, idx, rank identical")
