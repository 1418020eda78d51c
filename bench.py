"""Benchmark: one forward of token-level dynamic local-global attention.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa32k]
                    [--rho R] [--no-cpu-baseline]

A step is one logo_forward over one batch of seeded synthetic input already
resident in HBM: budget-controller selection, local band attention for every
query, query-sparse global attention for the selected rows, gated combine.
Prints one JSON line.

value    effective attention TFLOP/s of the whole layer:
         F = 4 d sum_b sum_h [ sum_i min(W, i+1) + sum_{i in S_b} (i+1) ]
         (2 flops per multiply-add, Q K^T and P V both counted, softmax not
         counted, masked pairs not counted; S is the realised selection)
         divided by the measured time per step.
roofline the dominant kernel (the query-sparse global branch at the default
         workload): its algorithmic FLOPs per launch over its average launch
         time, measured with HIP events recorded by the library on the
         kernel's own stream during the timed steps, against the bf16 dense
         matrix-core peak of MI355X (2500 TFLOP/s). `traffic` is the HBM
         bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE counters,
         scaled by a copy-kernel calibration (profiles/), reported only while
         the kernel sources match the ones the counters were taken on.
cpu_baseline the CPU fp64 oracle, timed on this host on a bounded random
         sample of the same layer's rows (the oracle is a reported baseline,
         not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
HBM_PEAK_GBS = 8000.0
METRIC = "effective attn TFLOP/s + ms/layer fwd at 32K ctx, rho=0.2; % of bf16 MFMA peak"
ROUTED_METRIC = ("effective attn TFLOP/s + ms/layer of the routed forward (local branch, gate "
                 "from its output, select, global branch) at 32K ctx, rho=0.2; % of bf16 MFMA "
                 "peak")
TRAIN_METRIC = ("effective attn TFLOP/s + ms/layer of one training pass (forward with saved "
                "statistics + backward) at 32K ctx, rho=0.2; % of bf16 MFMA peak")
KERNEL_SOURCES = ["attn_bf16.hip", "select.hip", "combine.hip", "abi.cpp"]
TRAIN_SOURCES = KERNEL_SOURCES + ["backward_prep.hip", "backward_bf16.hip"]
COPY_BYTES = 1 << 30


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for name in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "token_level_dynamic_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def input_sha256(*arrays) -> str:
    """SHA-256 (first 16 hex digits) of the input arrays' bytes, in order: the
    same seed and workload give the same digest on any machine."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]


def effective_flops(w, idx: np.ndarray) -> dict:
    """Effective FLOPs of the layer from the realised selection idx [B, k];
    `distinct` counts each (query, key) pair once: a selected row's window
    pairs are part of its prefix (what the single launch computes)."""
    i = np.arange(w.n, dtype=np.float64)
    band_pairs = float(np.minimum(w.window, i + 1).sum())          # per (b, h)
    glob_pairs = [float((idx[b].astype(np.float64) + 1).sum()) for b in range(w.B)]
    sel_band = [float(np.minimum(w.window, idx[b].astype(np.float64) + 1).sum())
                for b in range(w.B)]
    per_pair = 4.0 * w.d
    local = per_pair * w.Hq * w.B * band_pairs
    glob = per_pair * w.Hq * sum(glob_pairs)
    distinct = local + glob - per_pair * w.Hq * sum(sel_band)
    return {"local": local, "global": glob, "total": local + glob, "distinct": distinct}


# The CPU oracle's worker processes: forked in main() before the GPU is
# touched, so they inherit the inputs and the oracle's selection and hold no
# GPU state. Each runs NumPy with one BLAS thread.
_CPU = {}


def _cpu_worker_init() -> None:
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # threadpoolctl missing: the environment variables stand
        pass


def _cpu_rows(rows):
    import oracle
    c = _CPU
    r = oracle.forward_rows(c["q"], c["k"], c["v"], c["gate"], c["window"], c["rho"], rows,
                            selection=c["selection"])
    return rows, r["o_rows"]


def cpu_cores() -> int:
    """Cores the oracle may use: this process's CPU affinity, at most 16
    (one GPU's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def start_cpu_oracle(w, inp):
    """Selection by the oracle (timed: it is part of the oracle's forward),
    then the worker pool. Call before any GPU work."""
    import multiprocessing as mp
    import oracle
    t0 = time.perf_counter()
    sel = oracle.select_queries(inp.gate, w.rho)
    _CPU.update(q=inp.q, k=inp.k, v=inp.v, gate=inp.gate, window=w.window, rho=w.rho,
                selection=sel, select_s=time.perf_counter() - t0)
    cores = cpu_cores()
    _CPU["pool"] = mp.get_context("fork").Pool(cores, initializer=_cpu_worker_init)
    _CPU["cores"] = cores


def _host_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = [f"{x.get('internal_api')} {x.get('version')}" for x in threadpool_info()
                if x.get("user_api") == "blas"]
        blas = ", ".join(blas) or None
    except Exception:
        pass
    return {"cpu_model": model, "numpy": np.__version__, "blas": blas}


def cpu_baseline(w, o_dev, budget_s: float = 15.0, seed: int = 0, chunk: int = 16) -> dict:
    """The CPU oracle (oracle.forward_rows, row by row in float64) over a
    uniform seeded sample of the layer's rows (b, h, i), spread over the
    worker pool for about budget_s seconds of wall time. The rate is the
    sample's effective FLOPs (4 d per (query, key) pair of each row's local
    window and, for selected rows, its causal prefix) over the wall time; the
    whole layer's time is extrapolated from it by the layer's pair count
    (plus the one selection). The sampled rows are also compared with the
    GPU's output of the timed run (o_dev)."""
    pool, cores = _CPU["pool"], _CPU["cores"]
    mask = _CPU["selection"][0]
    r = np.random.default_rng(seed)
    pending = []
    done = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s or pending:
        while time.perf_counter() - t0 < budget_s and len(pending) < 2 * cores:
            rows = [(int(r.integers(0, w.B)), int(r.integers(0, w.Hq)), int(r.integers(0, w.n)))
                    for _ in range(chunk)]
            pending.append(pool.apply_async(_cpu_rows, (rows,)))
        still = []
        for a in pending:
            if a.ready():
                done.append(a.get())
            else:
                still.append(a)
        pending = still
        time.sleep(0.002)
    wall = time.perf_counter() - t0
    pool.terminate()
    rows = [x for rs, _ in done for x in rs]
    ref = np.concatenate([o for _, o in done])
    pairs = sum(min(w.window, i + 1) + (i + 1 if mask[b, i] else 0) for b, _, i in rows)
    rate = 4.0 * w.d * pairs / wall                            # flops per second
    layer_pairs = band_pairs(w) * w.B * w.Hq + w.Hq * float(
        sum((np.flatnonzero(mask[b]) + 1).sum() for b in range(w.B)))
    layer_s = 4.0 * w.d * layer_pairs / rate + _CPU["select_s"]
    import torch
    bi = torch.tensor([x[0] for x in rows], device=o_dev.device)
    hi = torch.tensor([x[1] for x in rows], device=o_dev.device)
    ii = torch.tensor([x[2] for x in rows], device=o_dev.device)
    got = o_dev[bi, hi, ii].double().cpu().numpy()
    err = float(np.abs(got - ref).max())
    nsel = sum(int(mask[b, i]) for b, _, i in rows)
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(rows)} rows (b, h, i) drawn uniformly with seed {seed} from the "
                      f"{w.name} layer ({nsel} selected, so also global), {chunk} rows per "
                      f"task over {cores} worker processes (one BLAS thread each), "
                      f"{wall:.1f} s wall; the selection computed once",
            "extrapolated": {"layer_s": float(f"{layer_s:.4g}"),
                             "how": "the whole layer's (query, key) pairs at the sample's rate, "
                                    "plus the selection's time"},
            "host": _host_info(),
            "parity": {"rows": len(rows), "max_abs": err,
                       "tolerance": 2e-2 if w.dtype == "bf16" else 1e-4,
                       "against": "the GPU output of the timed run"}}


def load_traffic(workload: str, current_hash: str, key: str = "global_bytes_per_launch"):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(workload)
    if not ent or ent.get("source_hash") != current_hash:
        return None
    return ent.get(key)


def copy_calibration(torch) -> int:
    """An elementwise copy that reads and writes exactly COPY_BYTES each."""
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                                           "launches": 3, "kernel": "torch elementwise add"}}))
    return 0


def _counter_means(csv_dir: str, counter: str, n_first: int = 3) -> dict:
    """Mean value of `counter` over the first n_first dispatches of each
    kernel in a rocprofv3 --pmc csv directory (values summed per dispatch)."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "*counter_collection.csv"))
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv in {csv_dir}")
    per = {}
    order = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            order.setdefault(r["Kernel_Name"], set()).add(int(r["Dispatch_Id"]))
    out = {}
    for name, ids in order.items():
        first = sorted(ids)[:n_first]
        out[name] = sum(per[(name, i)] for i in first) / len(first)
    return out


def _pick(means: dict, fragment: str) -> float:
    hits = [v for k, v in means.items() if fragment in k]
    if len(hits) != 1:
        raise SystemExit(f"kernel {fragment!r}: {len(hits)} matches")
    return hits[0]


def record_traffic(args) -> int:
    """Write profiles/traffic.json from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (KiB per dispatch): the copy calibration fixes the scale of each counter
    (bytes the 1 GiB copy moves over what the counter reports), and each
    kernel's bytes per launch are its mean counter value (warm-up and the two
    timed dispatches) times 1024 times that scale. The current kernel-source
    hashes are stored with them, so bench.py reports the figures only while
    the kernels are unchanged."""
    fs = COPY_BYTES / (1024.0 * _pick(_counter_means(args.copy_fetch, "FETCH_SIZE"), "add"))
    ws = COPY_BYTES / (1024.0 * _pick(_counter_means(args.copy_write, "WRITE_SIZE"), "add"))
    fm = _counter_means(args.fwd_fetch, "FETCH_SIZE")
    wm = _counter_means(args.fwd_write, "WRITE_SIZE")
    note = ("FETCH_SIZE/WRITE_SIZE KiB per dispatch (rocprofv3 --pmc, one counter per run; "
            "mean of the warm-up and the two timed dispatches) times 1024 times the "
            "copy-kernel scale; written by bench.py --record-traffic, see "
            "hbm_traffic_gqa32k.md")
    fz = "attn_bf16_fused_kernel<128, false>"
    if any(fz in k for k in fm):
        # the single-launch forward: one kernel for both branches
        fr, fw = _pick(fm, fz) * 1024 * fs, _pick(wm, fz) * 1024 * ws
        data = {"gqa32k": {
            "source_hash": kernel_source_hash(),
            "fused_bytes_per_launch": round(fr + fw),
            "fused_read_bytes": round(fr),
            "fused_write_bytes": round(fw),
            "fetch_scale": round(fs, 5),
            "write_scale": round(ws, 5),
            "note": note}}
    else:
        g = "attn_bf16_kernel<128, true, 3, false, false>"
        lo = "attn_bf16_kernel<128, false, 1, false, false>"
        gr, gw = _pick(fm, g) * 1024 * fs, _pick(wm, g) * 1024 * ws
        data = {"gqa32k": {
            "source_hash": kernel_source_hash(),
            "global_bytes_per_launch": round(gr + gw),
            "global_read_bytes": round(gr),
            "global_write_bytes": round(gw),
            "local_bytes_per_launch": round((_pick(fm, lo) * fs + _pick(wm, lo) * ws) * 1024),
            "fetch_scale": round(fs, 5),
            "write_scale": round(ws, 5),
            "note": note}}
    if args.train_fetch and args.train_write:
        tf = _counter_means(args.train_fetch, "FETCH_SIZE")
        tw = _counter_means(args.train_write, "WRITE_SIZE")
        dk = "bwd_dkdv_kernel<128>"
        dq = ("bwd_dq_kernel<128, true>", "bwd_dq_kernel<128, false>")
        dr, dw = _pick(tf, dk) * 1024 * fs, _pick(tw, dk) * 1024 * ws
        data["gqa32k_train"] = {
            "source_hash": kernel_source_hash(TRAIN_SOURCES),
            "bwd_dkdv_bytes_per_launch": round(dr + dw),
            "bwd_dkdv_read_bytes": round(dr),
            "bwd_dkdv_write_bytes": round(dw),
            "bwd_dq_bytes_per_launch": round(sum((_pick(tf, x) * fs + _pick(tw, x) * ws) * 1024
                                                 for x in dq)),
            "fetch_scale": round(fs, 5),
            "write_scale": round(ws, 5),
            "note": "same counters on bench.py --mode train; bwd_dq is both dQ launches"}
    path = args.traffic_out or os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(path):
        # keep the entries these runs do not replace (e.g. the training pass)
        with open(path) as f:
            old = json.load(f)
        old.update(data)
        data = old
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(json.dumps(data))
    return 0


def gemm_ceiling(torch) -> int:
    """Sustained bf16 matrix-core rate of a plain library GEMM on this part,
    on random N(0,1) operands and on zero operands. The published dense peak
    assumes the top clock; under a full matrix-core load the clock is set by
    power, which depends on the data, so this is the practical ceiling that
    the attention kernels' rates can be read against."""
    out = {}
    for n in (8192, 16384):
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        z = torch.zeros_like(a)
        reps = 20 if n == 8192 else 5
        for name, (x, y) in (("random", (a, b)), ("zero", (z, z))):
            for _ in range(3):
                torch.matmul(x, y)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                torch.matmul(x, y)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            out[f"{n}^3 {name}"] = {"ms": round(ms, 4), "TFLOP/s": round(2 * n ** 3 / ms / 1e9, 1)}
    print(json.dumps({"gemm_ceiling": out, "kernel": "torch.matmul bf16 (hipBLASLt)",
                      "published_dense_peak_TFLOP/s": BF16_PEAK_TFLOPS}))
    return 0


def ceilings(torch) -> int:
    """Throughput ceilings of one compute unit from the microbenchmarks in
    csrc/ceiling.hip (libceiling.so): each kernel records the shader clock and
    the 100 MHz reference clock per workgroup, so rates come out per clock
    cycle (and the clock under that load as a frequency). Two resident
    256-thread workgroups per CU (2 waves per SIMD, as the attention kernels
    run) unless the row says otherwise."""
    import ctypes
    from token_level_dynamic_amd.build import CEILING_LIB
    lib = ctypes.CDLL(CEILING_LIB)
    lib.ceiling_launch.restype = ctypes.c_int
    lib.ceiling_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong,
                                   ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    # kind: name, work per wave per iteration, unit
    only = os.environ.get("CEILING_KINDS")
    kinds = {0: ("mfma_32x32x16_bf16", 4 * 32768.0, "flop"),
             1: ("ds_read_b128", 8 * 1024.0, "B"),
             2: ("ds_read_b64_tr_b16", 8 * 512.0, "B"),
             3: ("v_exp_f32", 8 * 64.0, "exp"),
             4: ("mfma + 0.5 KiB LDS per product", 4 * 32768.0, "flop"),
             5: ("mfma + 1 KiB LDS per product", 4 * 32768.0, "flop"),
             6: ("mfma + 2 KiB LDS per product", 4 * 32768.0, "flop"),
             7: ("V tile reads, stride 144", 32 * 512.0, "B"),
             8: ("V tile reads, stride 160", 32 * 512.0, "B"),
             9: ("V tile reads, swizzled 128", 32 * 512.0, "B"),
             10: ("K tile reads, stride 136", 16 * 1024.0, "B"),
             11: ("K tile reads, swizzled 128", 16 * 1024.0, "B"),
             # products counted for the waves that issue them (half of the
             # waves in the split forms)
             13: ("mfma + 2 rounds fma/exp2 per product, same wave", 4 * 32768.0, "flop"),
             14: ("mfma only (control for 13-18)", 4 * 32768.0, "flop"),
             15: ("fma/exp2 only, 8 per iteration", 4 * 2 * 2 * 64.0, "valu"),
             16: ("mfma in even waves, 2 rounds fma/exp2 in odd waves", 2 * 32768.0, "flop"),
             17: ("mfma + 4 rounds fma/exp2 per product, same wave", 4 * 32768.0, "flop"),
             18: ("mfma in even waves, 4 rounds fma/exp2 in odd waves", 2 * 32768.0, "flop"),
             19: ("mfma + 0.5 KiB LDS per product, random operands", 4 * 32768.0, "flop"),
             20: ("mfma, one dependent chain", 4 * 32768.0, "flop"),
             21: ("mfma, two dependent chains", 4 * 32768.0, "flop"),
             22: ("as 13, accumulators in VGPRs", 4 * 32768.0, "flop"),
             23: ("as 14, accumulators in VGPRs", 4 * 32768.0, "flop"),
             # 512-thread workgroups: waves w and w + 4 share a SIMD; products
             # counted for the waves that issue them
             25: ("8 waves: products in all", 2 * 4 * 32768.0, "flop"),
             26: ("8 waves: products in waves 0-3, 4-7 idle", 4 * 32768.0, "flop"),
             27: ("8 waves: products in 0-3, 8 FMA per product in 4-7", 4 * 32768.0, "flop"),
             28: ("8 waves: products in 0-3, 2 v_exp_f32 per product in 4-7", 4 * 32768.0,
                  "flop"),
             29: ("8 waves: products + 8 FMA per product in 0-3, 4-7 idle", 4 * 32768.0,
                  "flop"),
             30: ("8 waves: products + 2 v_exp_f32 per product in 0-3, 4-7 idle",
                  4 * 32768.0, "flop"),
             31: ("tile model, 1 wave/SIMD: 0.5 KiB LDS + 3.5 FMA per product", 4 * 32768.0,
                  "flop"),
             32: ("tile model, 2 waves/SIMD: 1 KiB LDS + 3.5 FMA per product",
                  2 * 4 * 32768.0, "flop"),
             33: ("tile model, 1 wave/SIMD: 0.5 KiB LDS per product", 4 * 32768.0, "flop"),
             34: ("tile model, 1 wave/SIMD: 3.5 FMA per product", 4 * 32768.0, "flop"),
             35: ("tile model, 2 waves/SIMD: 1 KiB LDS per product", 2 * 4 * 32768.0, "flop"),
             36: ("tile model, 2 waves/SIMD: 3.5 FMA per product", 2 * 4 * 32768.0, "flop"),
             37: ("8 waves: products in 0-3, 4 v_dot2_f32_bf16 per product in 4-7",
                  4 * 32768.0, "flop"),
             38: ("8 waves: products in 0-3, 4 FMA per product in 4-7", 4 * 32768.0, "flop")}
    if only:
        kinds = {k: v for k, v in kinds.items() if str(k) in only.split(",")}
    out = {}
    for kind, (name, per_iter, unit) in kinds.items():
        for wg_per_cu in (1, 2, 4):
            blocks = cus * wg_per_cu
            iters = 20000 if kind in (0, 4, 5, 6) or kind >= 13 else 4000 if kind >= 7 else 40000
            sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            clk = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
            rc = lib.ceiling_launch(kind, blocks, 10, sink.data_ptr(), clk.data_ptr(), None, 0,
                                    stream.cuda_stream)
            if rc != 0:
                raise SystemExit(f"ceiling kernel {kind} failed: hip error {rc}")
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.ceiling_launch(kind, blocks, iters, sink.data_ptr(), clk.data_ptr(), None, 0,
                                    stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise SystemExit(f"ceiling kernel {kind} failed: hip error {rc}")
            ms = e0.elapsed_time(e1)
            c = clk.view(blocks, 4).cpu().numpy().astype(np.float64)
            cyc = float(np.median(c[:, 1] - c[:, 0]))
            ref = float(np.median(c[:, 3] - c[:, 2]))
            ghz = cyc / ref * 0.1 if ref > 0 else None
            total = per_iter * iters * 4 * blocks / (ms * 1e-3)
            # per CU and shader clock cycle, at the clock the kernel ran at
            per_cu_clk = total / (cus * ghz * 1e9) if ghz else float("nan")
            out[f"{name} | {wg_per_cu} WG/CU"] = {
                f"{unit}_per_clk_per_cu": round(per_cu_clk, 1),
                "clock_GHz": round(ghz, 3) if ghz else None,
                f"{unit}_per_s_chip": total, "ms": round(ms, 3)}
            print(json.dumps({name: out[f"{name} | {wg_per_cu} WG/CU"],
                              "wg_per_cu": wg_per_cu}), flush=True)
    # HBM: streaming 16-byte reads over 4 GiB of random bytes, 4 passes
    # the HBM streams run with every kind, or alone with CEILING_KINDS=stream
    nbytes = 4 << 30 if not only or "stream" in only.split(",") else 0
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (max(nbytes, 16) // 4,), dtype=torch.int32,
                        device="cuda")
    for wg_per_cu in ((2, 4, 8) if nbytes else ()):
        blocks = cus * wg_per_cu
        sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        lib.ceiling_launch(12, blocks, 1, sink.data_ptr(), None, src.data_ptr(), nbytes,
                           stream.cuda_stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(4):
            rc = lib.ceiling_launch(12, blocks, 1, sink.data_ptr(), None, src.data_ptr(), nbytes,
                                    stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if rc != 0:
            raise SystemExit(f"stream read kernel failed: hip error {rc}")
        gbs = 4 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
        out[f"hbm stream read 4 GiB | {wg_per_cu} WG/CU"] = {"GB_per_s": round(gbs, 1)}
        print(json.dumps({"hbm stream read": round(gbs, 1), "wg_per_cu": wg_per_cu}), flush=True)
    # the same over 1 GiB, into registers (12) and through the LDS DMA (39)
    for kind, name in ((12, "registers"), (39, "LDS DMA")):
        for wg_per_cu in ((2, 4) if nbytes else ()):
            blocks = cus * wg_per_cu
            sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            sub = 1 << 30
            rc = lib.ceiling_launch(kind, blocks, 1, sink.data_ptr(), None, src.data_ptr(), sub,
                                    stream.cuda_stream)
            if rc != 0:
                raise SystemExit(f"stream kernel {kind} failed: hip error {rc}")
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(8):
                lib.ceiling_launch(kind, blocks, 1, sink.data_ptr(), None, src.data_ptr(), sub,
                                   stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            gbs = 8 * sub / (e0.elapsed_time(e1) * 1e-3) / 1e9
            out[f"hbm stream read 1 GiB, {name} | {wg_per_cu} WG/CU"] = {"GB_per_s": round(gbs, 1)}
            print(json.dumps({f"hbm stream read 1 GiB, {name}": round(gbs, 1),
                              "wg_per_cu": wg_per_cu}), flush=True)
    del src
    print(json.dumps({"ceilings": out, "cus": cus,
                      "source": "token_level_dynamic_amd/csrc/ceiling.hip"}))
    return 0


def per_step_timing(torch, step, stream, steps: int) -> dict:
    """Each forward timed on its own: warm (back to back) and cold (a 1 GiB
    device write before each forward evicts L2 and the MALL), median/min/max.
    Runs after the contract's timed region and does not change `value`."""
    flush = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    out = {}
    for mode in ("warm", "cold"):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            if mode == "cold":
                flush.fill_(1.0)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)
        out[mode] = {"median_ms": round(float(np.median(ms)), 4), "min_ms": round(ms[0], 4),
                     "max_ms": round(ms[-1], 4)}
    del flush
    return out


def band_pairs(w) -> float:
    i = np.arange(w.n, dtype=np.float64)
    return float(np.minimum(w.window, i + 1).sum())


def train_bench(args, torch, T, w, inp, p, q, k, v, gate, dev, digest) -> int:
    """One step = logo_forward_train + logo_backward over one batch."""
    from workloads import make_dout
    dvals, dbits = make_dout(w, args.seed)
    if dbits is not None:
        dout = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        dout = torch.from_numpy(dvals).to(dev)
    del dvals, dbits
    fw = T.alloc_train_buffers(p, dev)
    bw = T.alloc_backward_buffers(p, dev)

    def step():
        T.logo_forward_train(p, q, k, v, gate, fw["o"], fw["mask"], fw["idx"], fw["rank"],
                             fw["lse_local"], fw["lse_global"], fw["o_local_sel"],
                             fw["o_global"])
        T.logo_backward(p, q, k, v, gate, fw["o"], dout, fw["idx"], fw["rank"],
                        fw["lse_local"], fw["lse_global"], fw["o_local_sel"], fw["o_global"],
                        bw["dq"], bw["dk"], bw["dv"], bw["dgate"], bw["workspace"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    T.logo_profile_begin()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    stage_ms, stage_n = T.logo_profile_end()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    per_step = per_step_timing(torch, step, stream, args.steps)

    idx = fw["idx"].cpu().numpy()
    # pairs (query, key) of each branch, summed over b and query heads
    local_pairs = band_pairs(w) * w.B * w.Hq
    glob_pairs = w.Hq * float(sum((idx[b].astype(np.float64) + 1).sum() for b in range(w.B)))
    pairs = local_pairs + glob_pairs
    # 2 flops per multiply-add: forward QK^T and PV (4d per pair); backward
    # recompute QK^T, dO V^T, P^T dO, dS K, dS^T Q (10d per pair)
    F_fwd, F_bwd = 4.0 * w.d * pairs, 10.0 * w.d * pairs
    tflops = (F_fwd + F_bwd) / (ms_per_step * 1e-3) / 1e12
    avg = {s: (stage_ms[j] / stage_n[j] if stage_n[j] else None)
           for j, s in enumerate(T.STAGES)}
    # the dK/dV kernel runs QK^T, dO V^T, P^T dO and dS^T Q on every pair
    # (8d per pair); the dQ kernels run QK^T, dO V^T and dS K (6d per pair)
    kern = {"bwd_dkdv": 8.0 * w.d * pairs, "bwd_dq": 6.0 * w.d * pairs}
    dom = max(kern, key=lambda s: avg[s] or 0.0)
    dom_ms = avg[dom]
    achieved = kern[dom] / (dom_ms * 1e-3) / 1e12 if dom_ms else None
    traffic = load_traffic(w.name, kernel_source_hash(TRAIN_SOURCES), f"{dom}_bytes_per_launch")
    result = {
        "metric": TRAIN_METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "input_sha256": digest,
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "n": w.n,
                   "d": w.d, "window": w.window, "rho": w.rho,
                   "k_sel": int(T.logo_target_count(w.rho, w.n)), "seed": args.seed,
                   "mode": "train", "parallelism": "none (1 GPU)"},
        "pct_of_bf16_peak": round(100.0 * tflops / BF16_PEAK_TFLOPS, 2),
        "effective_flops": {"forward": F_fwd, "backward": F_bwd},
        "stage_ms_avg": {s: round(x, 4) for s, x in avg.items() if x is not None},
        "per_step_ms": per_step,
        "roofline": {
            "kernel": {"bwd_dkdv": "bwd_dkdv_kernel (dK, dV of both branches)",
                       "bwd_dq": "bwd_dq_kernel (dQ, local then global launch)"}[dom],
            "bound": "mfma",
            "achieved": round(achieved, 2) if achieved else None,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4) if achieved else None,
            "traffic": traffic,
            "algorithmic_flops_per_launch": kern[dom],
            "avg_launch_ms": round(dom_ms, 4) if dom_ms else None,
        },
    }
    print(json.dumps(result), flush=True)
    return 0


def routed_bench(args, torch, T, w, inp, p, q, k, v, dev, digest) -> int:
    """One step = logo_forward_routed (local, router logits, select, global)."""
    from workloads import make_router
    rw, rb = make_router(w, args.seed)
    router_w = torch.from_numpy(rw).to(dev)
    buf = T.alloc_routed_buffers(p, dev)

    def step():
        T.logo_forward_routed(p, q, k, v, router_w, rb, buf["gate"], buf["o"], buf["mask"],
                              buf["idx"], buf["rank"], buf["workspace"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    T.logo_profile_begin()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    stage_ms, stage_n = T.logo_profile_end()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    per_step = per_step_timing(torch, step, stream, args.steps)
    idx = buf["idx"].cpu().numpy()
    F = effective_flops(w, idx)
    F_router = 2.0 * w.Hq * w.d * w.n * w.B      # one multiply-add per local output element
    tflops = (F["total"] + F_router) / (ms_per_step * 1e-3) / 1e12
    avg = {s: (stage_ms[j] / stage_n[j] if stage_n[j] else None)
           for j, s in enumerate(T.STAGES)}
    dom = "global" if F["global"] >= F["local"] else "local"
    dom_ms = avg[dom]
    achieved = F[dom] / (dom_ms * 1e-3) / 1e12 if dom_ms else None
    result = {
        "metric": ROUTED_METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "input_sha256": digest,
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "n": w.n,
                   "d": w.d, "window": w.window, "rho": w.rho,
                   "k_sel": int(T.logo_target_count(w.rho, w.n)), "seed": args.seed,
                   "mode": "routed", "parallelism": "none (1 GPU)"},
        "pct_of_bf16_peak": round(100.0 * tflops / BF16_PEAK_TFLOPS, 2),
        "effective_flops": F["total"] + F_router,
        "stage_ms_avg": {s: round(x, 4) for s, x in avg.items() if x is not None},
        "per_step_ms": per_step,
        "roofline": {
            "kernel": f"attn_bf16_kernel ({dom} branch, routed epilogue)",
            "bound": "mfma",
            "achieved": round(achieved, 2) if achieved else None,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4) if achieved else None,
            "traffic": None,
            "algorithmic_flops_per_launch": F[dom],
            "avg_launch_ms": round(dom_ms, 4) if dom_ms else None,
        },
    }
    print(json.dumps(result), flush=True)
    return 0


def decode_bench(args, torch, T) -> int:
    """One step = logo_decode_step: controller, chunked decode, reduction."""
    from statistics import NormalDist
    from workloads import DECODE_WORKLOADS, make_decode_inputs
    cfg = DECODE_WORKLOADS["decode128k"]
    B, Hq, Hkv, cap, d, W = (cfg[x] for x in ("B", "Hq", "Hkv", "cap", "d", "window"))
    # threshold at the N(0,1) quantile the logits exceed with probability rho
    tau0 = NormalDist().inv_cdf(1.0 - cfg["rho"])
    inp = make_decode_inputs(B, Hq, Hkv, cap, d, cfg["dtype"], seed=args.seed,
                             tau=np.full(B, tau0, np.float32))
    dev = torch.device("cuda:0")

    def cv(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    digest = input_sha256(inp.bits["q"], inp.bits["k"], inp.bits["v"], inp.lens, inp.gate, inp.tau)
    q, k, v = cv(inp.bits["q"]), cv(inp.bits["k"]), cv(inp.bits["v"])
    del inp.k, inp.v, inp.bits
    lens = torch.from_numpy(inp.lens).to(dev)
    gate = torch.from_numpy(inp.gate).to(dev)
    tau = torch.from_numpy(inp.tau).to(dev)
    # eta = 0: the controller is frozen so every timed step makes the same decisions
    p = T.make_decode_problem(B, Hq, Hkv, cap, d, W, cfg["rho"], eta=0.0, dtype=cfg["dtype"])
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    sel = torch.empty(B, dtype=torch.uint8, device=dev)
    ws = torch.empty(T.logo_decode_workspace_size(p), dtype=torch.uint8, device=dev)

    def step():
        T.logo_decode_step(p, q, k, v, lens, gate, tau, o, sel, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    T.logo_profile_begin()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    stage_ms, stage_n = T.logo_profile_end()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    per_step = per_step_timing(torch, step, stream, args.steps)
    selected = sel.cpu().numpy().astype(bool)
    nl = inp.lens.astype(np.float64)
    keys = np.where(selected, nl, np.minimum(W, nl))      # cached keys read per (b, kv head)
    # algorithmic bytes: each needed cached key and value once (bf16), q and o once
    algo = float(keys.sum()) * Hkv * d * 2 * 2 + 2.0 * B * Hq * d * 2
    dec_ms = stage_ms[T.STAGES.index("decode")] / max(stage_n[T.STAGES.index("decode")], 1)
    gbs = algo / (dec_ms * 1e-3) / 1e9
    result = {
        "metric": "decode step of 8 sequences with 128K caches: effective HBM GB/s (cached "
                  "K/V bytes the step must read over its time), ms per step",
        "value": round(algo / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "input_sha256": digest,
        "config": {"workload": "decode128k", "B": B, "Hq": Hq, "Hkv": Hkv, "cap": cap, "d": d,
                   "window": W, "rho": cfg["rho"], "tau": round(tau0, 6), "eta": 0.0,
                   "selected": int(selected.sum()), "seed": args.seed, "mode": "decode",
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "algorithmic_bytes": algo,
        "stage_ms_avg": {s: round(stage_ms[j] / stage_n[j], 4)
                         for j, s in enumerate(T.STAGES) if stage_n[j]},
        "per_step_ms": per_step,
        "roofline": {
            "kernel": "decode_stream_kernel + decode_reduce_kernel",
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": algo,
            "avg_launch_ms": round(dec_ms, 4),
        },
    }
    print(json.dumps(result), flush=True)
    return 0


def varlen_bench(args, torch, T) -> int:
    """One step = logo_forward_varlen over the packed varlen64k batch."""
    from workloads import VARLEN_WORKLOADS, make_varlen_inputs
    cfg = VARLEN_WORKLOADS["varlen64k"]
    lens, Hq, Hkv, d, W, rho = (cfg[x] for x in ("lens", "Hq", "Hkv", "d", "window", "rho"))
    inp = make_varlen_inputs(lens, Hq, Hkv, d, cfg["dtype"], seed=args.seed)
    dev = torch.device("cuda:0")

    def cv(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)[None]
    digest = input_sha256(inp["bits"]["q"], inp["bits"]["k"], inp["bits"]["v"], inp["gate"],
                          inp["cu"])
    q, k, v = cv(inp["bits"]["q"]), cv(inp["bits"]["k"]), cv(inp["bits"]["v"])
    Tn = int(inp["cu"][-1])
    p = T.make_problem(1, Hq, Hkv, Tn, d, W, rho)
    K = T.logo_varlen_selected_count(rho, inp["cu"])
    cu = torch.from_numpy(inp["cu"]).to(dev)
    gate = torch.from_numpy(inp["gate"]).to(dev)
    o = torch.empty((1, Hq, Tn, d), dtype=torch.bfloat16, device=dev)
    mask = torch.empty(Tn, dtype=torch.uint8, device=dev)
    idx = torch.empty(K, dtype=torch.int32, device=dev)
    rank = torch.empty(Tn, dtype=torch.int32, device=dev)
    ws = torch.empty(T.logo_varlen_workspace_size(p, len(lens), K), dtype=torch.uint8,
                     device=dev)

    def step():
        T.logo_forward_varlen(p, cu, K, q, k, v, gate, o, mask, idx, rank, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    T.logo_profile_begin()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    stage_ms, stage_n = T.logo_profile_end()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    per_step = per_step_timing(torch, step, stream, args.steps)
    # effective FLOPs: 4 d per (query, key) pair of each example's band and
    # of its selected rows' prefixes (positions relative to the example)
    sel = idx.cpu().numpy().astype(np.int64)
    cu_h = inp["cu"].astype(np.int64)
    ex = np.searchsorted(cu_h, sel, side="right") - 1
    glob_pairs = float((sel - cu_h[ex] + 1).sum())
    band_pairs = float(sum(np.minimum(W, np.arange(n, dtype=np.float64) + 1).sum() for n in lens))
    F_loc, F_glb = 4.0 * d * Hq * band_pairs, 4.0 * d * Hq * glob_pairs
    tflops = (F_loc + F_glb) / (ms_per_step * 1e-3) / 1e12
    avg = {s: (stage_ms[j] / stage_n[j] if stage_n[j] else None) for j, s in enumerate(T.STAGES)}
    if avg.get("fused"):
        # the single launch: both branches of every example (its FLOPs are all of them)
        dom, dF = "fused", F_loc + F_glb
        kname = "attn_bf16_fused_kernel (both branches, one launch, packed examples)"
    else:
        dom, dF = ("global", F_glb) if F_glb >= F_loc else ("local", F_loc)
        kname = f"attn_bf16_kernel ({dom} branch, packed examples)"
    achieved = dF / (avg[dom] * 1e-3) / 1e12 if avg[dom] else None
    result = {
        "metric": "effective attn TFLOP/s + ms/layer fwd over a packed batch of 65536 tokens "
                  "(9 examples, 32K down to 256), rho=0.2; % of bf16 MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "input_sha256": digest,
        "config": {"workload": "varlen64k", "lens": lens, "Hq": Hq, "Hkv": Hkv, "d": d,
                   "window": W, "rho": rho, "k_sel": K, "seed": args.seed, "mode": "varlen",
                   "parallelism": "none (1 GPU)"},
        "pct_of_bf16_peak": round(100.0 * tflops / BF16_PEAK_TFLOPS, 2),
        "effective_flops": F_loc + F_glb,
        "stage_ms_avg": {s: round(x, 4) for s, x in avg.items() if x is not None},
        "per_step_ms": per_step,
        "roofline": {
            "kernel": kname,
            "bound": "mfma",
            "achieved": round(achieved, 2) if achieved else None,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4) if achieved else None,
            "traffic": None,
            "algorithmic_flops_per_launch": dF,
            "avg_launch_ms": round(avg[dom], 4) if avg[dom] else None,
        },
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa32k")
    ap.add_argument("--rho", type=float, default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--mode", choices=("forward", "train", "routed", "decode", "varlen"),
                    default="forward",
                    help="forward: one logo_forward per step (the headline); train: one "
                         "logo_forward_train + logo_backward per step; routed: one "
                         "logo_forward_routed per step (gate computed from the local branch); "
                         "decode: one logo_decode_step of the 128K decode workload per step; "
                         "varlen: one logo_forward_varlen over a packed 64K-token batch")
    ap.add_argument("--record-traffic", action="store_true",
                    help="write profiles/traffic.json from rocprofv3 counter csv directories "
                         "(--copy-fetch, --copy-write, --fwd-fetch, --fwd-write, optionally "
                         "--train-fetch, --train-write) and exit; needs no GPU")
    for opt in ("copy-fetch", "copy-write", "fwd-fetch", "fwd-write", "train-fetch",
                "train-write", "traffic-out"):
        ap.add_argument("--" + opt, default=None)
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="time a plain bf16 GEMM on random and on zero operands and exit")
    ap.add_argument("--ceilings", action="store_true",
                    help="run the matrix-core, LDS and exp2 throughput microbenchmarks "
                         "(libceiling.so) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (read N, write N "
                         "bytes) so HBM counters can be scaled to bytes")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library runs on one GPU and has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        return 2

    if args.record_traffic:
        return record_traffic(args)

    import torch

    import token_level_dynamic_amd as T
    from workloads import get_workload, make_inputs

    if args.copy_calibration:
        return copy_calibration(torch)
    if args.gemm_ceiling:
        return gemm_ceiling(torch)
    if args.ceilings:
        return ceilings(torch)

    from token_level_dynamic_amd._lib import LIB_PATH
    if not os.path.exists(LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    T.lib()

    w = get_workload(args.workload)
    if args.rho is not None:
        w = w.with_(rho=args.rho)
    inp = None
    if args.mode == "forward":
        inp = make_inputs(w, args.seed)
        if not args.no_cpu_baseline:
            start_cpu_oracle(w, inp)     # before the GPU is touched
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    if args.mode == "decode":
        return decode_bench(args, torch, T)
    if args.mode == "varlen":
        return varlen_bench(args, torch, T)
    if inp is None:
        inp = make_inputs(w, args.seed)
    if w.dtype == "bf16":
        digest = input_sha256(inp.q_bits, inp.k_bits, inp.v_bits, inp.gate)
    else:
        digest = input_sha256(inp.q, inp.k, inp.v, inp.gate)
    dev = torch.device("cuda:0")
    if w.dtype == "bf16":
        def cv(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        q, k, v = cv(inp.q_bits), cv(inp.k_bits), cv(inp.v_bits)
    else:
        q, k, v = (torch.from_numpy(x).to(dev) for x in (inp.q, inp.k, inp.v))
    gate = torch.from_numpy(inp.gate).to(dev)
    p = T.make_problem(w.B, w.Hq, w.Hkv, w.n, w.d, w.window, w.rho, dtype=w.dtype)
    if args.mode == "train":
        return train_bench(args, torch, T, w, inp, p, q, k, v, gate, dev, digest)
    if args.mode == "routed":
        return routed_bench(args, torch, T, w, inp, p, q, k, v, dev, digest)
    buf = T.alloc_forward_buffers(p, dev)

    def step():
        T.logo_forward(p, q, k, v, gate, buf["o"], buf["mask"], buf["idx"], buf["rank"],
                       buf["workspace"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    T.logo_profile_begin()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    stage_ms, stage_n = T.logo_profile_end()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    per_step = per_step_timing(torch, step, stream, args.steps)

    idx = buf["idx"].cpu().numpy()
    F = effective_flops(w, idx)
    tflops = F["total"] / (ms_per_step * 1e-3) / 1e12
    avg = {s: (stage_ms[j] / stage_n[j] if stage_n[j] else None)
           for j, s in enumerate(T.STAGES)}
    if avg.get("fused"):
        # one launch computes both branches: its FLOPs are the layer's
        dom, dom_flops = "fused", F["total"]
        kname = "attn_bf16_fused_kernel (both branches, one launch)"
    elif avg.get("pair"):
        # the local band and the key-range-split global branch in one launch,
        # then their merge: the layer's FLOPs over both kernels' time
        dom, dom_flops = "pair", F["total"]
        kname = ("attn_bf16_pair_kernel + global_merge_kernel (both branches, one launch, "
                 "split key ranges)")
    else:
        dom = "global" if F["global"] >= F["local"] else "local"
        dom_flops = F[dom]
        kname = f"attn_bf16_kernel ({dom} branch, fused epilogue)"
    dom_ms = avg[dom]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12 if dom_ms else None
    traffic = (load_traffic(w.name, kernel_source_hash(), f"{dom}_bytes_per_launch")
               if dom in ("global", "fused") else None)

    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "input_sha256": digest,
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "n": w.n,
                   "d": w.d, "window": w.window, "rho": w.rho,
                   "k_sel": int(T.logo_target_count(w.rho, w.n)), "seed": args.seed,
                   "parallelism": "none (1 GPU)"},
        "pct_of_bf16_peak": round(100.0 * tflops / BF16_PEAK_TFLOPS, 2),
        "effective_flops": F["total"],
        "stage_ms_avg": {s: round(x, 4) for s, x in avg.items() if x is not None},
        "per_step_ms": per_step,
        "timing": {"primary": "warm: value and ms_per_step are the K timed steps run back to "
                              "back (the benchmark's contract); per_step_ms.cold times each "
                              "forward after a 1 GiB write that evicts L2 and the MALL",
                   "cold_median_ms": per_step["cold"]["median_ms"]},
        "roofline": {
            "kernel": kname,
            "bound": "mfma",
            "achieved": round(achieved, 2) if achieved else None,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4) if achieved else None,
            "traffic": traffic,
            "algorithmic_flops_per_launch": dom_flops,
            "avg_launch_ms": round(dom_ms, 4) if dom_ms else None,
        },
    }
    if dom == "fused" and dom_ms:
        # the single launch derives both outputs of a selected row's window
        # pairs from one product each: its distinct pair work, and the rate on it
        result["roofline"]["distinct_pair_flops_per_launch"] = F["distinct"]
        result["roofline"]["frac_of_distinct_pairs"] = round(
            F["distinct"] / (dom_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, buf["o"], budget_s=args.cpu_budget)
        result["parity"] = result["cpu_baseline"]["parity"]
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
