"""bench.py's host-side contract: the one-GPU guard, and the reduction of
rocprofv3 counter runs into traffic.json. No GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counters(path, counter, kernels):
    """A rocprofv3-style counter csv: kernels = {name: [values per dispatch]},
    each value split over two rows (two shader engines)."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        did = 0
        for name, vals in kernels.items():
            for v in vals:
                did += 1
                for part in (0.25 * v, 0.75 * v):
                    w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                                "Counter_Value": part})


def test_record_traffic(tmp_path):
    g = "void logo::attn_bf16_kernel<128, true, 3, false, false>(Params)"
    lo = "void logo::attn_bf16_kernel<128, false, 1, false, false>(Params)"
    add = "void at::native::vectorized_elementwise_kernel<4, CUDAFunctorOnSelf_add<float>>"
    gib_kib = (1 << 30) / 1024
    # FETCH_SIZE reads half of what a streaming read moves, WRITE_SIZE all of it
    _counters(tmp_path / "cf", "FETCH_SIZE", {add: [gib_kib / 2] * 3})
    _counters(tmp_path / "cw", "WRITE_SIZE", {add: [gib_kib] * 3})
    # the mean of the first three dispatches is taken; later ones are ignored
    _counters(tmp_path / "ff", "FETCH_SIZE", {g: [1000, 1002, 1004, 9999], lo: [10, 10, 10]})
    _counters(tmp_path / "fw", "WRITE_SIZE", {g: [50, 50, 50, 9999], lo: [7, 7, 7]})
    out = tmp_path / "traffic.json"
    args = bench.argparse.Namespace(copy_fetch=str(tmp_path / "cf"),
                                    copy_write=str(tmp_path / "cw"),
                                    fwd_fetch=str(tmp_path / "ff"), fwd_write=str(tmp_path / "fw"),
                                    train_fetch=None, train_write=None, traffic_out=str(out))
    assert bench.record_traffic(args) == 0
    d = json.loads(out.read_text())["gqa32k"]
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert d["global_read_bytes"] == round(1002 * 1024 * 2)
    assert d["global_write_bytes"] == 50 * 1024
    assert d["global_bytes_per_launch"] == d["global_read_bytes"] + d["global_write_bytes"]
    assert d["local_bytes_per_launch"] == (10 * 2 + 7) * 1024
    assert d["source_hash"] == bench.kernel_source_hash()


def test_input_digest_follows_the_seed():
    # the bench line's input_sha256: same workload and seed -> same digest;
    # another seed or another array order -> another
    from workloads import get_workload, make_inputs
    w = get_workload("gqa32k", B=1, Hq=2, Hkv=1, n=64, window=16, rho=0.25)
    a, b, c = make_inputs(w, 0), make_inputs(w, 0), make_inputs(w, 1)
    da = bench.input_sha256(a.q_bits, a.k_bits, a.v_bits, a.gate)
    assert da == bench.input_sha256(b.q_bits, b.k_bits, b.v_bits, b.gate)
    assert da != bench.input_sha256(c.q_bits, c.k_bits, c.v_bits, c.gate)
    assert da != bench.input_sha256(a.k_bits, a.q_bits, a.v_bits, a.gate)
    assert len(da) == 16


def test_cpu_baseline_protocol():
    # the oracle leg: a pool of worker processes over the host's cores, the
    # selection computed once, a labelled extrapolation, host details, and
    # the sampled rows compared with an output (here the oracle's own, so
    # the difference is zero)
    import torch
    import oracle
    from workloads import get_workload, make_inputs
    w = get_workload("gqa32k", B=1, Hq=2, Hkv=1, n=300, window=40, rho=0.25)
    inp = make_inputs(w, 0)
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.gate, w.window, w.rho)
    bench.start_cpu_oracle(w, inp)
    out = bench.cpu_baseline(w, torch.from_numpy(ref["o"]), budget_s=1.0, chunk=8)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s" and out["value"] > 0
    assert out["cores"] == bench.cpu_cores() >= 1
    assert out["extrapolated"]["layer_s"] > 0
    assert out["parity"]["rows"] >= 8 and out["parity"]["max_abs"] < 1e-12
    assert "cpu_model" in out["host"] and "blas" in out["host"]
