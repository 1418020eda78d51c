"""Helpers shared by the GPU tests: move seeded inputs to the device and run
the C ABI entry points. Holds no attention arithmetic."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import token_level_dynamic_amd as T


def ensure_built():
    from token_level_dynamic_amd._lib import LIB_PATH
    if not os.path.exists(LIB_PATH):
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        sys.path.insert(0, root)
        import __graft_entry__
        __graft_entry__.build()
    T.lib()


def dev():
    return torch.device("cuda:0")


def to_dev(inp):
    """Device tensors for q, k, v (bf16 bit patterns or float32) and the gate."""
    w = inp.workload
    if w.dtype == "bf16":
        def cv(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev())
        q, k, v = cv(inp.q_bits), cv(inp.k_bits), cv(inp.v_bits)
    else:
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())
                   for x in (inp.q, inp.k, inp.v))
    gate = torch.from_numpy(np.ascontiguousarray(inp.gate, dtype=np.float32)).to(dev())
    return q, k, v, gate


def problem(w, rho=None, scale=0.0):
    return T.make_problem(w.B, w.Hq, w.Hkv, w.n, w.d, w.window,
                          w.rho if rho is None else rho, scale, dtype=w.dtype)


def run_forward(p, q, k, v, gate):
    buf = T.alloc_forward_buffers(p, dev())
    T.logo_forward(p, q, k, v, gate, buf["o"], buf["mask"], buf["idx"], buf["rank"],
                   buf["workspace"])
    torch.cuda.synchronize()
    return buf


def run_unfused(p, q, k, v, gate):
    kk = T.logo_target_count(p.rho, p.n)
    d = dev()
    mask = torch.empty((p.B, p.n), dtype=torch.uint8, device=d)
    idx = torch.empty((p.B, kk), dtype=torch.int32, device=d)
    rank = torch.empty((p.B, p.n), dtype=torch.int32, device=d)
    o_local = torch.empty((p.B, p.Hq, p.n, p.d), dtype=torch.float32, device=d)
    o_global = torch.empty((p.B, p.Hq, kk, p.d), dtype=torch.float32, device=d)
    o = torch.empty((p.B, p.Hq, p.n, p.d), dtype=T.io_dtype(p), device=d)
    T.logo_select_queries(p, gate, mask, idx, rank)
    T.logo_local_attn(p, q, k, v, o_local)
    T.logo_global_attn_sparse(p, q, k, v, idx, o_global)
    T.logo_combine(p, o_local, o_global, rank, gate, o)
    torch.cuda.synchronize()
    return {"mask": mask, "idx": idx, "rank": rank, "o_local": o_local,
            "o_global": o_global, "o": o}


def host(t):
    return t.float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) \
        else t.cpu().numpy()


def say(msg):
    print(msg, flush=True)


def global_splits(p):
    """True when logo_forward splits this problem's global branch into key
    ranges: its workspace then holds more than the selected rows' float32
    local outputs and the (b, kv head) queue counters."""
    kk = T.logo_target_count(p.rho, p.n)

    def r256(x):
        return (x + 255) // 256 * 256
    base = r256(p.B * p.Hq * kk * p.d * 4) + (r256(4 * p.B * p.Hkv) if kk else 0)
    return p.dtype == 1 and T.logo_workspace_size(p) > base
