"""logo_forward_noalloc (the forward on the library's own scratch array, for
callers that cannot allocate) against logo_forward with a caller workspace:
the same kernels on the same inputs, so every output must be identical, bit
for bit. Two calls in a row, the second on a smaller problem, so the array's
leftover contents from the first must not leak into the second; a problem
whose global branch splits key ranges (partials in the scratch) and one with
fewer (batch, kv head) units than XCDs (zeroed queue counters in it); the
headline layer; and the refusal of a problem too large for the array."""
import ctypes

import numpy as np
import pytest
import torch

import token_level_dynamic_amd as T
from token_level_dynamic_amd import _lib
from gpu_util import dev, ensure_built, global_splits, problem, say, to_dev
from workloads import get_workload, make_inputs


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _both(w, seed):
    p = problem(w)
    inp = make_inputs(w, seed)
    q, k, v, gate = to_dev(inp)
    ref = T.alloc_forward_buffers(p, dev())
    T.logo_forward(p, q, k, v, gate, ref["o"], ref["mask"], ref["idx"], ref["rank"],
                   ref["workspace"])
    got = {key: torch.full_like(ref[key], 7) for key in ("o", "mask", "idx", "rank")}
    T.logo_forward_noalloc(p, q, k, v, gate, got["o"], got["mask"], got["idx"], got["rank"])
    torch.cuda.synchronize()
    return p, ref, got


def _same(ref, got, label):
    for key in ("mask", "idx", "rank"):
        assert torch.equal(ref[key], got[key]), (label, key)
    a = ref["o"].view(torch.int16) if ref["o"].dtype == torch.bfloat16 else ref["o"]
    b = got["o"].view(torch.int16) if got["o"].dtype == torch.bfloat16 else got["o"]
    assert torch.equal(a, b), (label, "o")
    say(f"  {label}: outputs identical to logo_forward")


@pytest.mark.gpu
def test_noalloc_matches_forward_twice_second_smaller():
    big = get_workload("gqa32k", B=2, Hq=8, Hkv=2, n=5000, window=300, rho=0.2)
    small = get_workload("gqa32k", B=1, Hq=4, Hkv=2, n=1100, window=128, rho=0.3)
    for label, w in (("first call", big), ("second call, smaller", small)):
        say(f"[noalloc] {label}: {w}")
        _, ref, got = _both(w, 1)
        _same(ref, got, label)


@pytest.mark.gpu
def test_noalloc_split_and_queue_paths():
    # few selected rows: the global branch splits key ranges (partials live
    # in the scratch); B * Hkv < 8: the queue counters live there too
    w = get_workload("mha4k")
    p = problem(w)
    assert global_splits(p)
    _, ref, got = _both(w, 0)
    _same(ref, got, "mha4k (split key ranges)")
    w = get_workload("gqa32k", B=1, Hq=8, Hkv=2, n=9000, window=512, rho=0.2)
    _, ref, got = _both(w, 2)
    _same(ref, got, "B*Hkv = 2 (queued global branch)")
    w = get_workload("tiny")
    _, ref, got = _both(w, 3)
    _same(ref, got, "tiny float32")


@pytest.mark.gpu
def test_noalloc_headline_layer():
    w = get_workload("gqa32k")
    p = problem(w)
    size = ctypes.c_size_t(0)
    assert T.lib().logo_workspace_size(ctypes.byref(p), ctypes.byref(size)) == 0
    assert 0 < size.value <= _lib.NOALLOC_SCRATCH_BYTES
    say(f"[noalloc] headline layer, {size.value} of {_lib.NOALLOC_SCRATCH_BYTES} bytes")
    _, ref, got = _both(w, 0)
    _same(ref, got, "gqa32k")


def test_noalloc_refuses_a_problem_beyond_its_array():
    # host-side check, before anything is enqueued: no GPU needed
    w = get_workload("gqa128k")
    p = problem(w)
    size = ctypes.c_size_t(0)
    L = T.lib()
    assert L.logo_workspace_size(ctypes.byref(p), ctypes.byref(size)) == 0
    assert size.value > _lib.NOALLOC_SCRATCH_BYTES
    st = L.logo_forward_noalloc(ctypes.byref(p), None, None, None, None, None, None, None, None,
                                None)
    assert st == _lib.LOGO_ERR_WORKSPACE
    assert b"logo_forward_noalloc holds" in L.logo_last_error()


def test_noalloc_header_constant_matches_binding():
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    text = open(os.path.join(root, "include", "logo.h")).read()
    m = re.search(r"#define LOGO_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)", text)
    assert m and int(m[1]) * int(m[2]) * int(m[3]) == _lib.NOALLOC_SCRATCH_BYTES
