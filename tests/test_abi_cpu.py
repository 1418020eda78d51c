"""The C ABI on the CPU: the library loads, exports every entry point the
header declares, and rejects bad arguments before enqueueing anything (no
call here reaches a kernel launch). No GPU."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import token_level_dynamic_amd as T
from token_level_dynamic_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "logo.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return T.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(logo_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("logo_select_queries", "logo_local_attn", "logo_global_attn_sparse",
                 "logo_combine", "logo_forward", "logo_target_count", "logo_workspace_size"):
        assert want in names


def test_every_declared_symbol_is_exported(L):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(logo_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_target_count(L):
    for rho, n, k in [(0.2, 32768, 6554), (0.25, 256, 64), (0.2, 131072, 26215),
                      (0.05, 65536, 3277), (0.0, 10, 0), (1.0, 10, 10), (0.11, 10, 2)]:
        assert T.logo_target_count(rho, n) == k
    assert T.logo_target_count(math.nan, 10) == -1
    assert T.logo_target_count(0.5, -1) == -1


def _prob(**kw):
    base = dict(B=2, Hq=4, Hkv=2, n=100, d=128, window=16, rho=0.2, scale=0.0, dtype=1)
    base.update(kw)
    return _lib.logo_problem(**base)


FAKE = 1 << 20          # an aligned non-null address; never dereferenced here
MISALIGNED = FAKE + 4


def _forward(L, p, q=FAKE, k=FAKE, v=FAKE, gate=FAKE, o=FAKE, mask=FAKE, idx=FAKE,
             rank=FAKE, ws=None, ws_bytes=0):
    return L.logo_forward(ctypes.byref(p) if p is not None else None, q, k, v, gate, o, mask,
                          idx, rank, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=3, Hkv=2), _lib.LOGO_ERR_INVALID_ARG),
    (dict(rho=-0.1), _lib.LOGO_ERR_INVALID_ARG),
    (dict(rho=1.5), _lib.LOGO_ERR_INVALID_ARG),
    (dict(rho=math.nan), _lib.LOGO_ERR_INVALID_ARG),
    (dict(window=0), _lib.LOGO_ERR_INVALID_ARG),
    (dict(d=96), _lib.LOGO_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.LOGO_ERR_INVALID_ARG),
    (dict(scale=-1.0), _lib.LOGO_ERR_INVALID_ARG),
    (dict(scale=math.inf), _lib.LOGO_ERR_INVALID_ARG),
    (dict(n=-1), _lib.LOGO_ERR_INVALID_ARG),
    (dict(Hkv=0), _lib.LOGO_ERR_INVALID_ARG),
    (dict(n=1 << 31), _lib.LOGO_ERR_UNSUPPORTED),
])
def test_problem_validation(L, kw, status):
    p = _prob(**kw)
    assert _forward(L, p) == status
    assert L.logo_last_error()
    size = ctypes.c_size_t(123)
    assert L.logo_workspace_size(ctypes.byref(p), ctypes.byref(size)) == status
    assert L.logo_local_attn(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None) == status


def test_null_problem(L):
    assert _forward(L, None) == _lib.LOGO_ERR_INVALID_ARG


@pytest.mark.parametrize("field", ["q", "k", "v", "gate", "o", "mask", "idx", "rank"])
def test_null_and_misaligned_pointers(L, field):
    p = _prob()
    assert _forward(L, p, **{field: None}) == _lib.LOGO_ERR_INVALID_ARG
    assert field.encode() in L.logo_last_error()
    assert _forward(L, p, **{field: MISALIGNED}) == _lib.LOGO_ERR_INVALID_ARG


def test_workspace_checks(L):
    p = _prob()
    size = ctypes.c_size_t(0)
    assert L.logo_workspace_size(ctypes.byref(p), ctypes.byref(size)) == 0
    k = T.logo_target_count(0.2, 100)
    want = 2 * 4 * k * 128 * 4           # float32 local outputs of the selected rows
    # + B*Hkv int32 queues + the unselected positions (single-launch forward:
    # bf16, no key-range split, B*Hkv = 4 divides the 8 XCDs)
    assert size.value == (want + 255) // 256 * 256 + 256 + _round(2 * (100 - k) * 4)
    assert _forward(L, p, ws=None) == _lib.LOGO_ERR_WORKSPACE
    assert _forward(L, p, ws=FAKE, ws_bytes=size.value - 1) == _lib.LOGO_ERR_WORKSPACE
    # rho = 0 selects nothing: no workspace needed
    p0 = _prob(rho=0.0)
    assert L.logo_workspace_size(ctypes.byref(p0), ctypes.byref(size)) == 0
    assert size.value == 0


def _ws_bytes(L, **kw):
    p = _prob(**kw)
    size = ctypes.c_size_t(0)
    assert L.logo_workspace_size(ctypes.byref(p), ctypes.byref(size)) == 0
    return size.value


def _round(x):
    return (x + 255) // 256 * 256


def test_workspace_split_partials(L):
    # A bf16 problem with fewer than 512 global row-block workgroups splits
    # each block's keys over ceil(512 / workgroups) ranges, or, when the
    # local band's workgroups (every row) and two ranges per global block fit
    # in 512, over the most ranges that still fit beside them; at most 8 and
    # at least 4 key tiles of 64 each. The workspace then adds
    # splits * B * Hq * k * (d + 4) float32 partials.
    # n=1000, rho=0.2: k=200, 7 row blocks x 2 heads per (b, kv head) = 4
    # workgroups each, 16 in all; 64 local workgroups; 16 key tiles -> 4 ranges
    k = T.logo_target_count(0.2, 1000)
    base = _round(2 * 4 * k * 128 * 4) + 256
    assert _ws_bytes(L, n=1000) == base + _round(4 * 2 * 4 * k * (128 + 4) * 4)
    # d = 64, n = 4000: k=800, 13 global workgroups per (b, kv head), 52 in
    # all; 4 x 63 = 252 local workgroups; (512 - 252) // 52 = 5 ranges
    k = T.logo_target_count(0.2, 4000)
    base = _round(2 * 4 * k * 64 * 4) + 256
    assert _ws_bytes(L, n=4000, d=64) == base + _round(5 * 2 * 4 * k * (64 + 4) * 4)
    # B=2, 16 query / 4 kv heads, n = 4000: k=800, 25 x 4 units -> 25
    # global workgroups per (b, kv head), 200 in all; 2 x 4 x 125 = 1000
    # local workgroups do not fit beside them: ceil(512 / 200) = 3 ranges
    k = T.logo_target_count(0.2, 4000)
    base = _round(2 * 16 * k * 128 * 4) + 256
    assert _ws_bytes(L, n=4000, Hq=16, Hkv=4) == base + _round(3 * 2 * 16 * k * (128 + 4) * 4)
    # two key tiles: too few to split (single launch: + unselected positions);
    # float32: never split, never a single launch
    assert _ws_bytes(L, n=100) == _round(2 * 4 * 20 * 128 * 4) + 256 + _round(2 * 80 * 4)
    assert _ws_bytes(L, n=1000, dtype=0) == _round(2 * 4 * 200 * 128 * 4) + 256
    # 32K positions, 16 query / 4 kv heads: 1640 workgroups, no split;
    # B * Hkv = 8: the single launch
    k = T.logo_target_count(0.2, 32768)
    assert _ws_bytes(L, n=32768, Hq=16, Hkv=4) == (_round(2 * 16 * k * 128 * 4) + 256
                                                  + _round(2 * (32768 - k) * 4))
    # B * Hkv = 6 does not map onto the 8 XCDs: two launches, no list
    k = T.logo_target_count(0.2, 32768)
    assert _ws_bytes(L, n=32768, B=3, Hq=8, Hkv=2) == _round(3 * 8 * k * 128 * 4) + 256


def test_empty_problems_enqueue_nothing(L):
    for kw in (dict(B=0), dict(n=0)):
        p = _prob(**kw)
        assert _forward(L, p, q=None, k=None, v=None, gate=None, o=None, mask=None, idx=None,
                        rank=None) == 0
        assert L.logo_select_queries(ctypes.byref(p), None, None, None, None, None) == 0
        assert L.logo_combine(ctypes.byref(p), None, None, None, None, None, None) == 0


def test_status_strings(L):
    for s in range(5):
        assert L.logo_status_string(s)
    assert L.logo_status_string(99) == b"unknown status"


def test_profile_end_argument_check(L):
    assert L.logo_profile_begin() == 0
    assert L.logo_profile_end(None, None, 4) == _lib.LOGO_ERR_INVALID_ARG
    assert L.logo_profile_end(None, None, 0) == 0


def test_no_undefined_kernel_stubs(L):
    """Every kernel launch stub is defined in the library: a device-only
    construct that fails on the host compile pass can otherwise drop a stub
    silently and leave the library unloadable on the GPU side."""
    out = subprocess.run(["nm", "-D", "--undefined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert "device_stub" not in out, [l for l in out.splitlines() if "device_stub" in l]


def _ws_status(L, **kw):
    p = _prob(**kw)
    size = ctypes.c_size_t(0)
    return L.logo_workspace_size(ctypes.byref(p), ctypes.byref(size))


def _strides(**kw):
    out = {}
    for name, st in kw.items():
        arr = (ctypes.c_int64 * 3)(*st)
        out[f"{name}_strides"] = arr
    return out


@pytest.mark.parametrize("kw,status", [
    # bshd layouts (token stride H*d): valid for inputs and outputs
    (dict(q=(100 * 4 * 128, 128, 4 * 128), o=(100 * 4 * 128, 128, 4 * 128)), 0),
    # k, v as halves of one fused [B][n][2][Hkv][d] buffer
    (dict(k=(100 * 2 * 2 * 128, 128, 2 * 2 * 128), v=(100 * 2 * 2 * 128, 128, 2 * 2 * 128)), 0),
    # inputs may broadcast over batch / heads
    (dict(k=(0, 0, 128), v=(0, 100 * 128, 128)), 0),
    # padded token rows
    (dict(q=(4 * 100 * 136, 100 * 136, 136)), 0),
    (dict(q=(4 * 100 * 128, 100 * 128, -128)), _lib.LOGO_ERR_INVALID_ARG),
    (dict(k=(0, 0, 64)), _lib.LOGO_ERR_INVALID_ARG),            # token stride < d
    (dict(v=(0, 0, 132)), _lib.LOGO_ERR_INVALID_ARG),           # 264 B: not 16-B multiple
    (dict(o=(100 * 128, 0, 128)), _lib.LOGO_ERR_INVALID_ARG),   # heads overlap
    (dict(o=(4 * 100 * 128, 128, 128)), _lib.LOGO_ERR_INVALID_ARG),  # tokens and heads overlap
    (dict(o=(0, 100 * 128, 128)), _lib.LOGO_ERR_INVALID_ARG),   # batches overlap (B = 2)
])
def test_stride_validation(L, kw, status):
    assert _ws_status(L, **_strides(**kw)) == status, L.logo_last_error()


def test_stride_span_limit(L):
    n = 1 << 20
    ok = _strides(k=(0, 0, 128))
    assert _ws_status(L, n=n, **ok) == 0
    big = _strides(k=(0, 0, 1040))      # one sequence spans over 2 GiB of bf16
    assert _ws_status(L, n=n, **big) == _lib.LOGO_ERR_UNSUPPORTED
    # the same stride in float32 with fewer tokens fits
    assert _ws_status(L, n=1 << 18, dtype=0, **big) == 0


def test_problem_struct_layout_matches_header(tmp_path):
    """The ctypes mirror of logo_problem has the C struct's size and offsets."""
    src = tmp_path / "layout.c"
    fields = [f for f, _ in _lib.logo_problem._fields_]
    body = "".join(f'  printf("{f} %zu\\n", offsetof(logo_problem, {f}));\n' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "logo.h"\n'
                   'int main(void) {\n' + body +
                   '  printf("size %zu\\n", sizeof(logo_problem));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True,
                                                        text=True, check=True).stdout.split("\n")
               if line)
    for f in fields:
        assert int(out[f]) == getattr(_lib.logo_problem, f).offset, f
    assert int(out["size"]) == ctypes.sizeof(_lib.logo_problem)


def _backward(L, p, ws=None, ws_bytes=0, **ptrs):
    names = ["q", "k", "v", "gate", "o", "dout", "idx", "rank", "lse_local", "lse_global",
             "o_local_sel", "o_global", "dq", "dk", "dv", "dgate"]
    args = [ptrs.get(nm, FAKE) for nm in names]
    return L.logo_backward(ctypes.byref(p), *args, ws, ws_bytes, None)


def test_backward_workspace_size(L):
    p = _prob()
    size = ctypes.c_size_t(0)
    assert L.logo_backward_workspace_size(ctypes.byref(p), ctypes.byref(size)) == 0
    k = T.logo_target_count(0.2, 100)
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    want = 2 * (up(2 * 4 * 100 * 4) + up(2 * 4 * k * 4)) + 2 * up(2 * 4 * k * 128 * 2)
    assert size.value == want
    p32 = _prob(dtype=0)
    assert L.logo_backward_workspace_size(ctypes.byref(p32), ctypes.byref(size)) == 0
    assert size.value == 2 * (up(2 * 4 * 100 * 4) + up(2 * 4 * k * 4)) + \
        2 * up(2 * 4 * k * 128 * 4)


@pytest.mark.parametrize("field", ["q", "k", "v", "gate", "o", "dout", "idx", "rank",
                                   "lse_local", "lse_global", "o_local_sel", "o_global", "dq",
                                   "dk", "dv", "dgate"])
def test_backward_null_pointers(L, field):
    p = _prob()
    assert _backward(L, p, ws=FAKE, ws_bytes=1 << 30, **{field: None}) == \
        _lib.LOGO_ERR_INVALID_ARG
    assert field.encode() in L.logo_last_error()
    assert _backward(L, p, ws=FAKE, ws_bytes=1 << 30, **{field: MISALIGNED}) == \
        _lib.LOGO_ERR_INVALID_ARG


def test_backward_workspace_checks(L):
    p = _prob()
    assert _backward(L, p) == _lib.LOGO_ERR_WORKSPACE
    size = ctypes.c_size_t(0)
    L.logo_backward_workspace_size(ctypes.byref(p), ctypes.byref(size))
    assert _backward(L, p, ws=FAKE, ws_bytes=size.value - 1) == _lib.LOGO_ERR_WORKSPACE
    assert _backward(L, p, ws=MISALIGNED, ws_bytes=size.value) == _lib.LOGO_ERR_INVALID_ARG


def test_forward_train_validation(L):
    p = _prob()
    names = ["q", "k", "v", "gate", "o", "mask", "idx", "rank", "lse_local", "lse_global",
             "o_local_sel", "o_global"]
    for nm in names:
        args = [None if x == nm else FAKE for x in names]
        assert L.logo_forward_train(ctypes.byref(p), *args, None) == _lib.LOGO_ERR_INVALID_ARG
        assert nm.encode() in L.logo_last_error()
    # empty problems enqueue nothing and accept NULL everywhere
    p0 = _prob(n=0)
    assert L.logo_forward_train(ctypes.byref(p0), *([None] * 12), None) == 0
    assert L.logo_backward(ctypes.byref(p0), *([None] * 16), None, 0, None) == 0


# ---- decode step ---------------------------------------------------------------

def _dprob(**kw):
    base = dict(B=3, Hq=8, Hkv=2, cap=5000, d=128, window=64, rho=0.25, eta=0.1, scale=0.0,
                dtype="bf16")
    base.update(kw)
    return T.make_decode_problem(**base)


def _dsize(L, p):
    size = ctypes.c_size_t(0)
    st = L.logo_decode_workspace_size(ctypes.byref(p), ctypes.byref(size))
    return st, size.value


def test_decode_group_sizes(L):
    # bf16 caches of at most 1023 sequences: any group up to 16
    for hq, hkv in ((3, 1), (12, 4), (16, 1), (10, 2)):
        assert _dsize(L, _dprob(Hq=hq, Hkv=hkv))[0] == 0


def test_decode_workspace_formula(L):
    # one (d + 4)-float record per (b, query head, 1024-key chunk, branch)
    st, size = _dsize(L, _dprob())
    assert st == 0
    want = 3 * 8 * math.ceil(5000 / 1024) * 2 * (128 + 4) * 4
    assert size == (want + 255) // 256 * 256
    st, size = _dsize(L, _dprob(B=0))
    assert st == 0 and size == 0


@pytest.mark.parametrize("bad", [dict(Hq=6, Hkv=4), dict(Hq=0), dict(cap=0), dict(window=0),
                                 dict(rho=1.5), dict(rho=math.nan), dict(eta=-1.0),
                                 dict(eta=math.inf), dict(scale=math.nan), dict(B=-1)])
def test_decode_rejects_bad_problems(L, bad):
    st, _ = _dsize(L, _dprob(**bad))
    assert st == _lib.LOGO_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(d=96), dict(Hq=17, Hkv=1), dict(Hq=12, Hkv=4, dtype="f32"),
                                 dict(Hq=12, Hkv=4, B=1024), dict(cap=1 << 30),
                                 # work items beyond 32-bit counts
                                 dict(B=(1 << 19) - 1, Hq=64, Hkv=64, cap=1 << 20)])
def test_decode_unsupported_sizes(L, bad):
    st, _ = _dsize(L, _dprob(**bad))
    assert st == _lib.LOGO_ERR_UNSUPPORTED
    assert L.logo_last_error()


def test_decode_step_rejects_null_pointers_before_launching(L):
    p = _dprob()
    args = [FAKE] * 8  # q, k_cache, v_cache, lens, gate, tau, o, selected
    for i, name in enumerate(["q", "k_cache", "v_cache", "lens", "gate", "tau", "o", "selected"]):
        a = list(args)
        a[i] = None
        st = L.logo_decode_step(ctypes.byref(p), *a, FAKE, 1 << 30, None)
        assert st == _lib.LOGO_ERR_INVALID_ARG, name
        assert name.encode() in L.logo_last_error()
    # too small a workspace
    _, need = _dsize(L, p)
    st = L.logo_decode_step(ctypes.byref(p), *args, FAKE, need - 1, None)
    assert st == _lib.LOGO_ERR_WORKSPACE
