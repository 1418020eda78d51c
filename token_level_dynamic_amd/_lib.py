"""ctypes binding of liblogo.so (include/logo.h), argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of the method: it checks tensor placement, dtypes and shapes,
passes device pointers and the current HIP stream, and turns a non-zero
status into an exception. PyTorch supplies device memory and streams.
If the shared library is missing, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

# the in-tree build; LOGO_LIBRARY names another build of the same library
# (for example to compare two builds on one machine)
LIB_PATH = os.environ.get("LOGO_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "liblogo.so")

LOGO_OK = 0
LOGO_ERR_INVALID_ARG = 1
LOGO_ERR_UNSUPPORTED = 2
LOGO_ERR_WORKSPACE = 3
LOGO_ERR_HIP = 4
LOGO_F32 = 0
LOGO_BF16 = 1
STAGES = ("select", "local", "global", "combine", "bwd_prep", "bwd_dkdv", "bwd_dq",
          "router", "decode", "fused", "pair")


class LogoError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class logo_problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64),
        ("Hq", ctypes.c_int64),
        ("Hkv", ctypes.c_int64),
        ("n", ctypes.c_int64),
        ("d", ctypes.c_int64),
        ("window", ctypes.c_int64),
        ("rho", ctypes.c_double),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("q_strides", ctypes.c_int64 * 3),
        ("k_strides", ctypes.c_int64 * 3),
        ("v_strides", ctypes.c_int64 * 3),
        ("o_strides", ctypes.c_int64 * 3),
    ]


def make_problem(B: int, Hq: int, Hkv: int, n: int, d: int, window: int, rho: float,
                 scale: float = 0.0, dtype: str = "bf16", q_strides=None, k_strides=None,
                 v_strides=None, o_strides=None) -> logo_problem:
    """Problem description. `*_strides` are (batch, head, token) element
    strides of a strided [B][H][n][d] view (see view_strides); None means
    the contiguous layout."""
    dt = {"bf16": LOGO_BF16, "f32": LOGO_F32}[dtype]
    p = logo_problem(B, Hq, Hkv, n, d, window, float(rho), float(scale), dt)
    for name, st in (("q", q_strides), ("k", k_strides), ("v", v_strides), ("o", o_strides)):
        if st is not None:
            getattr(p, f"{name}_strides")[:] = [int(x) for x in st]
    return p


def view_strides(t: torch.Tensor) -> Tuple[int, int, int]:
    """(batch, head, token) element strides of a [B][H][n][d] view whose d
    elements are contiguous, for make_problem."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B][H][n][d] view with unit stride along d")
    return t.stride(0), t.stride(1), t.stride(2)


class logo_decode_problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64),
        ("Hq", ctypes.c_int64),
        ("Hkv", ctypes.c_int64),
        ("cap", ctypes.c_int64),
        ("d", ctypes.c_int64),
        ("window", ctypes.c_int64),
        ("rho", ctypes.c_double),
        ("eta", ctypes.c_float),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


def make_decode_problem(B: int, Hq: int, Hkv: int, cap: int, d: int, window: int, rho: float,
                        eta: float = 0.0, scale: float = 0.0,
                        dtype: str = "bf16") -> logo_decode_problem:
    dt = {"bf16": LOGO_BF16, "f32": LOGO_F32}[dtype]
    return logo_decode_problem(B, Hq, Hkv, cap, d, window, float(rho), float(eta), float(scale),
                               dt)


_lib = None
_P = ctypes.c_void_p
_PP = ctypes.POINTER(logo_problem)

_SIGS = {
    "logo_target_count": (ctypes.c_int64, [ctypes.c_double, ctypes.c_int64]),
    "logo_workspace_size": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_size_t)]),
    "logo_select_queries": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P]),
    "logo_local_attn": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P]),
    "logo_global_attn_sparse": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P]),
    "logo_combine": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P]),
    "logo_forward_noalloc": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "logo_forward": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P]),
    "logo_forward_train": (ctypes.c_int, [_PP] + [_P] * 13),
    "logo_backward_workspace_size": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_size_t)]),
    "logo_backward": (ctypes.c_int, [_PP] + [_P] * 17 + [ctypes.c_size_t, _P]),
    "logo_routed_workspace_size": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_size_t)]),
    "logo_forward_routed": (ctypes.c_int, [_PP, _P, _P, _P, _P, ctypes.c_float] + [_P] * 6 +
                            [ctypes.c_size_t, _P]),
    "logo_decode_workspace_size": (ctypes.c_int, [ctypes.POINTER(logo_decode_problem),
                                                   ctypes.POINTER(ctypes.c_size_t)]),
    "logo_decode_step": (ctypes.c_int, [ctypes.POINTER(logo_decode_problem)] + [_P] * 9 +
                         [ctypes.c_size_t, _P]),
    "logo_calibrate_threshold": (ctypes.c_int, [_PP, _P, _P, _P, _P]),
    "logo_select_threshold": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P]),
    "logo_varlen_selected_count": (ctypes.c_int64, [ctypes.c_double, _P, ctypes.c_int64]),
    "logo_varlen_workspace_size": (ctypes.c_int, [_PP, ctypes.c_int64, ctypes.c_int64,
                                                   ctypes.POINTER(ctypes.c_size_t)]),
    "logo_forward_varlen": (ctypes.c_int, [_PP, _P, ctypes.c_int64, ctypes.c_int64] + [_P] * 9 +
                            [ctypes.c_size_t, _P]),
    "logo_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "logo_last_error": (ctypes.c_char_p, []),
    "logo_profile_begin": (ctypes.c_int, []),
    "logo_profile_end": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_int32]),
}


def lib() -> ctypes.CDLL:
    """The loaded liblogo.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m token_level_dynamic_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != LOGO_OK:
        detail = lib().logo_last_error().decode(errors="replace")
        raise LogoError(status, where, detail)


def _ptr(t: Optional[torch.Tensor], name: str, strided: bool = False) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not strided and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def _strided(p: logo_problem, t: Optional[torch.Tensor], name: str, heads: int) -> bool:
    """True when the problem declares strides for this tensor; then t must be
    the [B][H][n][d] view those strides describe."""
    st = tuple(getattr(p, f"{name}_strides"))
    if st == (0, 0, 0) or t is None:
        return False
    if tuple(t.shape) != (p.B, heads, p.n, p.d) or view_strides(t) != st:
        raise ValueError(f"{name} must be a ({p.B}, {heads}, {p.n}, {p.d}) view with strides "
                         f"{st + (1,)}, got shape {tuple(t.shape)} strides {t.stride()}")
    return True


def _io(p: logo_problem, t: Optional[torch.Tensor], name: str, heads: int) -> Optional[int]:
    """Pointer of q, k, v or o: contiguous, or the strided view p declares."""
    dt = io_dtype(p)
    if _strided(p, t, name, heads):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        return _ptr(t, name, strided=True)
    _expect(t, name, dt, p.B * heads * p.n * p.d)
    return _ptr(t, name)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _expect(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, numel: int) -> None:
    if t is None:
        if numel:
            raise ValueError(f"{name} is required")
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def io_dtype(p: logo_problem) -> torch.dtype:
    return torch.bfloat16 if p.dtype == LOGO_BF16 else torch.float32


def logo_target_count(rho: float, n: int) -> int:
    return int(lib().logo_target_count(float(rho), int(n)))


def logo_workspace_size(p: logo_problem) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().logo_workspace_size(ctypes.byref(p), ctypes.byref(out)), "logo_workspace_size")
    return int(out.value)


def logo_select_queries(p: logo_problem, gate, mask, idx, rank, stream=None) -> None:
    k = logo_target_count(p.rho, p.n)
    _expect(gate, "gate", torch.float32, p.B * p.n)
    _expect(mask, "mask", torch.uint8, p.B * p.n)
    _expect(idx, "idx", torch.int32, p.B * k)
    _expect(rank, "rank", torch.int32, p.B * p.n)
    _check(lib().logo_select_queries(ctypes.byref(p), _ptr(gate, "gate"), _ptr(mask, "mask"),
                                     _ptr(idx, "idx"), _ptr(rank, "rank"), _stream(stream)),
           "logo_select_queries")


def _qkv(p: logo_problem, q, k, v) -> Tuple[Optional[int], Optional[int], Optional[int]]:
    return _io(p, q, "q", p.Hq), _io(p, k, "k", p.Hkv), _io(p, v, "v", p.Hkv)


def logo_local_attn(p: logo_problem, q, k, v, o_local, stream=None) -> None:
    qp, kp, vp = _qkv(p, q, k, v)
    _expect(o_local, "o_local", torch.float32, p.B * p.Hq * p.n * p.d)
    _check(lib().logo_local_attn(ctypes.byref(p), qp, kp, vp, _ptr(o_local, "o_local"),
                                 _stream(stream)), "logo_local_attn")


def logo_global_attn_sparse(p: logo_problem, q, k, v, idx, o_global, stream=None) -> None:
    kk = logo_target_count(p.rho, p.n)
    qp, kp, vp = _qkv(p, q, k, v)
    _expect(idx, "idx", torch.int32, p.B * kk)
    _expect(o_global, "o_global", torch.float32, p.B * p.Hq * kk * p.d)
    _check(lib().logo_global_attn_sparse(ctypes.byref(p), qp, kp, vp, _ptr(idx, "idx"),
                                         _ptr(o_global, "o_global"), _stream(stream)),
           "logo_global_attn_sparse")


def logo_combine(p: logo_problem, o_local, o_global, rank, gate, o, stream=None) -> None:
    kk = logo_target_count(p.rho, p.n)
    _expect(o_local, "o_local", torch.float32, p.B * p.Hq * p.n * p.d)
    _expect(o_global, "o_global", torch.float32, p.B * p.Hq * kk * p.d)
    _expect(rank, "rank", torch.int32, p.B * p.n)
    _expect(gate, "gate", torch.float32, p.B * p.n)
    op = _io(p, o, "o", p.Hq)
    _check(lib().logo_combine(ctypes.byref(p), _ptr(o_local, "o_local"),
                              _ptr(o_global, "o_global"), _ptr(rank, "rank"),
                              _ptr(gate, "gate"), op, _stream(stream)), "logo_combine")


def logo_forward(p: logo_problem, q, k, v, gate, o, mask, idx, rank, workspace,
                 stream=None) -> None:
    kk = logo_target_count(p.rho, p.n)
    qp, kp, vp = _qkv(p, q, k, v)
    _expect(gate, "gate", torch.float32, p.B * p.n)
    op = _io(p, o, "o", p.Hq)
    _expect(mask, "mask", torch.uint8, p.B * p.n)
    _expect(idx, "idx", torch.int32, p.B * kk)
    _expect(rank, "rank", torch.int32, p.B * p.n)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().logo_forward(ctypes.byref(p), qp, kp, vp,
                              _ptr(gate, "gate"), op, _ptr(mask, "mask"),
                              _ptr(idx, "idx"), _ptr(rank, "rank"),
                              _ptr(workspace, "workspace"), ws_bytes, _stream(stream)),
           "logo_forward")


# bytes of the scratch array logo_forward_noalloc uses (include/logo.h)
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024


def logo_forward_noalloc(p: logo_problem, q, k, v, gate, o, mask, idx, rank,
                         stream=None) -> None:
    """logo_forward without a workspace (the library's own scratch array)."""
    kk = logo_target_count(p.rho, p.n)
    qp, kp, vp = _qkv(p, q, k, v)
    _expect(gate, "gate", torch.float32, p.B * p.n)
    op = _io(p, o, "o", p.Hq)
    _expect(mask, "mask", torch.uint8, p.B * p.n)
    _expect(idx, "idx", torch.int32, p.B * kk)
    _expect(rank, "rank", torch.int32, p.B * p.n)
    _check(lib().logo_forward_noalloc(ctypes.byref(p), qp, kp, vp, _ptr(gate, "gate"), op,
                                      _ptr(mask, "mask"), _ptr(idx, "idx"), _ptr(rank, "rank"),
                                      _stream(stream)),
           "logo_forward_noalloc")


def logo_forward_train(p: logo_problem, q, k, v, gate, o, mask, idx, rank, lse_local,
                       lse_global, o_local_sel, o_global, stream=None) -> None:
    """Forward that also saves what logo_backward needs (see include/logo.h)."""
    kk = logo_target_count(p.rho, p.n)
    qp, kp, vp = _qkv(p, q, k, v)
    _expect(gate, "gate", torch.float32, p.B * p.n)
    op = _io(p, o, "o", p.Hq)
    _expect(mask, "mask", torch.uint8, p.B * p.n)
    _expect(idx, "idx", torch.int32, p.B * kk)
    _expect(rank, "rank", torch.int32, p.B * p.n)
    _expect(lse_local, "lse_local", torch.float32, p.B * p.Hq * p.n)
    _expect(lse_global, "lse_global", torch.float32, p.B * p.Hq * kk)
    _expect(o_local_sel, "o_local_sel", torch.float32, p.B * p.Hq * kk * p.d)
    _expect(o_global, "o_global", torch.float32, p.B * p.Hq * kk * p.d)
    _check(lib().logo_forward_train(
        ctypes.byref(p), qp, kp, vp, _ptr(gate, "gate"), op, _ptr(mask, "mask"),
        _ptr(idx, "idx"), _ptr(rank, "rank"), _ptr(lse_local, "lse_local"),
        _ptr(lse_global, "lse_global"), _ptr(o_local_sel, "o_local_sel"),
        _ptr(o_global, "o_global"), _stream(stream)), "logo_forward_train")


def logo_backward_workspace_size(p: logo_problem) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().logo_backward_workspace_size(ctypes.byref(p), ctypes.byref(out)),
           "logo_backward_workspace_size")
    return int(out.value)


def logo_backward(p: logo_problem, q, k, v, gate, o, dout, idx, rank, lse_local, lse_global,
                  o_local_sel, o_global, dq, dk, dv, dgate, workspace, stream=None) -> None:
    """Gradients dq, dk, dv (float32) and dgate for upstream gradient dout."""
    kk = logo_target_count(p.rho, p.n)
    qp, kp, vp = _qkv(p, q, k, v)
    _expect(gate, "gate", torch.float32, p.B * p.n)
    op = _io(p, o, "o", p.Hq)
    dop = _io(p, dout, "o", p.Hq)
    _expect(idx, "idx", torch.int32, p.B * kk)
    _expect(rank, "rank", torch.int32, p.B * p.n)
    _expect(lse_local, "lse_local", torch.float32, p.B * p.Hq * p.n)
    _expect(lse_global, "lse_global", torch.float32, p.B * p.Hq * kk)
    _expect(o_local_sel, "o_local_sel", torch.float32, p.B * p.Hq * kk * p.d)
    _expect(o_global, "o_global", torch.float32, p.B * p.Hq * kk * p.d)
    _expect(dq, "dq", torch.float32, p.B * p.Hq * p.n * p.d)
    _expect(dk, "dk", torch.float32, p.B * p.Hkv * p.n * p.d)
    _expect(dv, "dv", torch.float32, p.B * p.Hkv * p.n * p.d)
    _expect(dgate, "dgate", torch.float32, p.B * p.n)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().logo_backward(
        ctypes.byref(p), qp, kp, vp, _ptr(gate, "gate"), op, dop, _ptr(idx, "idx"),
        _ptr(rank, "rank"), _ptr(lse_local, "lse_local"), _ptr(lse_global, "lse_global"),
        _ptr(o_local_sel, "o_local_sel"), _ptr(o_global, "o_global"), _ptr(dq, "dq"),
        _ptr(dk, "dk"), _ptr(dv, "dv"), _ptr(dgate, "dgate"), _ptr(workspace, "workspace"),
        ws_bytes, _stream(stream)), "logo_backward")


def alloc_train_buffers(p: logo_problem, device="cuda") -> dict:
    """Output, selection and saved-statistics tensors for logo_forward_train."""
    kk = logo_target_count(p.rho, p.n)
    f32 = dict(dtype=torch.float32, device=device)
    return {
        "o": torch.empty((p.B, p.Hq, p.n, p.d), dtype=io_dtype(p), device=device),
        "mask": torch.empty((p.B, p.n), dtype=torch.uint8, device=device),
        "idx": torch.empty((p.B, kk), dtype=torch.int32, device=device),
        "rank": torch.empty((p.B, p.n), dtype=torch.int32, device=device),
        "lse_local": torch.empty((p.B, p.Hq, p.n), **f32),
        "lse_global": torch.empty((p.B, p.Hq, kk), **f32),
        "o_local_sel": torch.empty((p.B, p.Hq, kk, p.d), **f32),
        "o_global": torch.empty((p.B, p.Hq, kk, p.d), **f32),
    }


def alloc_backward_buffers(p: logo_problem, device="cuda") -> dict:
    """Gradient and workspace tensors for logo_backward."""
    ws = logo_backward_workspace_size(p)
    f32 = dict(dtype=torch.float32, device=device)
    return {
        "dq": torch.empty((p.B, p.Hq, p.n, p.d), **f32),
        "dk": torch.empty((p.B, p.Hkv, p.n, p.d), **f32),
        "dv": torch.empty((p.B, p.Hkv, p.n, p.d), **f32),
        "dgate": torch.empty((p.B, p.n), **f32),
        "workspace": torch.empty((ws,), dtype=torch.uint8, device=device) if ws else None,
    }


def logo_routed_workspace_size(p: logo_problem) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().logo_routed_workspace_size(ctypes.byref(p), ctypes.byref(out)),
           "logo_routed_workspace_size")
    return int(out.value)


def logo_forward_routed(p: logo_problem, q, k, v, router_w, router_bias: float, gate, o, mask,
                        idx, rank, workspace, stream=None) -> None:
    """Routed forward: local branch, router logits (written to `gate`),
    selection, global branch, combine (see include/logo.h)."""
    kk = logo_target_count(p.rho, p.n)
    qp, kp, vp = _qkv(p, q, k, v)
    _expect(router_w, "router_w", torch.float32, p.Hq * p.d)
    _expect(gate, "gate", torch.float32, p.B * p.n)
    op = _io(p, o, "o", p.Hq)
    _expect(mask, "mask", torch.uint8, p.B * p.n)
    _expect(idx, "idx", torch.int32, p.B * kk)
    _expect(rank, "rank", torch.int32, p.B * p.n)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().logo_forward_routed(
        ctypes.byref(p), qp, kp, vp, _ptr(router_w, "router_w"), float(router_bias),
        _ptr(gate, "gate"), op, _ptr(mask, "mask"), _ptr(idx, "idx"), _ptr(rank, "rank"),
        _ptr(workspace, "workspace"), ws_bytes, _stream(stream)), "logo_forward_routed")


def alloc_routed_buffers(p: logo_problem, device="cuda") -> dict:
    """Gate, output, selection and workspace tensors for logo_forward_routed."""
    kk = logo_target_count(p.rho, p.n)
    ws = logo_routed_workspace_size(p)
    return {
        "gate": torch.empty((p.B, p.n), dtype=torch.float32, device=device),
        "o": torch.empty((p.B, p.Hq, p.n, p.d), dtype=io_dtype(p), device=device),
        "mask": torch.empty((p.B, p.n), dtype=torch.uint8, device=device),
        "idx": torch.empty((p.B, kk), dtype=torch.int32, device=device),
        "rank": torch.empty((p.B, p.n), dtype=torch.int32, device=device),
        "workspace": torch.empty((ws,), dtype=torch.uint8, device=device) if ws else None,
    }


def logo_decode_workspace_size(p: logo_decode_problem) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().logo_decode_workspace_size(ctypes.byref(p), ctypes.byref(out)),
           "logo_decode_workspace_size")
    return int(out.value)


def logo_decode_step(p: logo_decode_problem, q, k_cache, v_cache, lens, gate, tau, o, selected,
                     workspace, stream=None) -> None:
    """One decode step (see include/logo.h); tau is updated in place."""
    dt = torch.bfloat16 if p.dtype == LOGO_BF16 else torch.float32
    _expect(q, "q", dt, p.B * p.Hq * p.d)
    _expect(k_cache, "k_cache", dt, p.B * p.Hkv * p.cap * p.d)
    _expect(v_cache, "v_cache", dt, p.B * p.Hkv * p.cap * p.d)
    _expect(lens, "lens", torch.int32, p.B)
    _expect(gate, "gate", torch.float32, p.B)
    _expect(tau, "tau", torch.float32, p.B)
    _expect(o, "o", dt, p.B * p.Hq * p.d)
    _expect(selected, "selected", torch.uint8, p.B)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().logo_decode_step(
        ctypes.byref(p), _ptr(q, "q"), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
        _ptr(lens, "lens"), _ptr(gate, "gate"), _ptr(tau, "tau"), _ptr(o, "o"),
        _ptr(selected, "selected"), _ptr(workspace, "workspace"), ws_bytes, _stream(stream)),
        "logo_decode_step")


def logo_calibrate_threshold(p: logo_problem, gate, mask, tau, stream=None) -> None:
    _expect(gate, "gate", torch.float32, p.B * p.n)
    _expect(mask, "mask", torch.uint8, p.B * p.n)
    _expect(tau, "tau", torch.float32, p.B)
    _check(lib().logo_calibrate_threshold(ctypes.byref(p), _ptr(gate, "gate"), _ptr(mask, "mask"),
                                          _ptr(tau, "tau"), _stream(stream)),
           "logo_calibrate_threshold")


def logo_select_threshold(p: logo_problem, gate, tau, mask, idx, count, stream=None) -> None:
    _expect(gate, "gate", torch.float32, p.B * p.n)
    _expect(tau, "tau", torch.float32, p.B)
    _expect(mask, "mask", torch.uint8, p.B * p.n)
    _expect(idx, "idx", torch.int32, p.B * p.n)
    _expect(count, "count", torch.int32, p.B)
    _check(lib().logo_select_threshold(ctypes.byref(p), _ptr(gate, "gate"), _ptr(tau, "tau"),
                                       _ptr(mask, "mask"), _ptr(idx, "idx"),
                                       _ptr(count, "count"), _stream(stream)),
           "logo_select_threshold")


def logo_varlen_selected_count(rho: float, cu_seqlens) -> int:
    """K = sum of ceil(rho * n_e) over the examples of host offsets cu_seqlens."""
    import numpy as np
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    return int(lib().logo_varlen_selected_count(float(rho), cu.ctypes.data, cu.size - 1))


def logo_varlen_workspace_size(p: logo_problem, n_examples: int, total_selected: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().logo_varlen_workspace_size(ctypes.byref(p), int(n_examples), int(total_selected),
                                            ctypes.byref(out)), "logo_varlen_workspace_size")
    return int(out.value)


def logo_forward_varlen(p: logo_problem, cu_seqlens, total_selected: int, q, k, v, gate, o, mask,
                        idx, rank, workspace, stream=None) -> None:
    """Forward over a packed batch (B = 1, n = total tokens); cu_seqlens is a
    device int32 tensor of E+1 offsets (see include/logo.h)."""
    E = cu_seqlens.numel() - 1
    _expect(cu_seqlens, "cu_seqlens", torch.int32, E + 1)
    qp, kp, vp = _qkv(p, q, k, v)
    _expect(gate, "gate", torch.float32, p.n)
    op = _io(p, o, "o", p.Hq)
    _expect(mask, "mask", torch.uint8, p.n)
    _expect(idx, "idx", torch.int32, total_selected)
    _expect(rank, "rank", torch.int32, p.n)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().logo_forward_varlen(
        ctypes.byref(p), _ptr(cu_seqlens, "cu_seqlens"), E, int(total_selected), qp, kp, vp,
        _ptr(gate, "gate"), op, _ptr(mask, "mask"), _ptr(idx, "idx"), _ptr(rank, "rank"),
        _ptr(workspace, "workspace"), ws_bytes, _stream(stream)), "logo_forward_varlen")


def logo_profile_begin() -> None:
    _check(lib().logo_profile_begin(), "logo_profile_begin")


def logo_profile_end() -> Tuple[list, list]:
    n = len(STAGES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().logo_profile_end(ms, cnt, n), "logo_profile_end")
    return list(ms), list(cnt)


def alloc_forward_buffers(p: logo_problem, device="cuda") -> dict:
    """Output, selection and workspace tensors for logo_forward."""
    kk = logo_target_count(p.rho, p.n)
    ws = logo_workspace_size(p)
    return {
        "o": torch.empty((p.B, p.Hq, p.n, p.d), dtype=io_dtype(p), device=device),
        "mask": torch.empty((p.B, p.n), dtype=torch.uint8, device=device),
        "idx": torch.empty((p.B, kk), dtype=torch.int32, device=device),
        "rank": torch.empty((p.B, p.n), dtype=torch.int32, device=device),
        "workspace": torch.empty((ws,), dtype=torch.uint8, device=device) if ws else None,
    }
