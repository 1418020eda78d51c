"""Seeded synthetic workloads for token-level dynamic local-global attention.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds shapes and random draws only: no attention, no selection,
no softmax and no combine arithmetic lives here, so neither side of a parity
comparison can borrow the other's logic through it.

Recipe (identical for every consumer):

* ``numpy.random.default_rng(seed)`` (PCG64) draws, in this order, q, k, v
  (standard normal, float32, shapes ``[B,Hq,n,d]``, ``[B,Hkv,n,d]``,
  ``[B,Hkv,n,d]``), then the gate logits ``[B,n]`` (standard normal, float32),
  then, for bursty gates, the run gaps.
* A workload flagged ``qkv_scale`` multiplies q, k, v by ``d**-0.5`` before
  rounding (the 4K multi-head workload draws N(0,1)/sqrt(d) entries).
* Where the workload is bf16, q, k, v are rounded float32 -> bfloat16 by
  round-to-nearest-even on the bit pattern. The oracle receives those exact
  values widened to float32 (exact), the GPU receives the 16-bit patterns.
* Bursty gates: run starts p_1 = G_1, p_{m+1} = p_m + G_{m+1}, with each gap
  G ~ Poisson(1000) drawn again while it is below 64 (so runs never overlap);
  every run covers positions [p, p + 63] within the sequence and adds +4 to
  those gate logits. One independent run sequence per batch row.

The five workloads follow the shapes the LoGo / L2A pages discuss: long
prefill at 32K-128K context with about a fifth of the tokens routed to global
attention ("Learning When to Attend", section "The Architecture of Conditional
Attention"), standing in for the long-context suites those pages evaluate on.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "get_workload",
    "round_to_bf16",
    "bf16_bits",
    "make_inputs",
    "make_far_below",
    "bursty_gate_runs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    n: int
    d: int
    window: int
    rho: float
    dtype: str            # "f32" or "bf16" for q, k, v and the output
    qkv_scale: bool = False   # entries drawn as N(0,1) / sqrt(d)
    bursty: bool = False      # bursty gate logits (runs of 64 with +4)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def describe(self) -> dict:
        return dataclasses.asdict(self)


# The workloads the pages' setting implies (sizes of a long-context prefill
# layer, grouped-query heads as in the Qwen models the L2A page evaluates).
WORKLOADS = {
    "tiny": Workload("tiny", B=1, Hq=1, Hkv=1, n=256, d=64, window=32, rho=0.25,
                     dtype="f32"),
    "mha4k": Workload("mha4k", B=1, Hq=8, Hkv=8, n=4096, d=128, window=512, rho=0.2,
                      dtype="bf16", qkv_scale=True),
    "gqa32k": Workload("gqa32k", B=2, Hq=16, Hkv=4, n=32768, d=128, window=1024,
                       rho=0.2, dtype="bf16"),
    "gqa128k": Workload("gqa128k", B=1, Hq=28, Hkv=4, n=131072, d=128, window=4096,
                        rho=0.2, dtype="bf16"),
    "sweep64k": Workload("sweep64k", B=1, Hq=16, Hkv=16, n=65536, d=64, window=2048,
                         rho=0.2, dtype="bf16", bursty=True),
}

SWEEP_RHOS = (0.0, 0.05, 0.2, 0.5, 1.0)


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN inputs are mapped to a quiet NaN pattern so rounding cannot turn them
    into infinities."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """The float32 value of the nearest-even bfloat16 to each entry."""
    return bits_to_f32(bf16_bits(x))


def bursty_gate_runs(rng: np.random.Generator, n: int, run: int = 64,
                     mean_gap: float = 1000.0) -> np.ndarray:
    """Start positions of the +4 runs for one sequence (seeded Poisson gaps)."""
    starts = []
    p = 0
    while True:
        g = int(rng.poisson(mean_gap))
        while g < run:
            g = int(rng.poisson(mean_gap))
        p += g
        if p >= n:
            break
        starts.append(p)
    return np.asarray(starts, dtype=np.int64)


@dataclasses.dataclass
class Inputs:
    workload: Workload
    seed: int
    q: np.ndarray        # float32 values (bf16-representable when dtype == bf16)
    k: np.ndarray
    v: np.ndarray
    gate: np.ndarray     # float32 [B, n]
    q_bits: Optional[np.ndarray] = None   # uint16 bf16 patterns when dtype == bf16
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.k, self.v, self.gate):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def make_inputs(w: Workload, seed: int = 0, *, gate: Optional[np.ndarray] = None,
                gate_only: bool = False) -> Inputs:
    """Draw q, k, v and the gate for workload ``w`` from ``seed``.

    ``gate`` overrides the drawn gate logits (tests that force ties use it).
    ``gate_only`` skips q, k, v (they are still drawn, to keep the stream
    order, unless the workload is large; then they are left empty)."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, n, d = w.B, w.Hq, w.Hkv, w.n, w.d
    if gate_only:
        # advance past q, k, v without keeping them: same stream as a full draw
        for shape in ((B, Hq, n, d), (B, Hkv, n, d), (B, Hkv, n, d)):
            _skip_normals(rng, int(np.prod(shape)))
        q = k = v = np.zeros((0,), np.float32)
    else:
        q = rng.standard_normal((B, Hq, n, d), dtype=np.float32)
        k = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
        v = rng.standard_normal((B, Hkv, n, d), dtype=np.float32)
        if w.qkv_scale:
            s = np.float32(1.0 / np.sqrt(d))
            q *= s
            k *= s
            v *= s
    g = rng.standard_normal((B, n), dtype=np.float32)
    if w.bursty:
        for b in range(B):
            for p in bursty_gate_runs(rng, n):
                g[b, p:p + 64] += np.float32(4.0)
    if gate is not None:
        g = np.ascontiguousarray(gate, dtype=np.float32).reshape(B, n)
    inp = Inputs(w, seed, q, k, v, g)
    if w.dtype == "bf16" and not gate_only:
        inp.q_bits = bf16_bits(q)
        inp.k_bits = bf16_bits(k)
        inp.v_bits = bf16_bits(v)
        inp.q = bits_to_f32(inp.q_bits)
        inp.k = bits_to_f32(inp.k_bits)
        inp.v = bits_to_f32(inp.v_bits)
    return inp


# A packed batch of 65536 tokens: examples of 32K, 16K, 8K, 4K, 2K, 1K, 512,
# 256 and 256 tokens (a length mix halving per example), otherwise the 32K GQA
# layer's shape.
VARLEN_WORKLOADS = {
    "varlen64k": dict(lens=[32768, 16384, 8192, 4096, 2048, 1024, 512, 256, 256], Hq=16, Hkv=4,
                      d=128, window=1024, rho=0.2, dtype="bf16"),
}


def make_far_below(inp: Inputs, seed: int = 11) -> Inputs:
    """Inputs whose kv group 0 has every score far below zero: the query
    heads of group 0 get entries 8 + 0.5 N(0,1) and kv head 0's keys
    -8 + 0.5 N(0,1) (then bf16-rounded like every bf16 input), so the scaled
    scores sit near -1000 in log2 units at d = 128 and the query norm is
    eight times the standard draw's. Other heads, v and the gate are kept."""
    w = inp.workload
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(seed)
    q = inp.q.copy()
    k = inp.k.copy()
    q[:, :G] = 8.0 + 0.5 * rng.standard_normal(q[:, :G].shape, dtype=np.float32)
    k[:, 0] = -8.0 + 0.5 * rng.standard_normal(k[:, 0].shape, dtype=np.float32)
    out = Inputs(w, inp.seed, q, k, inp.v, inp.gate)
    if w.dtype == "bf16":
        out.q_bits, out.k_bits, out.v_bits = bf16_bits(q), bf16_bits(k), inp.v_bits
        out.q, out.k = bits_to_f32(out.q_bits), bits_to_f32(out.k_bits)
    return out


def make_varlen_inputs(lens, Hq, Hkv, d, dtype="bf16", seed=0):
    """Seeded packed-batch inputs (stream (seed, 0x7A)): q [Hq, T, d], k, v
    [Hkv, T, d] N(0,1), gate [T] N(0,1); cu_seqlens from the lengths."""
    rng = np.random.default_rng([seed, 0x7A])
    T = int(sum(lens))
    q = rng.standard_normal((Hq, T, d), dtype=np.float32)
    k = rng.standard_normal((Hkv, T, d), dtype=np.float32)
    v = rng.standard_normal((Hkv, T, d), dtype=np.float32)
    gate = rng.standard_normal(T, dtype=np.float32)
    bits = {}
    if dtype == "bf16":
        for name, x in (("q", q), ("k", k), ("v", v)):
            bits[name] = bf16_bits(x)
        q, k, v = (bits_to_f32(bits[x]) for x in ("q", "k", "v"))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return {"q": q, "k": k, "v": v, "gate": gate, "cu": cu, "bits": bits}


def make_dout(w: Workload, seed: int = 0):
    """Upstream gradient of the layer output for the backward: N(0,1) entries
    of shape [B, Hq, n, d] from a stream of its own (seed, 0xD0), rounded to
    bf16 when the workload is bf16. Returns (values as float32, bf16 bits or
    None)."""
    rng = np.random.default_rng([seed, 0xD0])
    x = rng.standard_normal((w.B, w.Hq, w.n, w.d), dtype=np.float32)
    if w.dtype == "bf16":
        bits = bf16_bits(x)
        return bits_to_f32(bits), bits
    return x, None


def make_router(w: Workload, seed: int = 0):
    """Synthetic router weights for the routed forward: w [Hq, d] with N(0,1)
    entries from a stream of its own (seed, 0x50), and a bias of 0.25."""
    rng = np.random.default_rng([seed, 0x50])
    return rng.standard_normal((w.Hq, w.d), dtype=np.float32), 0.25


@dataclasses.dataclass
class DecodeInputs:
    q: np.ndarray          # [B, Hq, d] values (bf16-exact for bf16)
    k: np.ndarray          # [B, Hkv, cap, d]
    v: np.ndarray
    lens: np.ndarray       # [B] int32
    gate: np.ndarray       # [B] float32
    tau: np.ndarray        # [B] float32
    bits: dict             # bf16 bit patterns of q, k, v (bf16 only)


DECODE_WORKLOADS = {
    # one decode step of the 128K GQA layer: 8 sequences with full caches;
    # gates N(0,1), threshold at the N(0,1) quantile of 1 - rho, controller frozen
    "decode128k": dict(B=8, Hq=28, Hkv=4, cap=131072, d=128, window=4096, rho=0.25,
                       dtype="bf16"),
}


def make_decode_inputs(B, Hq, Hkv, cap, d, dtype="bf16", seed=0, lens=None, tau=None):
    """Seeded decode-step inputs: N(0,1) q, caches and gates (stream (seed, 0xDEC)),
    lens = cap unless given, tau = 0 unless given."""
    rng = np.random.default_rng([seed, 0xDEC])
    q = rng.standard_normal((B, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, cap, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, cap, d), dtype=np.float32)
    gate = rng.standard_normal(B, dtype=np.float32)
    bits = {}
    if dtype == "bf16":
        for name in ("q", "k", "v"):
            x = {"q": q, "k": k, "v": v}[name]
            bits[name] = bf16_bits(x)
        q, k, v = (bits_to_f32(bits[x]) for x in ("q", "k", "v"))
    lens = np.full(B, cap, np.int32) if lens is None else np.asarray(lens, np.int32)
    tau = np.zeros(B, np.float32) if tau is None else np.asarray(tau, np.float32)
    return DecodeInputs(q, k, v, lens, gate, tau, bits)


def _skip_normals(rng: np.random.Generator, count: int, chunk: int = 1 << 24) -> None:
    while count > 0:
        m = min(count, chunk)
        rng.standard_normal(m, dtype=np.float32)
        count -= m
