"""A process pool that runs the CPU oracle for the full-size GPU tests.

The oracle computes rows one by one in float64; at full size the tests need
tens of thousands of rows, so they are spread over worker processes. The
workers are forked before the test process touches the GPU (``start()`` is
called from ``conftest.py`` when GPU tests are selected), hold no GPU state
and run NumPy with one BLAS thread each. Inputs reach them as float32 .npy
files that every worker memory-maps read-only: the arrays are written once by
the test process and shared through the page cache. Holds no attention
arithmetic: every number comes from a function of ``oracle``.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

_POOL = None
_WORKERS = 0
_INPUTS: Dict[str, Dict[str, np.ndarray]] = {}   # per worker: directory -> arrays


def workers() -> int:
    """Worker count: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - not Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init_worker() -> None:
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # threadpoolctl missing: the environment variables stand
        pass


def start() -> None:
    """Fork the workers now (call before any GPU work in this process)."""
    global _POOL, _WORKERS
    if _POOL is None:
        _WORKERS = workers()
        _POOL = mp.get_context("fork").Pool(_WORKERS, initializer=_init_worker)


def pool():
    if _POOL is None:
        start()
    return _POOL


def stop() -> None:
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None


class SharedInputs:
    """float32 arrays written to a temporary directory for the workers; a
    context manager that removes the directory afterwards."""

    def __init__(self, **arrays: np.ndarray):
        self.dir = tempfile.mkdtemp(prefix="oracle_inputs_")
        self.add(**arrays)

    def add(self, **arrays: np.ndarray) -> None:
        """More arrays, for tasks submitted after this call."""
        for name, a in arrays.items():
            np.save(os.path.join(self.dir, name + ".npy"), np.ascontiguousarray(a))

    def __enter__(self) -> "SharedInputs":
        return self

    def __exit__(self, *exc) -> None:
        shutil.rmtree(self.dir, ignore_errors=True)


def _array(d: str, name: str) -> np.ndarray:
    if d not in _INPUTS:
        _INPUTS.clear()
        _INPUTS[d] = {}
    arrays = _INPUTS[d]
    if name not in arrays:
        arrays[name] = np.load(os.path.join(d, name + ".npy"), mmap_mode="r")
    return arrays[name]


def _run(task):
    d, fn_name, args, kwargs = task
    import oracle
    import oracle.backward
    import oracle.router
    import routed_bound
    mods = {"oracle": oracle, "backward": oracle.backward, "router": oracle.router,
            "routed_bound": routed_bound}
    mod, fn = fn_name.split(".")
    args = [_array(d, a[1:]) if isinstance(a, str) and a.startswith("@") else a for a in args]
    return getattr(mods[mod], fn)(*args, **kwargs)


def map_chunks(shared: SharedInputs, fn_name: str, make_args: Callable[[Sequence], tuple],
               items: Sequence, chunk: int, kwargs: Optional[dict] = None) -> List:
    """Calls ``fn_name`` ("oracle.forward_rows", "router.router_logits_at",
    "backward.dkdv_keys", "routed_bound.logit_error_scales", ...) once per
    chunk of ``items``, in the workers;
    ``make_args(chunk_items)`` gives the positional arguments, where a string
    "@name" stands for the shared array ``name``. Returns the results in
    chunk order."""
    tasks = [(shared.dir, fn_name, make_args(items[i:i + chunk]), kwargs or {})
             for i in range(0, len(items), chunk)]
    return pool().map(_run, tasks, chunksize=1)
