import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def _gpu_selected(config) -> bool:
    expr = (config.getoption("markexpr") or "").replace(" ", "")
    return "gpu" in expr and "notgpu" not in expr


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    if _gpu_selected(config):
        # the oracle's worker processes are forked now, before any test
        # touches the GPU (full-size parity tests spread oracle rows over them)
        import oracle_pool
        oracle_pool.start()


def pytest_unconfigure(config):
    mod = sys.modules.get("oracle_pool")
    if mod is not None:
        mod.stop()
