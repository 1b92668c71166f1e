import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    # the largest achieved error of each test's floating-point checks
    from parity import ERRORS, TOL

    if not ERRORS:
        return
    tr = terminalreporter
    tr.section(f"largest relative error vs the oracle (max |gpu - oracle| / max |oracle|; bound {TOL})")
    for name, v in sorted(ERRORS.items()):
        tr.write_line(f"{v:.3e}  {name}")


@pytest.fixture(autouse=True)
def _release_pinned_host_memory():
    # torch keeps freed pinned host blocks for reuse; tests that pin tens of
    # gigabytes (full-size pools) hand them back so later tests can pin
    yield
    torch = sys.modules.get("torch")
    if torch is not None and torch.cuda.is_initialized():
        import gc

        gc.collect()
        torch.cuda.synchronize()
        if hasattr(torch._C, "_host_emptyCache"):
            torch._C._host_emptyCache()
        torch.cuda.empty_cache()


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle

    oracle.build(force=False)
    yield
