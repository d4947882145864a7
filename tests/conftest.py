import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large oracle cases")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; report them as skipped rather than
    # failing when someone runs the whole suite on a CPU-only host.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    """After a GPU run, write every parity comparison's error and bound
    (worst ratio first) to the file the environment variable
    SDPA_PARITY_MARGINS names, when it is set: the margin under the bound,
    not only pass or fail."""
    gu = sys.modules.get("gpu_util")
    path = os.environ.get("SDPA_PARITY_MARGINS")
    if gu is None or not getattr(gu, "MARGINS", None) or not path:
        return
    rows = sorted(gu.MARGINS, key=lambda r: -r[3] / r[4])
    with open(path, "w") as fh:
        fh.write("# err/bound  err  bound  dtype  what  test\n")
        for test, what, dtype, e, tol in rows:
            fh.write(f"{e / tol:.3f} {e:.3e} {tol:.0e} {dtype} {what} {test}\n")
