import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; mark them skipped rather than failing when
    # the CPU suite is run without "-m 'not gpu'".
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    path = os.environ.get("GVA_PARITY_LOG")
    mod = sys.modules.get("tests.gpu_cases")
    if not path or mod is None or not mod.ERRORS:
        return
    with open(path, "w") as f:
        f.write("check\tdtype\tmax_abs\trel_l2\n")
        for what, dtype, err, r in mod.ERRORS:
            f.write(f"{what}\t{dtype}\t{err:.3e}\t{r:.3e}\n")
