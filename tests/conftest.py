import json
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
    # GPU tests are skipped, not failed, on a machine without a GPU.
    try:
        import torch

        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """The GEMM tolerance slack of every GPU parity check that ran (worst |gpu - ref| / bound per
    check; <= 1 passes), and, if FP8RL_SLACK_REPORT names a file, the same list as JSON."""
    mod = sys.modules.get("tests.gpu_util")
    rows = getattr(mod, "SLACK", None) if mod else None
    if not rows:
        return
    terminalreporter.write_sep("-", "GEMM parity slack: worst |gpu - ref| / bound per check")
    for r in rows:
        terminalreporter.write_line(f"{r['slack']:7.4f}  {r['kind']:<9} {r['out']:<4} "
                                    f"{'x'.join(map(str, r['shape'])):<13} {r['test']} [{r['check']}]")
    path = os.environ.get("FP8RL_SLACK_REPORT")
    if path:
        with open(path, "w") as f:
            json.dump(rows, f, indent=1)
