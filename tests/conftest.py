import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    return torch.cuda.is_available()


def pytest_terminal_summary(terminalreporter):
    """Worst |got - ref| / bound of the output checks per test (GPU runs)."""
    import json
    mod = sys.modules.get("tests.gpu_support")
    ratios = getattr(mod, "WORST_RATIO", None) if mod else None
    if not ratios:
        return
    terminalreporter.write_sep("-", "worst output error / bound per test")
    for name, r in sorted(ratios.items(), key=lambda kv: -kv[1]):
        terminalreporter.write_line(f"{r:8.4f}  {name}")
    path = os.environ.get("KVS_RATIO_FILE")
    if path:
        with open(path, "w") as f:
            json.dump(ratios, f, indent=1, sort_keys=True)
    amb = getattr(mod, "AMB_LOG", None)
    if amb:
        terminalreporter.write_sep("-", "selection near-ties |Amb| per test (checked steps)")
        for name, rows in sorted(amb.items()):
            sizes = [r[-3] for r in rows]
            bands = [r[-2] for r in rows if r[-2] >= 0]
            differ = sum(1 for r in rows if not r[-1])
            line = (f"{name}: {len(rows)} checks, |Amb| max {max(sizes)}, mean {sum(sizes) / len(sizes):.2f}, "
                    f"sets differing inside Amb {differ}")
            if bands:
                line += f", observed-error band max {max(bands)}, mean {sum(bands) / len(bands):.2f}"
            terminalreporter.write_line(line)


def pytest_sessionfinish(session, exitstatus):
    """|Amb| (near-ties of the selection protocol) per checked step, written
    to KVS_AMB_FILE when set."""
    import json
    mod = sys.modules.get("tests.gpu_support")
    log = getattr(mod, "AMB_LOG", None) if mod else None
    path = os.environ.get("KVS_AMB_FILE")
    if log and path:
        with open(path, "w") as f:
            json.dump(log, f)
