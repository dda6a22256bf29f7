import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


def _parity_report():
    lib = sys.modules.get("rkv_testlib")
    return getattr(lib, "REPORT", None) or None


def pytest_terminal_summary(terminalreporter):
    rep = _parity_report()
    if not rep:
        return
    tot = {}
    for counts in rep.values():
        for k, v in counts.items():
            tot[k] = tot.get(k, 0) + v
    terminalreporter.write_line(
        "parity counts over %d tests: %s" % (len(rep), json.dumps(tot, sort_keys=True)))


def pytest_sessionfinish(session):
    """Write the accepted near-ties and rounding-boundary cases of every
    encode comparison to a JSON record ($RKV_PARITY_REPORT, by default
    reports/parity_counts.json under the repository root)."""
    rep = _parity_report()
    if not rep:
        return
    path = os.environ.get("RKV_PARITY_REPORT",
                          os.path.join(ROOT, "reports", "parity_counts.json"))
    try:
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            json.dump({"tests": rep}, f, indent=1, sort_keys=True)
    except OSError:
        pass
