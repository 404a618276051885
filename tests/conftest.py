import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU statistics test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Parity figures of every GPU comparison of the run (tests/gpu_harness.py RECORDS): per
    test, the in-band and mismatch fractions of codes and signs, the largest score error
    against the row's largest logit and the largest output error against the row's largest
    output magnitude."""
    mod = sys.modules.get("tests.gpu_harness") or sys.modules.get("gpu_harness")
    records = getattr(mod, "RECORDS", None)
    if not records:
        return
    tr = terminalreporter
    tr.section("parity figures (worst per test)")
    for test, figs in records.items():
        tr.write_line(test.split("::", 1)[-1])
        tr.write_line("    " + "  ".join(f"{k}={v:.3g}" for k, v in sorted(figs.items())))
