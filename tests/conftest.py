import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_terminal_summary(terminalreporter):
    """How much of the parity bar's slack the session used (oracle/check.py LEDGER)."""
    try:
        from oracle import check
    except Exception:  # the oracle is not importable: nothing was compared
        return
    s = check.slack_summary()
    if not s["reports"]:
        return
    terminalreporter.write_line(
        f"parity slack: {s['reports']} comparisons over {s['outputs']} outputs; {s['over_2ulp']} over 2 ULP, "
        f"{s['interval_pass']} admitted by the interval ({s['widened_pass']} of them only inside its +-2 ULP "
        f"widening); {s['small_sample_slack_reports']} comparisons met the bit-exact bar only through the "
        f"small-sample slack; {s['pooled_only_calls']} grouped calls only as a pooled rate; "
        f"{s['failures']} failures")
    path = os.environ.get("GLU_PARITY_LEDGER")
    if path:
        import json
        with open(path, "w") as f:
            json.dump(s, f, indent=1)
