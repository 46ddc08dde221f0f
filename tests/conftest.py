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

# Where the parity report of a session goes (Markdown, plus JSON beside it).
REPORT_PATH = os.environ.get("FA_PARITY_REPORT",
                             os.path.join(ROOT, "gpurun_out", "parity_report.md"))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _fmt(x):
    return f"{x:.3e}" if isinstance(x, float) else str(x)


def _row(r):
    return "| " + " | ".join([
        r["test"].split("::", 1)[-1], r["output"], str(r["n"]), _fmt(r["max_abs"]), r["tol"],
        _fmt(r["floor"]) if "floor" in r else "-",
        str(r["beyond_plain"]) if "beyond_plain" in r else "-",
        f"{r['max_ratio']:.3f}", "yes" if r["passed"] else "**NO**"]) + " |"


def write_parity_report(records, path):
    """One table row per check: the test, the output, its element count, the
    plain max-abs error, the tolerance rule, the bf16 rounding floor, the
    elements beyond a plain 1e-2, the largest error / allowed ratio, and the
    verdict. The checks of the named benchmark workloads come first."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(os.path.splitext(path)[0] + ".json", "w") as f:
        json.dump(records, f, indent=1)
    head = ["| test | output | n | max-abs | tolerance | bf16 floor | beyond 1e-2 | "
            "max err/allowed | pass |",
            "|---|---|---|---|---|---|---|---|---|"]
    named = [r for r in records if "workload" in r["test"]]
    failed = sum(1 for r in records if not r["passed"])
    lines = ["# Parity report (GPU results against the fp64 oracle)", "",
             f"{len(records)} checks, {failed} failed.", "",
             "## The named workloads", ""] + head + [_row(r) for r in named] + [
             "", "## Every check", ""] + head
    for r in records:
        lines.append(_row(r))
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def pytest_sessionfinish(session, exitstatus):
    mod = sys.modules.get("parity_util")
    records = getattr(mod, "RECORDS", None) if mod is not None else None
    if records:
        write_parity_report(records, REPORT_PATH)
