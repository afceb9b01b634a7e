import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: long CPU test (oracle at large sizes)")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """Print the GPU/oracle parity record of the session (every compare()
    call: rows compared, decisions taken, sequences within 1e-6 of a decision
    boundary, excused mismatches, largest probability errors), one line per
    test, and write the per-comparison table to gpurun_out/parity_summary.txt."""
    parity = sys.modules.get("tests.parity")
    reports = getattr(parity, "REPORTS", None)
    if not reports:
        return
    per_test = {}
    for r in reports:
        t = per_test.setdefault(r["test"], dict(calls=0, rows=0, decisions=0, near=0, mism=0,
                                                err=0.0))
        t["calls"] += 1
        t["rows"] += r["rows"]
        t["decisions"] += r["decisions"]
        t["near"] += r["near_boundary"]
        t["mism"] += r["mismatches"]
        t["err"] = max([t["err"]] + [r[k] for k in ("p_err", "q_err", "z_err") if k in r])
    tot = {k: sum(t[k] for t in per_test.values()) for k in ("calls", "rows", "decisions",
                                                              "near", "mism")}
    tr = terminalreporter
    tr.write_sep("=", "GPU/oracle parity")
    tr.write_line("test: compares, rows, decisions, within 1e-6 of a boundary, excused "
                  "mismatches, max |p|q|Z err|")
    for name, t in per_test.items():
        short = name.replace("tests/", "").replace(".py::", "::")
        tr.write_line(f"{short}: {t['calls']} {t['rows']} {t['decisions']} {t['near']} "
                      f"{t['mism']} {t['err']:.1e}")
    tr.write_line(f"total: {tot['calls']} compares, {tot['rows']} rows, {tot['decisions']} "
                  f"decisions, {tot['near']} within 1e-6 of a boundary, {tot['mism']} excused "
                  f"mismatches (rate {tot['mism'] / max(1, tot['decisions']):.2e})")
    out_dir = os.path.join(ROOT, "gpurun_out")
    try:
        os.makedirs(out_dir, exist_ok=True)
        with open(os.path.join(out_dir, "parity_summary.txt"), "w") as f:
            f.write("test | label | rows | decisions | near boundary | mismatches | "
                    "p_err | q_err | z_err\n")
            for r in reports:
                f.write(" | ".join(str(r.get(k, "")) for k in (
                    "test", "label", "rows", "decisions", "near_boundary", "mismatches",
                    "p_err", "q_err", "z_err")) + "\n")
    except OSError:
        pass
