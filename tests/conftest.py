import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes on the CPU side)")


def pytest_terminal_summary(terminalreporter):
    """Near-tie rates observed by the GPU parity checks (tests/parity.py):
    printed at the end of the run, and appended as JSON lines to the file
    named by NVFP4_PARITY_LOG when that is set."""
    mod = sys.modules.get("parity")
    rates = getattr(mod, "RATES", None) if mod else None
    if not rates:
        return
    agg = {}
    for r in rates:
        key = (r["what"].split("[")[0] or "?", r["kind"])
        a = agg.setdefault(key, [0, 0, 0])
        a[0] += r["diff"]
        a[1] += r["total"]
        a[2] += r["flagged"]
    terminalreporter.write_line("near-tie differences GPU vs oracle (differing / judged, flagged):")
    for (what, kind), (d, n, f) in sorted(agg.items()):
        terminalreporter.write_line(f"  {what:40s} {kind:13s} {d:7d} / {n:10d} = {d / max(1, n):.2e}"
                                    f"  (flagged {f})")
    path = os.environ.get("NVFP4_PARITY_LOG")
    if path:
        import json
        with open(path, "a") as f:
            for r in rates:
                f.write(json.dumps(r) + "\n")
