import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from tests.parity_log import RECORDS as PARITY_RECORDS  # noqa: E402


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    markexpr = getattr(config.option, "markexpr", "") or ""
    if "gpu" in markexpr and "not gpu" not in markexpr:
        # The oracle's process pool must be started before any test
        # initialises the GPU (its workers never hold a GPU context).
        from oracle import pool
        pool.start()


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if not PARITY_RECORDS:
        return
    tr = terminalreporter
    tr.section("max-abs error against the fp64 oracle")
    for r in PARITY_RECORDS:
        extra = "".join(f" {k}={v:.3e}" for k, v in r.items()
                        if k.startswith("delta") and isinstance(v, float))
        tr.write_line(f"{r['name']:<48} {r['dtype']:<5} err {r['err']:.3e}  tol {r['tol']:.0e}"
                      f"  elements {r['elements']}{extra}")
    out_dir = os.path.join(ROOT, "gpurun_out")
    try:
        os.makedirs(out_dir, exist_ok=True)
        with open(os.path.join(out_dir, "parity_errors.json"), "w") as f:
            json.dump(PARITY_RECORDS, f, indent=1)
    except OSError:
        pass
