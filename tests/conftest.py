import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_sessionfinish(session, exitstatus):
    """Write every bf16 comparison's flat-bar figures (tests/gpu_harness.py
    BAR_LOG) to the JSON file named by CPATTN_BAR_REPORT, if set, and print
    the comparisons that have elements over max-abs 2e-2."""
    mod = sys.modules.get("tests.gpu_harness")
    if mod is None or not getattr(mod, "BAR_LOG", None):
        return
    import json
    path = os.environ.get("CPATTN_BAR_REPORT")
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump(mod.BAR_LOG, f, indent=1)
    over = [e for e in mod.BAR_LOG if e.get("n_over_2e-2")]
    n_el = sum(e["n"] for e in mod.BAR_LOG)
    print(f"\n[flat bar] {len(mod.BAR_LOG)} bf16 comparisons, {n_el} elements; "
          f"{len(over)} with elements over max-abs 2e-2 "
          f"({sum(e['n_over_2e-2'] for e in over)} elements, "
          f"{sum(e['n_over_2e-2_ref_lt_2'] for e in over)} of them with |ref| < 2)")
    for e in over:
        print(f"  {e['test']} {e['tensor']}: {e['n_over_2e-2']} over, max {e['max_abs']:.4f}, "
              f"|ref|<2: {e['n_over_2e-2_ref_lt_2']} / {e['max_abs_ref_lt_2']:.4f}"
              + (f"; ideal {e['ideal']}" if "ideal" in e else ""))
