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


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()


def pytest_sessionfinish(session, exitstatus):
    """Write the achieved parity errors of this session (tests/gpu_util.py records every
    comparison) to gpurun_out/parity_errors.json."""
    mod = sys.modules.get("gpu_util")
    recs = getattr(mod, "RECORDS", None) if mod else None
    if not recs:
        return
    import json
    out = os.path.join(ROOT, "gpurun_out")
    os.makedirs(out, exist_ok=True)
    worst = {}
    for r in recs:
        w = worst.setdefault(r["test"], {})
        for k in ("normwise", "elementwise"):
            w[f"{r['what']}_{k}"] = max(w.get(f"{r['what']}_{k}", 0.0), r[k])
    with open(os.path.join(out, "parity_errors.json"), "w") as f:
        json.dump({"records": len(recs), "worst_per_test": worst}, f, indent=1, sort_keys=True)
