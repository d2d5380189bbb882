"""The bench's JSON line on the GPU (a shortened run without the CPU leg): the fields the
line promises, the roofline object of the verify kernel and the prefill leg beside it, and
values that agree with one another (value from the step time, frac from achieved / peak)."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "8", "--warmup", "8", "--no-cpu-baseline"]
    print("child:", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 8 and d["warmup"] == 8
    assert d["higher_is_better"] is True and d["unit"] == "verified tokens/s"
    c = d["config"]
    assert c["workload"] == "hybrid_decode" and c["layers"] == 24 and c["batch"] == 32 and c["drafts_K"] == 4
    # value: verified tokens (batch x K) per step over the step's time
    assert d["value"] > 0 and abs(d["value"] * d["ms_per_step"] * 1e-3 - c["batch"] * c["drafts_K"]) < 1e-6 * d["value"]
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] <= 1 and abs(roof["achieved"] / roof["peak"] - roof["frac"]) < 1e-9
    assert roof["traffic"] is None or roof["traffic"] > 0
    p = d["prefill"]
    assert p["config"]["workload"] == "llama8b_long_prefill" and p["unit"] == "prefill tokens/s" and p["value"] > 0
    assert 0 < p["roofline"]["frac"] <= 1
    print(f"value {d['value']:.0f} verified tokens/s, verify frac {roof['frac']:.3f}, "
          f"prefill {p['value']:.3g} tokens/s (frac {p['roofline']['frac']:.3f})")
