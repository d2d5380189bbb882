"""MIL_SSM_DEBUG=1 on the GPU: a call that enqueued work is synchronized and every slot
whose device error word it set is named on stderr (here a commit with an accepted length
outside 0..K), while the call's own status stays MIL_OK."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROG = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import numpy as np, torch
from gpu_util import dev_layer, dev_tokens
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache
w = synth.WORKLOADS["tiny_f32"]
rng = np.random.default_rng(7)
layer = synth.draw_layer(rng, w.H)
A, D = dev_layer(layer)
cache = SSMCache(2, w.H, w.P, w.N, w.G, w.K, w.dtype)
cache.prefill(*dev_tokens(synth.draw_tokens(rng, 2, 64, w.H, w.P, w.N, w.G, w.dtype)), A, D, chunk=64)
drf = dev_tokens(synth.draw_tokens(rng, 2, w.K, w.H, w.P, w.N, w.G, w.dtype))
cache.verify(*drf, A, D)
cache.commit(torch.tensor([2, w.K + 1], dtype=torch.int32, device="cuda"), drf[0], drf[1], drf[3])
torch.cuda.synchronize()
print("done")
"""


def test_debug_mode_names_device_errors():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    prog = PROG.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    env = dict(os.environ, MIL_SSM_DEBUG="1")
    print("child: tiny cache, commit with j = K + 1 under MIL_SSM_DEBUG=1", flush=True)
    r = subprocess.run([sys.executable, "-c", prog], capture_output=True, text=True, env=env, timeout=240)
    print(r.stderr[-2000:])
    assert r.returncode == 0 and r.stdout.strip().endswith("done"), r.stderr[-2000:]
    assert "mil_ssm debug: mil_ssm_commit: cache 0 slot 1 error word 0x1 (accept 1" in r.stderr
    assert "slot 0" not in r.stderr
