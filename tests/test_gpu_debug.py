"""MIL_SSM_DEBUG=1 on the GPU: a call that enqueued work is synchronized and every slot
whose device error word it set is named on stderr (here a commit with an accepted length
outside 0..K), while the call's own status stays MIL_OK; calls captured into a HIP graph
are not synchronized (that would end the capture) and their replays stay exact."""
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


PROG_GRAPH = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import numpy as np, torch
from gpu_util import dev_layer, dev_tokens
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache
w = synth.WORKLOADS["tiny_f32"]
rng = np.random.default_rng(11)
layer = synth.draw_layer(rng, w.H)
A, D = dev_layer(layer)
pre = dev_tokens(synth.draw_tokens(rng, 2, 64, w.H, w.P, w.N, w.G, w.dtype))
eager, graph = (SSMCache(2, w.H, w.P, w.N, w.G, w.K, w.dtype) for _ in range(2))
for c in (eager, graph):
    c.prefill(*pre, A, D, chunk=64)
torch.cuda.synchronize()
x, B, C, dt = (t.clone() for t in dev_tokens(synth.draw_tokens(rng, 2, w.K, w.H, w.P, w.N, w.G, w.dtype)))
j = torch.zeros(2, dtype=torch.int32, device="cuda")
y = torch.empty((2, w.K, w.H, w.P), dtype=torch.float32, device="cuda")
side = torch.cuda.Stream()
side.wait_stream(torch.cuda.current_stream())
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=side):
    graph.verify(x, B, C, dt, A, D, y=y)
    graph.commit(j, x, B, dt)
torch.cuda.synchronize()
for rnd in range(3):
    drf = dev_tokens(synth.draw_tokens(rng, 2, w.K, w.H, w.P, w.N, w.G, w.dtype))
    jj = torch.from_numpy(synth.draw_accept_uniform(rng, 2, w.K)).cuda()
    for dst, src in zip((x, B, C, dt), drf):
        dst.copy_(src)
    j.copy_(jj)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ye = eager.verify(*drf, A, D)
    eager.commit(jj, drf[0], drf[1], drf[3])
    torch.cuda.synchronize()
    assert torch.equal(ye, y), rnd
    assert torch.equal(eager.state(), graph.state()) and torch.equal(eager.pending(), graph.pending()), rnd
print("done")
"""


def test_debug_mode_leaves_graph_capture_intact():
    """MIL_SSM_DEBUG=1 while a verify and a commit are captured into a HIP graph: the calls
    must not synchronize the capturing stream (that would end the capture), and every
    replay must equal the same calls run eagerly, with nothing reported."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    prog = PROG_GRAPH.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    env = dict(os.environ, MIL_SSM_DEBUG="1")
    print("child: tiny cache, verify + commit captured and replayed 3 times under MIL_SSM_DEBUG=1", flush=True)
    r = subprocess.run([sys.executable, "-c", prog], capture_output=True, text=True, env=env, timeout=240)
    print(r.stderr[-2000:])
    assert r.returncode == 0 and r.stdout.strip().endswith("done"), r.stderr[-2000:]
    assert "mil_ssm debug:" not in r.stderr
