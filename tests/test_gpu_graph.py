"""A multi-layer decode step (every layer: verify K drafts, then commit) captured once in
a HIP graph and replayed round after round, against the same rounds run eagerly on a
twin set of caches.  Between replays the program does its own eager work (new drafts and
accepted lengths copied into the graph's input buffers) and synchronises; every replay's
outputs, states and counters must equal the eager ones bit for bit (same kernels, same
inputs)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import dev, dev_layer, dev_tokens
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from speculative_decode_amd import _lib
    _lib.lib()


@pytest.mark.parametrize("greedy", [False, True], ids=["commit", "greedy_commit"])
def test_graph_replays_match_eager(greedy):
    rng = np.random.default_rng(4242 + greedy)
    layers, Bt, H, P, N, G, K, vocab = 3, 3, 4, 64, 64, 2, 4, 5000
    dtype = synth.BF16
    params = [dev_layer(synth.draw_layer(rng, H)) for _ in range(layers)]
    pre = synth.draw_tokens(rng, Bt, 40, H, P, N, G, dtype)
    sets = []
    for _ in range(2):  # [0] eager, [1] graph
        cs = []
        for li in range(layers):
            c = SSMCache(Bt, H, P, N, G, K, dtype)
            c.prefill(*dev_tokens(pre), *params[li])
            cs.append(c)
        sets.append(cs)
    torch.cuda.synchronize()

    # the graph's input and output buffers (filled before every replay)
    stat = [dict(x=torch.empty((Bt, K, H, P), dtype=torch.bfloat16, device="cuda"),
                 B=torch.empty((Bt, K, G, N), dtype=torch.bfloat16, device="cuda"),
                 C=torch.empty((Bt, K, G, N), dtype=torch.bfloat16, device="cuda"),
                 dt=torch.empty((Bt, K, H), dtype=torch.bfloat16, device="cuda"),
                 j=torch.zeros(Bt, dtype=torch.int32, device="cuda"),
                 tok=torch.zeros((Bt, K), dtype=torch.int32, device="cuda"),
                 lg=torch.zeros((Bt, K, vocab), dtype=torch.bfloat16, device="cuda"),
                 acc=torch.zeros(Bt, dtype=torch.int32, device="cuda"),
                 ws=torch.empty(sets[1][0].greedy_workspace_bytes(K, vocab) + 256, dtype=torch.uint8, device="cuda"),
                 y=torch.empty((Bt, K, H, P), dtype=torch.float32, device="cuda")) for _ in range(layers)]

    def layer_step(c, li, s, A, D):
        c.verify(s["x"], s["B"], s["C"], s["dt"], A, D, y=s["y"])
        if greedy:
            c.commit_greedy(s["tok"], s["lg"], s["x"], s["B"], s["dt"], accepted=s["acc"], ws=s["ws"])
        else:
            c.commit(s["j"], s["x"], s["B"], s["dt"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for li in range(layers):
            layer_step(sets[1][li], li, stat[li], *params[li])
    torch.cuda.synchronize()

    for rnd in range(4):
        # new drafts and decisions for this round (eager work between replays)
        rounds = []
        for li in range(layers):
            drf = synth.draw_tokens(rng, Bt, K, H, P, N, G, dtype)
            j = synth.draw_accept_uniform(rng, Bt, K)
            tok, lg = synth.draw_greedy(rng, Bt, K, vocab, synth.BF16, j)
            x, B, C, dt = dev_tokens(drf)
            stat[li]["x"].copy_(x), stat[li]["B"].copy_(B), stat[li]["C"].copy_(C), stat[li]["dt"].copy_(dt)
            stat[li]["j"].copy_(torch.from_numpy(j).cuda())
            stat[li]["tok"].copy_(torch.from_numpy(tok).cuda())
            stat[li]["lg"].copy_(dev(lg))
            rounds.append((x, B, C, dt, torch.from_numpy(j).cuda(), torch.from_numpy(tok).cuda(), dev(lg)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # the same round eagerly on the twin caches
        for li in range(layers):
            x, B, C, dt, jj, tok, lg = rounds[li]
            c = sets[0][li]
            ye = c.verify(x, B, C, dt, *params[li])
            if greedy:
                acc, _ = c.commit_greedy(tok, lg, x, B, dt)
                torch.cuda.synchronize()
                assert torch.equal(acc, stat[li]["acc"]), (rnd, li)
            else:
                c.commit(jj, x, B, dt)
            torch.cuda.synchronize()
            assert torch.equal(ye, stat[li]["y"]), (rnd, li)
            assert torch.equal(c.state(), sets[1][li].state()), (rnd, li)
            assert torch.equal(c.pos(), sets[1][li].pos()) and torch.equal(c.pending(), sets[1][li].pending())
