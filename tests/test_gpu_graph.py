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


@pytest.mark.parametrize("kmax,multi", [(4, False), (8, False), (8, True)],
                         ids=["kmax4", "kmax8", "kmax8_commit_layers"])
def test_graph_decode_step_at_hybrid_layer_shape_matches_oracle(kmax, multi):
    """The decode step of the hybrid workload's layer shape (32 sequences, 32 heads,
    P = 128, N = 256, 8 groups, K = 4, accepted lengths ~ Geometric(0.3) capped at 4) for
    three layers, captured once and replayed for five rounds, with caches holding K or 8
    pending rows (8: verifies write the state back only when a commit could overflow them).
    Each round, two sampled heads of every layer are checked against the oracle: the drafts'
    y against oracle verify from the oracle's committed state, and the stored state against
    the oracle's state through the previous round's accepted drafts where this round's
    verify wrote it back (else against the state before the verify, untouched); pending
    counts follow the rule; replay == eager stays bit for bit on the whole layer.  With
    `multi`, every layer accepts the same lengths each round (the verifier decides after
    the last layer) and the captured step commits all layers with one
    mil_ssm_commit_layers launch, whose per-layer pointers travel in the captured kernel
    arguments."""
    import oracle
    from gpu_util import BOUND, head_slice, state_err, y_err
    from speculative_decode_amd.ssm import commit_layers

    rng = np.random.default_rng(5005)
    layers, Bt, H, P, N, G, K, L0 = 3, 32, 32, 128, 256, 8, 4, 256
    dtype = synth.BF16
    lay = [synth.draw_layer(rng, H) for _ in range(layers)]
    params = [dev_layer(l) for l in lay]
    pres = [synth.draw_tokens(rng, Bt, L0, H, P, N, G, dtype) for _ in range(layers)]
    sets = []
    for _ in range(2):  # [0] eager, [1] graph
        cs = []
        for li in range(layers):
            c = SSMCache(Bt, H, P, N, G, kmax, dtype)
            c.prefill(*dev_tokens(pres[li]), *params[li], want_y=False)
            cs.append(c)
        sets.append(cs)
    heads = [[int(h) for h in rng.choice(H, size=2, replace=False)] for _ in range(layers)]
    ref = {}  # (layer, head) -> oracle committed state [Bt][1][N][P]
    for li in range(layers):
        for h in heads[li]:
            x, B, C, dt, A, D = head_slice(pres[li], lay[li], h, H, G)
            _, ref[li, h] = oracle.prefill(x, B, C, dt, A, D)
    torch.cuda.synchronize()

    stat = [dict(x=torch.empty((Bt, K, H, P), dtype=torch.bfloat16, device="cuda"),
                 B=torch.empty((Bt, K, G, N), dtype=torch.bfloat16, device="cuda"),
                 C=torch.empty((Bt, K, G, N), dtype=torch.bfloat16, device="cuda"),
                 dt=torch.empty((Bt, K, H), dtype=torch.bfloat16, device="cuda"),
                 j=torch.zeros(Bt, dtype=torch.int32, device="cuda"),
                 y=torch.empty((Bt, K, H, P), dtype=torch.float32, device="cuda")) for _ in range(layers)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for li in range(layers):
            s = stat[li]
            sets[1][li].verify(s["x"], s["B"], s["C"], s["dt"], *params[li], y=s["y"])
            if not multi:
                sets[1][li].commit(s["j"], s["x"], s["B"], s["dt"])
        if multi:  # one accepted-length buffer (layer 0's) for every layer
            commit_layers(sets[1], stat[0]["j"], [s["x"] for s in stat], [s["B"] for s in stat],
                          [s["dt"] for s in stat])
    torch.cuda.synchronize()

    pos = [np.full(Bt, L0) for _ in range(layers)]
    pend = [np.zeros(Bt, np.int64) for _ in range(layers)]  # host mirror of the pending counts
    deferred = 0
    for rnd in range(5):
        rounds = []
        j_shared = synth.draw_accept_geometric(rng, Bt, K) if multi else None
        for li in range(layers):
            drf = synth.draw_tokens(rng, Bt, K, H, P, N, G, dtype)
            j = j_shared if multi else synth.draw_accept_geometric(rng, Bt, K)
            x, B, C, dt = dev_tokens(drf)
            for key, t in (("x", x), ("B", B), ("C", C), ("dt", dt)):
                stat[li][key].copy_(t)
            stat[li]["j"].copy_(torch.from_numpy(j).cuda())
            rounds.append((drf, j))
        torch.cuda.synchronize()
        before = [sets[1][li].state().cpu().numpy() for li in range(layers)]
        g.replay()
        torch.cuda.synchronize()
        for li in range(layers):
            drf, j = rounds[li]
            yg = stat[li]["y"].cpu().numpy()
            st = sets[1][li].state().cpu().numpy()
            m = pend[li]
            wb = (m > 0) & (m + K > kmax)  # slots whose verify wrote the folded state back
            deferred += int(((m > 0) & ~wb).sum())
            for h in heads[li]:
                x, B, C, dt, A, D = head_slice(drf, lay[li], h, H, G)
                ry = oracle.verify(ref[li, h], x, B, C, dt, A, D)
                assert y_err(yg[:, :, h:h + 1], ry) <= BOUND[dtype], (rnd, li, h)
                # the stored state: where this round's verify wrote back, the oracle's state
                # through the previous rounds' accepted rows; elsewhere what it was before
                if wb.any():
                    assert state_err(st[wb][:, h:h + 1].astype(np.float64), ref[li, h][wb]) <= BOUND[dtype], \
                        (rnd, li, h)
                keep = ~wb & (m > 0)
                assert np.array_equal(st[keep][:, h], before[li][keep][:, h]), (rnd, li, h)
                ref[li, h] = oracle.commit(ref[li, h], x, B, dt, A, D, j)
            pend[li] = np.where(wb | (m == 0), 0, m) + j
            assert sets[1][li].pending().cpu().tolist() == pend[li].tolist()
            pos[li] = pos[li] + j
            assert sets[1][li].pos().cpu().numpy().tolist() == pos[li].tolist()
        # the same round eagerly on the twin caches: bit for bit
        eager = []
        for li in range(layers):
            drf, j = rounds[li]
            c = sets[0][li]
            xe, Be, Ce, dte = dev_tokens(drf)
            ye = c.verify(xe, Be, Ce, dte, *params[li])
            if not multi:
                c.commit(torch.from_numpy(j).cuda(), xe, Be, dte)
            eager.append((ye, xe, Be, dte))
        if multi:
            commit_layers(sets[0], torch.from_numpy(rounds[0][1]).cuda(), [e[1] for e in eager],
                          [e[2] for e in eager], [e[3] for e in eager])
        torch.cuda.synchronize()
        for li in range(layers):
            c = sets[0][li]
            assert torch.equal(eager[li][0], stat[li]["y"]), (rnd, li)
            assert torch.equal(c.state(), sets[1][li].state()), (rnd, li)
            assert torch.equal(c.pending(), sets[1][li].pending()) and torch.equal(c.pos(), sets[1][li].pos())
    if kmax > K:
        assert deferred > 0
