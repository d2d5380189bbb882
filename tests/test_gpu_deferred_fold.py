"""The deferred state write-back: a cache whose pending area holds more rows than one
round's drafts (k_max > K) lets accepted rows accumulate, and a verify writes the folded
state back only when the next commit could overflow the pending area.

Two caches take the same inputs: one with k_max = K (every verify with pending rows writes
back) and one with k_max = 4K.  Every round's outputs must agree bit for bit and match the
oracle; the deferring cache's append and pending counts must follow the rule, and its
stored state must be untouched by a verify that defers; after a final commit with
MIL_COMMIT_MATERIALIZE both states agree bit for bit and match the oracle.  Chain, tree and
greedy commits, and a rejected accepted length, all take part.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import BOUND, dev, dev_layer, dev_tokens, state_err, y_err
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from speculative_decode_amd import _lib
    _lib.lib()


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dtype,K,kmax", [(synth.BF16, 4, 16), (synth.F32, 4, 16), (synth.BF16, 1, 3),
                                          (synth.BF16, 7, 9)])
def test_deferred_write_back_matches_eager(dtype, K, kmax):
    batch, H, P, N, G = 6, 4, 64, 64, 2
    rng = np.random.default_rng(6200 + 10 * K + kmax + (dtype == synth.F32))
    layer = synth.draw_layer(rng, H)
    A, D = dev_layer(layer)
    Af, Df = layer.A.f64, layer.D.f64
    pre = synth.draw_tokens(rng, batch, 48, H, P, N, G, dtype)
    eager = SSMCache(batch, H, P, N, G, K, dtype)
    lazy = SSMCache(batch, H, P, N, G, kmax, dtype)
    for c in (eager, lazy):
        c.prefill(*dev_tokens(pre), A, D, chunk=64, want_y=False)
    h = oracle.prefill(pre.x.f64, pre.B.f64, pre.C.f64, pre.dt.f64, Af, Df)[1]
    kinds = ["chain"] * 5 + ["tree", "chain", "greedy", "chain", "reject", "chain", "tree", "chain", "greedy"]
    deferred_rounds = 0
    for r, kind in enumerate(kinds):
        print(f"round {r}: {kind}", flush=True)
        drf = synth.draw_tokens(rng, batch, K, H, P, N, G, dtype)
        dx, dB, dC, ddt = dev_tokens(drf)
        m = lazy.pending().cpu().numpy().copy()
        raw = lazy.state().clone()
        par = synth.draw_tree(rng, batch, K, "random") if kind == "tree" else None
        if par is not None:
            ys = [c.verify_tree(i32(par), dx, dB, dC, ddt, A, D) for c in (eager, lazy)]
            ry = oracle.verify_tree(h, drf.x.f64, drf.B.f64, drf.C.f64, drf.dt.f64, Af, Df, par)
        else:
            ys = [c.verify(dx, dB, dC, ddt, A, D) for c in (eager, lazy)]
            ry = oracle.verify(h, drf.x.f64, drf.B.f64, drf.C.f64, drf.dt.f64, Af, Df)
        torch.cuda.synchronize()
        assert torch.equal(ys[0], ys[1]), r
        assert y_err(ys[1].cpu().numpy(), ry) <= BOUND[dtype]
        # the rule: write back only when pending + K could overflow the pending area
        wb = (m > 0) & (m + K > kmax)
        assert np.array_equal(lazy.append().cpu().numpy(), np.where(wb | (m == 0), 0, m)), r
        # a slot whose rows stayed pending keeps its stored state bit for bit
        keep = torch.from_numpy(~wb).cuda()
        assert torch.equal(lazy.state()[keep], raw[keep]), r
        deferred_rounds += int(((m > 0) & ~wb).sum())
        if kind == "tree":
            node = rng.integers(-1, K, size=batch)
            for c in (eager, lazy):
                c.commit_tree(i32(par), i32(node), dx, dB, ddt)
            h, _ = oracle.commit_tree(h, drf.x.f64, drf.B.f64, drf.dt.f64, Af, Df, par, node)
        elif kind == "greedy":
            planted = synth.draw_accept_uniform(rng, batch, K)
            tok, lg = synth.draw_greedy(rng, batch, K, 300, synth.F32, planted)
            j_ref, _ = oracle.greedy_accept(tok, lg.f64)
            accs = [c.commit_greedy(i32(tok), dev(lg), dx, dB, ddt)[0] for c in (eager, lazy)]
            assert np.array_equal(accs[1].cpu().numpy(), j_ref)
            h = oracle.commit(h, drf.x.f64, drf.B.f64, drf.dt.f64, Af, Df, j_ref)
        else:
            j = synth.draw_accept_uniform(rng, batch, K)
            if kind == "reject":
                j[1] = K + 1  # rejected: slot 1 keeps its logical state and pending rows
            for c in (eager, lazy):
                c.commit(i32(j), dx, dB, ddt)
            jr = j.copy()
            jr[(jr < 0) | (jr > K)] = 0
            h = oracle.commit(h, drf.x.f64, drf.B.f64, drf.dt.f64, Af, Df, jr)
            if kind == "reject":
                for c in (eager, lazy):
                    assert c.status(clear=True) == 1
        torch.cuda.synchronize()
        assert torch.equal(eager.pos(), lazy.pos()), r
        assert int(lazy.pending().max()) <= kmax
    assert deferred_rounds > 0  # the deferring cache did defer (slot-rounds left pending)
    # materialize both: one more verify, then a commit of nothing with the fold forced
    drf = synth.draw_tokens(rng, batch, K, H, P, N, G, dtype)
    dx, dB, dC, ddt = dev_tokens(drf)
    for c in (eager, lazy):
        c.verify(dx, dB, dC, ddt, A, D)
        c.commit(i32(np.zeros(batch)), dx, dB, ddt, A, D, materialize=True)
    torch.cuda.synchronize()
    assert torch.equal(eager.state(), lazy.state())
    assert int(lazy.pending().max()) == 0
    e = state_err(lazy.state().cpu().numpy(), h)
    print(f"final state err {e:.2e}", flush=True)
    assert e <= BOUND[dtype]


def test_snapshot_with_rows_pending_continues_bit_for_bit():
    """A cache holding accepted rows not yet written back, copied byte for byte and attached
    as a second cache (a snapshot of the whole resumable context), continues exactly as the
    original: same outputs and states, bit for bit, over further rounds."""
    batch, H, P, N, G, K, kmax = 4, 4, 64, 64, 2, 4, 12
    rng = np.random.default_rng(6300)
    layer = synth.draw_layer(rng, H)
    A, D = dev_layer(layer)
    pre = synth.draw_tokens(rng, batch, 40, H, P, N, G, synth.BF16)
    orig = SSMCache(batch, H, P, N, G, kmax, synth.BF16)
    orig.prefill(*dev_tokens(pre), A, D, chunk=64, want_y=False)

    def round_(caches, drf, j):
        dx, dB, dC, ddt = dev_tokens(drf)
        ys = [c.verify(dx, dB, dC, ddt, A, D) for c in caches]
        for c in caches:
            c.commit(i32(j), dx, dB, ddt)
        return ys

    for _ in range(3):
        round_([orig], synth.draw_tokens(rng, batch, K, H, P, N, G, synth.BF16),
               synth.draw_accept_uniform(rng, batch, K))
    torch.cuda.synchronize()
    assert int(orig.pending().max()) > 0  # rows are pending in the snapshot
    raw = torch.empty_like(orig.buffer)
    raw.copy_(orig.buffer)
    copy = SSMCache(batch, H, P, N, G, kmax, synth.BF16, attach_to=raw)
    for r in range(4):
        ys = round_([orig, copy], synth.draw_tokens(rng, batch, K, H, P, N, G, synth.BF16),
                    synth.draw_accept_uniform(rng, batch, K))
        torch.cuda.synchronize()
        assert torch.equal(ys[0], ys[1]), r
        assert torch.equal(orig.buffer, copy.buffer), r
