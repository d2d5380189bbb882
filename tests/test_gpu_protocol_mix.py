"""GPU: the whole protocol with operations interleaved at random, round by round against
the oracle.

Each round is one of: a flat verify and commit of j accepted drafts, a tree verify and
commit of one accepted node's root path, a flat round whose commit folds at once
(materialize), or a prefill that continues the slots' logical state.  After every
round the outputs and the positions are checked against the oracle's; at the end a
round committed at once (materialize) folds every pending row, and the stored state is
checked too.  Tolerances as in the other parity tests (normwise per slice).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import BOUND, dev_layer, dev_tokens, state_err, y_err
from speculative_decode_amd import _lib as L
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.lib()  # a missing library is a failure, not a skip


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _random_parents(rng, Bt, K):
    """A random tree per slot: draft k hangs under the state (-1) or an earlier draft."""
    par = np.empty((Bt, K), dtype=np.int32)
    for b in range(Bt):
        for k in range(K):
            par[b, k] = rng.integers(-1, k)
    return par


# (batch, H, P, N, G), token dtype, drafts per round, pending rows the cache holds, seed;
# with more pending rows than drafts, accepted rows collect over rounds and a verify
# writes the state back only when a commit could overflow the pending area
CASES = [
    ((3, 4, 64, 64, 2), synth.BF16, 4, 4, 1),
    ((2, 4, 32, 32, 2), synth.F32, 5, 5, 2),
    ((1, 32, 128, 128, 8), synth.BF16, 4, 4, 3),
    ((3, 4, 64, 64, 2), synth.BF16, 4, 13, 4),
    ((2, 4, 32, 32, 2), synth.F32, 5, 16, 5),
]


@pytest.mark.parametrize("shape,dtype,K,kmax,seed", CASES,
                         ids=[f"{c[0][1]}h_P{c[0][2]}_N{c[0][3]}_{'bf16' if c[1] == synth.BF16 else 'f32'}_kmax{c[3]}"
                              for c in CASES])
def test_mixed_protocol_against_oracle(shape, dtype, K, kmax, seed):
    Bt, H, P, N, G = shape
    rng = np.random.default_rng(1000 + seed)
    layer = synth.draw_layer(rng, H)
    A, D = dev_layer(layer)
    Af, Df = layer.A.f64, layer.D.f64
    tol = BOUND[dtype]

    L0 = int(rng.integers(20, 300))
    pre = synth.draw_tokens(rng, Bt, L0, H, P, N, G, dtype)
    cache = SSMCache(Bt, H, P, N, G, kmax, dtype)
    y = _np(cache.prefill(*dev_tokens(pre), A, D, chunk=256))
    ry, ref = oracle.prefill(pre.x.f64, pre.B.f64, pre.C.f64, pre.dt.f64, Af, Df)
    assert y_err(y, ry) <= tol
    pos = np.full(Bt, L0)

    ops = ["flat", "tree", "materialize", "continue"]
    order = list(rng.permutation(ops)) + list(rng.choice(ops, size=6))
    for r, op in enumerate(order):
        if op == "continue":
            Lc = int(rng.integers(1, 300))
            tok = synth.draw_tokens(rng, Bt, Lc, H, P, N, G, dtype)
            y = _np(cache.prefill(*dev_tokens(tok), A, D, chunk=256, cont=True))
            ry, ref = oracle.prefill(tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, Af, Df, h0=ref)
            assert y_err(y, ry) <= tol, (r, op)
            pos += Lc
            continue
        drf = synth.draw_tokens(rng, Bt, K, H, P, N, G, dtype)
        dx, dB, dC, ddt = dev_tokens(drf)
        if op == "tree":
            par = _random_parents(rng, Bt, K)
            node = rng.integers(-1, K, size=Bt).astype(np.int32)
            y = _np(cache.verify_tree(_i32(par), dx, dB, dC, ddt, A, D))
            ry = oracle.verify_tree(ref, drf.x.f64, drf.B.f64, drf.C.f64, drf.dt.f64, Af, Df, par)
            assert y_err(y, ry) <= tol, (r, op)
            cache.commit_tree(_i32(par), _i32(node), dx, dB, ddt)
            ref, lengths = oracle.commit_tree(ref, drf.x.f64, drf.B.f64, drf.dt.f64, Af, Df, par, node)
            pos += lengths
        else:
            j = synth.draw_accept_uniform(rng, Bt, K)
            y = _np(cache.verify(dx, dB, dC, ddt, A, D))
            ry = oracle.verify(ref, drf.x.f64, drf.B.f64, drf.C.f64, drf.dt.f64, Af, Df)
            assert y_err(y, ry) <= tol, (r, op)
            cache.commit(_i32(j), dx, dB, ddt, A, D, materialize=(op == "materialize"))
            ref = oracle.commit(ref, drf.x.f64, drf.B.f64, drf.dt.f64, Af, Df, j)
            pos += j
        assert np.array_equal(_np(cache.pos()), pos), (r, op)

    # fold whatever is pending with one more flat round committed at once, then compare
    drf = synth.draw_tokens(rng, Bt, K, H, P, N, G, dtype)
    dx, dB, dC, ddt = dev_tokens(drf)
    j = synth.draw_accept_uniform(rng, Bt, K)
    cache.verify(dx, dB, dC, ddt, A, D)
    cache.commit(_i32(j), dx, dB, ddt, A, D, materialize=True)
    ref = oracle.commit(ref, drf.x.f64, drf.B.f64, drf.dt.f64, Af, Df, j)
    pos += j
    torch.cuda.synchronize()
    assert int(cache.pending().max().item()) == 0
    assert state_err(cache.state().cpu().numpy().astype(np.float64), ref) <= tol
    assert np.array_equal(_np(cache.pos()), pos)
    assert cache.status() == -1  # no slot reported a device-side error
