"""The multi-layer commit (mil_ssm_commit_layers) against one mil_ssm_commit per layer.

Two sets of caches hold the same bytes and verify the same drafts; one set commits all its
layers in one call, the other layer by layer.  Every cache byte (state, pending rows, pos,
pending, err) must then agree, and so must the next round's verify outputs; that round is
also checked against the oracle on one layer.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import BOUND, dev_layer, dev_tokens, y_err
from speculative_decode_amd import _lib as L
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache, commit_layers

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.lib()


def make_layers(rng, n, batch, H, P, N, G, K, dtype, Lp):
    layers, caches_a, caches_b, pres = [], [], [], []
    for _ in range(n):
        layer = synth.draw_layer(rng, H)
        pre = synth.draw_tokens(rng, batch, Lp, H, P, N, G, dtype)
        A, D = dev_layer(layer)
        a = SSMCache(batch, H, P, N, G, K, dtype)
        a.prefill(*dev_tokens(pre), A, D, chunk=64, want_y=False)
        b = SSMCache(batch, H, P, N, G, K, dtype)
        b.buffer.copy_(a.buffer)  # every byte alike, padding included
        caches_a.append(a)
        caches_b.append(b)
        layers.append((layer, A, D))
        pres.append(pre)
    return layers, caches_a, caches_b, pres


@pytest.mark.parametrize("dtype,n", [(synth.BF16, 3), (synth.F32, 3), (synth.BF16, 34)])
def test_commit_layers_matches_per_layer_commits(dtype, n):
    small = n > 8
    batch, H, P, N, G, K = (2, 2, 16, 16, 1, 4) if small else (5, 4, 64, 32, 2, 4)
    rng = np.random.default_rng(5100 + n + (dtype == synth.F32))
    print(f"commit_layers dtype={dtype} layers={n}", flush=True)
    layers, ca, cb, pres = make_layers(rng, n, batch, H, P, N, G, K, dtype, 40)
    refs = [oracle.prefill(p.x.f64, p.B.f64, p.C.f64, p.dt.f64, ly.A.f64, ly.D.f64)[1] for p, (ly, _, _) in
            zip(pres[:1], layers[:1])]
    for rnd in range(3):
        drafts = [synth.draw_tokens(rng, batch, K, H, P, N, G, dtype) for _ in range(n)]
        dev = [dev_tokens(d) for d in drafts]
        ya, yb = [], []
        for li in range(n):
            _, A, D = layers[li]
            ya.append(ca[li].verify(*dev[li], A, D))
            yb.append(cb[li].verify(*dev[li], A, D))
        j = synth.draw_accept_uniform(rng, batch, K)
        if rnd == 1:
            j[0] = K + 1  # rejected: err set in every layer, slot 0 unchanged
        jd = torch.from_numpy(j).cuda()
        commit_layers(ca, jd, [d[0] for d in dev], [d[1] for d in dev], [d[3] for d in dev])
        for li in range(n):
            cb[li].commit(jd, dev[li][0], dev[li][1], dev[li][3])
        torch.cuda.synchronize()
        for li in range(n):
            assert torch.equal(ya[li], yb[li]), (rnd, li)
            if not torch.equal(ca[li].buffer, cb[li].buffer):
                diff = torch.nonzero(ca[li].buffer != cb[li].buffer).flatten()
                raise AssertionError(f"round {rnd} layer {li}: {diff.numel()} bytes differ, first at "
                                     f"{int(diff[0])} (layout {dict((f, getattr(ca[li].layout, f)) for f, _ in ca[li].layout._fields_)})")
            assert ca[li].phase() == cb[li].phase() == L.PHASE_READY
        if rnd == 1:
            assert all(int(c.err()[0]) & L.MIL_DEVERR_ACCEPT for c in ca)
        # the oracle follows layer 0
        ly, _, _ = layers[0]
        d0 = drafts[0]
        ry = oracle.verify(refs[0], d0.x.f64, d0.B.f64, d0.C.f64, d0.dt.f64, ly.A.f64, ly.D.f64)
        e = y_err(ya[0].cpu().numpy(), ry)
        print(f"round {rnd}: layer 0 verify y err {e:.2e}", flush=True)
        assert e <= BOUND[dtype]
        jr = j.copy()
        jr[(jr < 0) | (jr > K)] = 0  # a rejected j leaves the slot's state where it was
        refs[0] = oracle.commit(refs[0], d0.x.f64, d0.B.f64, d0.dt.f64, ly.A.f64, ly.D.f64, jr)
        for c in ca + cb:
            c.status(clear=True)
