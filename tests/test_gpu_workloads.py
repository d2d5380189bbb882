"""Parity at the full workload sizes, in the same launch configurations the bench uses.

The oracle cannot redo every head of these sizes in seconds, so it recomputes sampled
heads one by one (each as a one-head, one-group problem on exactly the same inputs);
everything the GPU produced for those heads is compared.  Properties that hold at any
size (pos bookkeeping, untouched state on j = 0) are checked on all slots.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, dev_layer, dev_tokens, head_slice, slice_err
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from speculative_decode_amd import _lib
    _lib.lib()


def sampled_heads(H, G):
    hpg = H // G
    return [0, hpg + 1, H - 1]  # first group, a second-group head, last head


def check_heads(y_gpu, ref_fn, heads, tol, what):
    for h in heads:
        ry = ref_fn(h)
        e = slice_err(y_gpu[:, :, h:h + 1], ry, head_axis=2)
        print(f"{what} head {h}: err {e:.2e}")
        assert e <= tol, (what, h, e)


def test_llama8b_single_sequence():
    """One 8B-shaped sequence: 1024-token prefill, then verify K=4, commit j, verify again."""
    w = synth.WORKLOADS["llama8b_single"]
    rng = np.random.default_rng(w.seed)
    layer = synth.draw_layer(rng, w.H)
    pre = synth.draw_tokens(rng, w.batch, w.L, w.H, w.P, w.N, w.G, w.dtype)
    cache = SSMCache(w.batch, w.H, w.P, w.N, w.G, w.K, w.dtype)
    A, D = dev_layer(layer)
    y = cache.prefill(*dev_tokens(pre), A, D, chunk=w.chunk)
    torch.cuda.synchronize()
    ry, ref = oracle.prefill(pre.x.f64, pre.B.f64, pre.C.f64, pre.dt.f64, layer.A.f64, layer.D.f64)
    e = slice_err(y.cpu().numpy(), ry, head_axis=2)
    print(f"prefill y err {e:.2e}")
    assert e <= TOL[w.dtype]
    assert slice_err(cache.state().cpu().numpy(), ref, head_axis=1) <= TOL[w.dtype]
    for r in range(3):
        drf = synth.draw_tokens(rng, w.batch, w.K, w.H, w.P, w.N, w.G, w.dtype)
        j = synth.draw_accept_uniform(rng, w.batch, w.K)
        dx, dB, dC, ddt = dev_tokens(drf)
        yv = cache.verify(dx, dB, dC, ddt, A, D)
        torch.cuda.synchronize()
        ryv = oracle.verify(ref, drf.x.f64, drf.B.f64, drf.C.f64, drf.dt.f64, layer.A.f64, layer.D.f64)
        e = slice_err(yv.cpu().numpy(), ryv, head_axis=2)
        print(f"round {r} verify y err {e:.2e}")
        assert e <= TOL[w.dtype]
        cache.commit(torch.from_numpy(j).cuda(), dx, dB, ddt)
        ref = oracle.commit(ref, drf.x.f64, drf.B.f64, drf.dt.f64, layer.A.f64, layer.D.f64, j)


def test_llama8b_batched_verify():
    """Batch 16, contexts U{256..4096}, K=8, ragged accepted lengths; sampled heads."""
    w = synth.WORKLOADS["llama8b_batched"]
    rng = np.random.default_rng(w.seed)
    layer = synth.draw_layer(rng, w.H)
    ctx = rng.integers(w.ctx_range[0], w.ctx_range[1] + 1, size=w.batch)
    cache = SSMCache(w.batch, w.H, w.P, w.N, w.G, w.K, w.dtype)
    A, D = dev_layer(layer)
    heads = sampled_heads(w.H, w.G)
    refs = {}
    for b in range(w.batch):
        pre = synth.draw_tokens(rng, 1, int(ctx[b]), w.H, w.P, w.N, w.G, w.dtype)
        cache.prefill(*dev_tokens(pre), A, D, slot0=b, chunk=w.chunk, want_y=False)
        for h in heads:
            x, B, C, dt, Ah, Dh = head_slice(pre, layer, h, w.H, w.G)
            refs[(b, h)] = oracle.prefill(x, B, C, dt, Ah, Dh)[1]
    torch.cuda.synchronize()
    assert cache.pos().cpu().tolist() == ctx.tolist()
    pos = ctx.copy()
    for r in range(2):
        drf = synth.draw_tokens(rng, w.batch, w.K, w.H, w.P, w.N, w.G, w.dtype)
        j = synth.draw_accept_uniform(rng, w.batch, w.K)
        dx, dB, dC, ddt = dev_tokens(drf)
        yv = cache.verify(dx, dB, dC, ddt, A, D)
        torch.cuda.synchronize()
        yv = yv.cpu().numpy()
        for h in heads:
            x, B, C, dt, Ah, Dh = head_slice(drf, layer, h, w.H, w.G)
            st = np.concatenate([refs[(b, h)] for b in range(w.batch)], axis=0)
            ry = oracle.verify(st, x, B, C, dt, Ah, Dh)
            e = slice_err(yv[:, :, h:h + 1], ry, head_axis=2)
            print(f"round {r} head {h} verify err {e:.2e}")
            assert e <= TOL[w.dtype]
            nst = oracle.commit(st, x, B, dt, Ah, Dh, j)
            for b in range(w.batch):
                refs[(b, h)] = nst[b:b + 1]
        cache.commit(torch.from_numpy(j).cuda(), dx, dB, ddt, A, D, materialize=(r == 1))
        pos += j
    torch.cuda.synchronize()
    assert np.array_equal(cache.pos().cpu().numpy(), pos)
    state = cache.state().cpu().numpy()
    for h in heads:
        st = np.concatenate([refs[(b, h)] for b in range(w.batch)], axis=0)
        assert slice_err(state[:, h:h + 1], st, head_axis=1) <= TOL[w.dtype]


def test_long_prefill_8192():
    """One 8192-token scan, chunk 256: sampled heads' y and final state."""
    w = synth.WORKLOADS["llama8b_long_prefill"]
    rng = np.random.default_rng(w.seed)
    layer = synth.draw_layer(rng, w.H)
    tok = synth.draw_tokens(rng, w.batch, w.L, w.H, w.P, w.N, w.G, w.dtype)
    cache = SSMCache(w.batch, w.H, w.P, w.N, w.G, 4, w.dtype)
    A, D = dev_layer(layer)
    y = cache.prefill(*dev_tokens(tok), A, D, chunk=w.chunk)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    state = cache.state().cpu().numpy()
    for h in sampled_heads(w.H, w.G):
        x, B, C, dt, Ah, Dh = head_slice(tok, layer, h, w.H, w.G)
        ry, rs = oracle.prefill(x, B, C, dt, Ah, Dh)
        ey = slice_err(y[:, :, h:h + 1], ry, head_axis=2)
        es = slice_err(state[:, h:h + 1], rs, head_axis=1)
        print(f"long prefill head {h}: y {ey:.2e} state {es:.2e}")
        assert ey <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_hybrid_decode_layer():
    """One layer of the hybrid decode step: batch 32, N=256, K=4, geometric accepted
    lengths; prior state from a (shortened, 256-token) GPU prefill per sequence."""
    w = synth.WORKLOADS["hybrid_decode"]
    rng = np.random.default_rng(w.seed)
    layer = synth.draw_layer(rng, w.H)
    Lp = 256
    pre = synth.draw_tokens(rng, w.batch, Lp, w.H, w.P, w.N, w.G, w.dtype)
    cache = SSMCache(w.batch, w.H, w.P, w.N, w.G, w.K, w.dtype)
    A, D = dev_layer(layer)
    cache.prefill(*dev_tokens(pre), A, D, chunk=w.chunk, want_y=False)
    heads = sampled_heads(w.H, w.G)
    refs = {}
    for h in heads:
        x, B, C, dt, Ah, Dh = head_slice(pre, layer, h, w.H, w.G)
        refs[h] = oracle.prefill(x, B, C, dt, Ah, Dh)[1]
    for r in range(2):
        drf = synth.draw_tokens(rng, w.batch, w.K, w.H, w.P, w.N, w.G, w.dtype)
        j = synth.draw_accept_geometric(rng, w.batch, w.K)
        dx, dB, dC, ddt = dev_tokens(drf)
        yv = cache.verify(dx, dB, dC, ddt, A, D)
        torch.cuda.synchronize()
        yv = yv.cpu().numpy()
        for h in heads:
            x, B, C, dt, Ah, Dh = head_slice(drf, layer, h, w.H, w.G)
            e = slice_err(yv[:, :, h:h + 1], oracle.verify(refs[h], x, B, C, dt, Ah, Dh), head_axis=2)
            print(f"hybrid round {r} head {h}: err {e:.2e}")
            assert e <= TOL[w.dtype]
            refs[h] = oracle.commit(refs[h], x, B, dt, Ah, Dh, j)
        cache.commit(torch.from_numpy(j).cuda(), dx, dB, ddt)
