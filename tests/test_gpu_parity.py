"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Each test draws seeded synthetic inputs (speculative_decode_amd.synth), runs the GPU
path, runs the oracle on exactly the same (bf16-rounded or fp32) values widened to
double, and compares with the slice-normwise metric of gpu_util (1e-5 for fp32
inputs, 2e-3 for bf16).  Integer cases and the roll-back invariants are compared
bit for bit.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (BOUND, dev, dev_layer, dev_tokens, head_slice, state_err, y_err)
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from speculative_decode_amd import _lib
    _lib.lib()  # a missing library is a failure, not a skip


def sync_np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def logical_state(cache: SSMCache) -> np.ndarray:
    """Stored state; only meaningful when no rows are pending."""
    torch.cuda.synchronize()
    assert int(cache.pending().max().item()) == 0
    return cache.state().cpu().numpy().astype(np.float64)


def make_layer_and_tokens(rng, batch, T, H, P, N, G, dtype, a_mode="cfg"):
    layer = synth.draw_layer(rng, H)
    if a_mode == "zero":
        layer = synth.Layer(synth.quantize(np.zeros(H), synth.F32), layer.D)
    elif a_mode == "tiny":
        layer = synth.Layer(synth.quantize(np.full(H, -1e-3), synth.F32), layer.D)
    tok = synth.draw_tokens(rng, batch, T, H, P, N, G, dtype)
    return layer, tok


# --------------------------------------------------------------------------- prefill

# (B, H, P, N, G): N = 32 takes the vector-ALU kernels; N = 64 / 128 with bf16 inputs
# takes the matrix-core kernels
VALU_SHAPE = (2, 4, 32, 32, 2)
MFMA_SHAPE = (2, 4, 64, 64, 2)
PREFILL_CASES = []
for dtype, shape in ((synth.F32, VALU_SHAPE), (synth.BF16, VALU_SHAPE), (synth.BF16, MFMA_SHAPE)):
    for L in (1, 31, 32, 33, 63, 64, 65, 255, 256, 257, 1000):
        for chunk in (64, 256):
            PREFILL_CASES.append((dtype, shape, L, chunk, "cfg"))
    for a_mode in ("zero", "tiny"):
        for (L, chunk) in ((300, 64), (1000, 128), (600, 256)):
            PREFILL_CASES.append((dtype, shape, L, chunk, a_mode))


@pytest.mark.parametrize("dtype,shape,L,chunk,a_mode", PREFILL_CASES)
def test_prefill_matches_oracle(dtype, shape, L, chunk, a_mode):
    rng = np.random.default_rng(7000 + L + chunk)
    Bt, H, P, N, G = shape
    layer, tok = make_layer_and_tokens(rng, Bt, L, H, P, N, G, dtype, a_mode)
    cache = SSMCache(Bt, H, P, N, G, 4, dtype)
    A, D = dev_layer(layer)
    y = sync_np(cache.prefill(*dev_tokens(tok), A, D, chunk=chunk))
    ry, rs = oracle.prefill(tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, layer.A.f64, layer.D.f64)
    ey, es = y_err(y, ry), state_err(logical_state(cache), rs)
    print(f"prefill {dtype} L={L} chunk={chunk} A={a_mode}: y {ey:.2e} state {es:.2e}")
    assert ey <= BOUND[dtype] and es <= BOUND[dtype]
    assert cache.pos().cpu().tolist() == [L] * Bt


@pytest.mark.parametrize("shape", [(1, 2, 16, 16, 1), (2, 4, 64, 16, 4), (1, 2, 128, 64, 1), (1, 4, 256, 32, 2),
                                   (1, 2, 16, 256, 2), (1, 2, 32, 128, 1), (1, 4, 128, 128, 4), (1, 2, 256, 64, 2),
                                   (1, 2, 64, 256, 1), (1, 2, 128, 256, 2), (1, 1, 256, 256, 1)])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("chunk", [128, 256])
def test_prefill_shapes(shape, dtype, chunk):
    Bt, H, P, N, G = shape
    rng = np.random.default_rng(sum(shape))
    layer, tok = make_layer_and_tokens(rng, Bt, 300, H, P, N, G, dtype)
    cache = SSMCache(Bt, H, P, N, G, 4, dtype)
    y = sync_np(cache.prefill(*dev_tokens(tok), *dev_layer(layer), chunk=chunk))
    ry, rs = oracle.prefill(tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, layer.A.f64, layer.D.f64)
    assert y_err(y, ry) <= BOUND[dtype]
    assert state_err(logical_state(cache), rs) <= BOUND[dtype]


def test_prefill_misaligned_inputs_take_the_vector_path():
    """Token tensors only 2-byte aligned cannot use the 16-byte loads of the matrix-core
    kernels; the result must be the same to tolerance."""
    rng = np.random.default_rng(37)
    Bt, L, H, P, N, G = 1, 200, 4, 64, 64, 2
    layer, tok = make_layer_and_tokens(rng, Bt, L, H, P, N, G, synth.BF16)
    cache = SSMCache(Bt, H, P, N, G, 4, synth.BF16)
    x, B, C, dt = dev_tokens(tok)
    xs = torch.empty(x.numel() + 1, dtype=x.dtype, device=x.device)
    xs[1:].copy_(x.reshape(-1))
    xm = xs[1:].view(x.shape)
    assert xm.data_ptr() % 16 != 0
    y = sync_np(cache.prefill(xm, B, C, dt, *dev_layer(layer), chunk=64))
    ry, rs = oracle.prefill(tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, layer.A.f64, layer.D.f64)
    assert y_err(y, ry) <= BOUND[synth.BF16]
    assert state_err(logical_state(cache), rs) <= BOUND[synth.BF16]


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("shape", [(2, 4, 32, 16, 2), (2, 4, 64, 64, 2)])
def test_integer_linear_attention_is_exact(dtype, shape):
    """A = 0, dt = 1, inputs in {-1, 0, 1}: every value is an exact small integer, so
    prefill, verify and the folded state must match the oracle exactly."""
    rng = np.random.default_rng(31)
    Bt, H, P, N, G = shape
    L, K = 150, 4
    tok = synth.integer_tokens(rng, Bt, L + K, H, P, N, G, dtype)
    layer = synth.Layer(synth.quantize(np.zeros(H), synth.F32),
                        synth.quantize(rng.integers(-2, 3, size=H).astype(np.float64), synth.F32))
    pre = synth.slice_tokens(tok, 0, Bt, 0, L)
    drf = synth.slice_tokens(tok, 0, Bt, L, L + K)
    cache = SSMCache(Bt, H, P, N, G, K, dtype)
    A, D = dev_layer(layer)
    y = sync_np(cache.prefill(*dev_tokens(pre), A, D, chunk=64))
    ry, rs = oracle.prefill(pre.x.f64, pre.B.f64, pre.C.f64, pre.dt.f64, layer.A.f64, layer.D.f64)
    assert np.array_equal(y.astype(np.float64), ry)
    assert np.array_equal(logical_state(cache), rs)
    yv = sync_np(cache.verify(*dev_tokens(drf), A, D))
    assert np.array_equal(yv.astype(np.float64),
                          oracle.verify(rs, drf.x.f64, drf.B.f64, drf.C.f64, drf.dt.f64, layer.A.f64, layer.D.f64))
    j = np.array([3, 1], dtype=np.int32)
    dx, dB, dC, ddt = dev_tokens(drf)
    cache.commit(torch.from_numpy(j).cuda(), dx, dB, ddt, A, D, materialize=True)
    assert np.array_equal(logical_state(cache),
                          oracle.commit(rs, drf.x.f64, drf.B.f64, drf.dt.f64, layer.A.f64, layer.D.f64, j))


@pytest.mark.parametrize("chunk", [64, 256])
@pytest.mark.parametrize("shape", [VALU_SHAPE, MFMA_SHAPE])
def test_prefill_continue_after_pending_rows(shape, chunk):
    """prefill L1, verify K, commit j (deferred), prefill L2 with CONTINUE == prefill of
    L1 + j accepted drafts + L2."""
    rng = np.random.default_rng(41)
    Bt, H, P, N, G = shape
    L1, K, L2 = 100, 4, 157
    dtype = synth.BF16
    layer, tok = make_layer_and_tokens(rng, Bt, L1 + K + L2, H, P, N, G, dtype)
    a = synth.slice_tokens(tok, 0, Bt, 0, L1)
    d = synth.slice_tokens(tok, 0, Bt, L1, L1 + K)
    c = synth.slice_tokens(tok, 0, Bt, L1 + K, L1 + K + L2)
    cache = SSMCache(Bt, H, P, N, G, K, dtype)
    A, D = dev_layer(layer)
    cache.prefill(*dev_tokens(a), A, D, chunk=chunk)
    dx, dB, dC, ddt = dev_tokens(d)
    cache.verify(dx, dB, dC, ddt, A, D)
    j = np.array([2, 4], dtype=np.int32)
    cache.commit(torch.from_numpy(j).cuda(), dx, dB, ddt)
    y2 = sync_np(cache.prefill(*dev_tokens(c), A, D, chunk=chunk, cont=True))
    _, h1 = oracle.prefill(a.x.f64, a.B.f64, a.C.f64, a.dt.f64, layer.A.f64, layer.D.f64)
    h1 = oracle.commit(h1, d.x.f64, d.B.f64, d.dt.f64, layer.A.f64, layer.D.f64, j)
    ry, rs = oracle.prefill(c.x.f64, c.B.f64, c.C.f64, c.dt.f64, layer.A.f64, layer.D.f64, h0=h1)
    assert y_err(y2, ry) <= BOUND[dtype]
    assert state_err(logical_state(cache), rs) <= BOUND[dtype]
    assert cache.pos().cpu().tolist() == [L1 + int(j[0]) + L2, L1 + int(j[1]) + L2]


@pytest.mark.parametrize("L", [257, 1000, 2048, 2100])
def test_prefill_back_to_back_single_launch(L):
    """The single-launch prefill hands chunk states between workgroups through flags in
    the cache: calls one after another on the slots of one cache (the flags reused call
    after call) report no error and match the oracle."""
    Bt, H, P, N, G = 3, 8, 128, 128, 4
    rng = np.random.default_rng(4200 + L)
    layer, tok = make_layer_and_tokens(rng, Bt, L, H, P, N, G, synth.BF16, "tiny")
    A, D = dev_layer(layer)
    cache = SSMCache(Bt, H, P, N, G, 4, synth.BF16)
    ys = []
    for b in range(Bt):   # one slot at a time: the counters are reused call after call
        one = synth.slice_tokens(tok, b, b + 1, 0, L)
        ys.append(sync_np(cache.prefill(*dev_tokens(one), A, D, slot0=b, chunk=256)))
    assert cache.status() == -1
    ry, rs = oracle.prefill(tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, layer.A.f64, layer.D.f64)
    assert y_err(np.concatenate(ys), ry) <= BOUND[synth.BF16]
    assert state_err(logical_state(cache), rs) <= BOUND[synth.BF16]


# The single launch's column slab follows from the number of chunk-heads (P halved until
# there is a workgroup per compute unit; at most 64 columns where N = 64, whole heads of
# 128 where N = 128), so the number of sequences picks it: with P = 128, 8 heads and 4
# chunks, 2 sequences give slabs of 32 columns, 4 give 64, and 8 give 64 (N = 64, two
# workgroups per compute unit: the later chunks' waits span dispatch rounds) or whole heads
# (N = 128).
SCAN_CONFIGS = [(64, 2), (64, 4), (64, 8), (128, 2), (128, 4), (128, 8)]


@pytest.mark.parametrize("N,Bt", SCAN_CONFIGS, ids=[f"N{n}_batch{b}" for n, b in SCAN_CONFIGS])
def test_prefill_single_launch_configs(N, Bt):
    """Every state size and column slab of the single-launch prefill, on a ragged last
    chunk (1000 tokens = 3 x 256 + 232)."""
    from speculative_decode_amd import _lib
    H, P, G, L = 8, 128, 2, 1000
    rng = np.random.default_rng(4300 + N + Bt)
    layer, tok = make_layer_and_tokens(rng, Bt, L, H, P, N, G, synth.BF16)
    cache = SSMCache(Bt, H, P, N, G, 4, synth.BF16)
    mask = _lib.lib().mil_ssm_prefill_kernels(ctypes.byref(cache.desc), Bt, L, 256)
    assert mask == 1 << _lib.TRACE["prefill_scan"], mask
    print(f"single-launch prefill N={N} batch={Bt}", flush=True)
    y = sync_np(cache.prefill(*dev_tokens(tok), *dev_layer(layer), chunk=256))
    assert cache.status() == -1
    ry, rs = oracle.prefill(tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, layer.A.f64, layer.D.f64)
    ey, es = y_err(y, ry), state_err(logical_state(cache), rs)
    print(f"  y {ey:.2e} state {es:.2e}")
    assert ey <= BOUND[synth.BF16] and es <= BOUND[synth.BF16]


LONG_CASES = [(L, a) for L in (2048, 2100, 4096, 8192) for a in ("zero", "tiny")] + [(16684, "tiny"), (16684, "cfg")]


@pytest.mark.parametrize("L,a_mode", LONG_CASES, ids=[f"L{L}_{a}" for L, a in LONG_CASES])
def test_single_launch_long_prompts(L, a_mode):
    """Prompts of many chunks through the single launch with decoupled look-back: each
    chunk publishes its own contribution, then (after looking back to the nearest chunk
    that has published the state after it) the state after itself.  A = 0 and -1e-3 carry
    the state across every chunk boundary.  16684 tokens (66 chunks) take two launches of
    at most 64 chunks, the second continuing from the state the first wrote."""
    from speculative_decode_amd import _lib
    Bt, H, P, N, G = (1, 8, 128, 128, 2) if L <= 8192 else (1, 4, 128, 128, 1)
    rng = np.random.default_rng(4600 + L)
    layer, tok = make_layer_and_tokens(rng, Bt, L, H, P, N, G, synth.BF16, a_mode)
    cache = SSMCache(Bt, H, P, N, G, 4, synth.BF16)
    assert cache.prefill_kernels(Bt, L) == 1 << _lib.TRACE["prefill_scan"]
    A, D = dev_layer(layer)
    print(f"single-launch prefill L={L} A={a_mode}", flush=True)
    y = sync_np(cache.prefill(*dev_tokens(tok), A, D, chunk=256))
    assert cache.status() == -1
    ry, rs = oracle.prefill(tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, layer.A.f64, layer.D.f64)
    ey, es = y_err(y, ry), state_err(logical_state(cache), rs)
    print(f"  y {ey:.2e} state {es:.2e}")
    assert ey <= BOUND[synth.BF16] and es <= BOUND[synth.BF16]
    assert cache.pos().cpu().tolist() == [L] * Bt
    launches = -(-((L + 255) // 256) // 64)
    epochs = cache.scan_words().cpu().numpy()[..., SSMCache.SCAN_EPOCH]
    assert epochs.any() and set(np.unique(epochs[epochs != 0]).tolist()) <= set(range(1, launches + 1))


def test_single_launch_long_prompt_is_bitwise_repeatable():
    """The look-back may end at different chunks from one run to the next, but the state a
    chunk receives is always the same fold in the same order: two runs of an 8192-token
    prefill give the same bits."""
    Bt, H, P, N, G, L = 1, 8, 128, 128, 2, 8192
    rng = np.random.default_rng(4700)
    layer, tok = make_layer_and_tokens(rng, Bt, L, H, P, N, G, synth.BF16, "tiny")
    A, D = dev_layer(layer)
    outs = []
    for _ in range(2):
        cache = SSMCache(Bt, H, P, N, G, 4, synth.BF16)
        y = cache.prefill(*dev_tokens(tok), A, D, chunk=256)
        torch.cuda.synchronize()
        outs.append((y.cpu(), cache.state().contiguous().cpu()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("want_y", [True, False], ids=["y", "state_only"])
def test_single_launch_continue(want_y):
    """Prefill, verify, commit, then a several-chunk prefill that continues from the
    committed state, all through the single launch (chunk 0 starts from the cache's state,
    the later chunks fold it through the published ones), with y or the state alone."""
    from speculative_decode_amd import _lib
    Bt, H, P, N, G = 2, 8, 128, 128, 2
    L1, K, L2 = 600, 4, 1000
    rng = np.random.default_rng(4400 + want_y)
    layer, tok = make_layer_and_tokens(rng, Bt, L1 + K + L2, H, P, N, G, synth.BF16)
    a = synth.slice_tokens(tok, 0, Bt, 0, L1)
    d = synth.slice_tokens(tok, 0, Bt, L1, L1 + K)
    c = synth.slice_tokens(tok, 0, Bt, L1 + K, L1 + K + L2)
    cache = SSMCache(Bt, H, P, N, G, K, synth.BF16)
    for n in (L1, L2):
        assert _lib.lib().mil_ssm_prefill_kernels(ctypes.byref(cache.desc), Bt, n, 256) == \
            1 << _lib.TRACE["prefill_scan"]
    A, D = dev_layer(layer)
    print(f"single-launch continue, y={want_y}", flush=True)
    cache.prefill(*dev_tokens(a), A, D, chunk=256)
    dx, dB, dC, ddt = dev_tokens(d)
    cache.verify(dx, dB, dC, ddt, A, D)
    j = np.array([3, 1], dtype=np.int32)
    cache.commit(torch.from_numpy(j).cuda(), dx, dB, ddt)
    y2 = cache.prefill(*dev_tokens(c), A, D, chunk=256, cont=True, want_y=want_y)
    torch.cuda.synchronize()
    assert cache.status() == -1
    _, h1 = oracle.prefill(a.x.f64, a.B.f64, a.C.f64, a.dt.f64, layer.A.f64, layer.D.f64)
    h1 = oracle.commit(h1, d.x.f64, d.B.f64, d.dt.f64, layer.A.f64, layer.D.f64, j)
    ry, rs = oracle.prefill(c.x.f64, c.B.f64, c.C.f64, c.dt.f64, layer.A.f64, layer.D.f64, h0=h1)
    if want_y:
        assert y_err(sync_np(y2), ry) <= BOUND[synth.BF16]
    assert state_err(logical_state(cache), rs) <= BOUND[synth.BF16]
    assert cache.pos().cpu().tolist() == [L1 + int(j[0]) + L2, L1 + int(j[1]) + L2]


# Where N = 128 and the prompt has at least one workgroup per compute unit at 128 columns
# (sequences x chunks x heads >= 256), the single launch takes whole heads (no column slabs):
# each C B^T tile and its decay mask is formed once per head, the light waves store their
# state tiles as they form them and read them back later, and the carried state reuses
# X^T's LDS.  These cases reach that form: one short chunk per sequence (chunk 0 is also
# the last), and several chunks continuing from a committed state, with y or without.
WIDE_CASES = [("one_chunk", 8, 200, 0), ("continue_y", 2, 1000, 1), ("continue_state", 2, 1000, 2)]


@pytest.mark.parametrize("name,Bt,L,mode", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_single_launch_whole_heads(name, Bt, L, mode):
    from speculative_decode_amd import _lib
    H, P, N, G, L1, K = 32, 128, 128, 8, 300, 4
    rng = np.random.default_rng(4800 + mode)
    layer, tok = make_layer_and_tokens(rng, Bt, L1 + K + L, H, P, N, G, synth.BF16, "tiny")
    A, D = dev_layer(layer)
    cache = SSMCache(Bt, H, P, N, G, K, synth.BF16)
    assert _lib.lib().mil_ssm_prefill_kernels(ctypes.byref(cache.desc), Bt, L, 256) == \
        1 << _lib.TRACE["prefill_scan"]
    print(f"single-launch whole heads {name}", flush=True)
    c = synth.slice_tokens(tok, 0, Bt, L1 + K, L1 + K + L)
    h1 = None
    if mode:
        a = synth.slice_tokens(tok, 0, Bt, 0, L1)
        d = synth.slice_tokens(tok, 0, Bt, L1, L1 + K)
        cache.prefill(*dev_tokens(a), A, D, chunk=256)
        dx, dB, dC, ddt = dev_tokens(d)
        cache.verify(dx, dB, dC, ddt, A, D)
        j = np.array([3, 0], dtype=np.int32)
        cache.commit(torch.from_numpy(j).cuda(), dx, dB, ddt)
        _, h1 = oracle.prefill(a.x.f64, a.B.f64, a.C.f64, a.dt.f64, layer.A.f64, layer.D.f64)
        h1 = oracle.commit(h1, d.x.f64, d.B.f64, d.dt.f64, layer.A.f64, layer.D.f64, j)
    y = cache.prefill(*dev_tokens(c), A, D, chunk=256, cont=bool(mode), want_y=mode != 2)
    torch.cuda.synchronize()
    assert cache.status() == -1
    ry, rs = oracle.prefill(c.x.f64, c.B.f64, c.C.f64, c.dt.f64, layer.A.f64, layer.D.f64, h0=h1)
    es = state_err(logical_state(cache), rs)
    ey = y_err(sync_np(y), ry) if mode != 2 else 0.0
    print(f"  y {ey:.2e} state {es:.2e}")
    assert ey <= BOUND[synth.BF16] and es <= BOUND[synth.BF16]


# --------------------------------------------------------------------------- verify / commit

def test_tiny_f32_protocol_against_oracle():
    """The tiny fp32 workload: prefill 64 tokens, then rounds of verify K=4 and commit
    j ~ U{0..4}; every y and the final state against the oracle at 1e-5."""
    w = synth.WORKLOADS["tiny_f32"]
    rng = np.random.default_rng(w.seed)
    layer = synth.draw_layer(rng, w.H)
    pre = synth.draw_tokens(rng, w.batch, w.L, w.H, w.P, w.N, w.G, w.dtype)
    cache = SSMCache(w.batch, w.H, w.P, w.N, w.G, w.K, w.dtype)
    A, D = dev_layer(layer)
    y = sync_np(cache.prefill(*dev_tokens(pre), A, D, chunk=w.chunk))
    ry, ref = oracle.prefill(pre.x.f64, pre.B.f64, pre.C.f64, pre.dt.f64, layer.A.f64, layer.D.f64)
    assert y_err(y, ry) <= 1e-5
    assert state_err(logical_state(cache), ref) <= 1e-5
    total = w.L
    for r in range(8):
        drf = synth.draw_tokens(rng, w.batch, w.K, w.H, w.P, w.N, w.G, w.dtype)
        j = synth.draw_accept_uniform(rng, w.batch, w.K)
        dx, dB, dC, ddt = dev_tokens(drf)
        yv = sync_np(cache.verify(dx, dB, dC, ddt, A, D))
        ey = y_err(yv, oracle.verify(ref, drf.x.f64, drf.B.f64, drf.C.f64, drf.dt.f64, layer.A.f64, layer.D.f64))
        assert ey <= 1e-5, (r, ey)
        cache.commit(torch.from_numpy(j).cuda(), dx, dB, ddt, A, D, materialize=(r == 7))
        ref = oracle.commit(ref, drf.x.f64, drf.B.f64, drf.dt.f64, layer.A.f64, layer.D.f64, j)
        total += int(j[0])
    assert state_err(logical_state(cache), ref) <= 1e-5
    assert cache.pos().cpu().tolist() == [total]


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("shape", [(3, 4, 16, 16, 2), (2, 4, 32, 64, 1), (2, 2, 128, 128, 1), (2, 4, 64, 256, 2),
                                   (1, 2, 256, 32, 2), (1, 1, 256, 256, 1)])
@pytest.mark.parametrize("K,k_max", [(1, 1), (4, 4), (5, 8), (8, 8), (16, 16)])
def test_verify_rounds_against_oracle(dtype, shape, K, k_max):
    """Several rounds with ragged accepted lengths per sequence: y of every round and
    pos exactly; the final folded state against the oracle."""
    verify_rounds(dtype, shape, K, k_max)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("shape,K,k_max", [((8, 32, 128, 256, 8), 4, 8), ((8, 32, 128, 256, 8), 16, 16),
                                           ((8, 32, 256, 128, 8), 4, 4), ((8, 32, 256, 128, 8), 1, 3)])
def test_verify_rounds_whole_row_workgroups(dtype, shape, K, k_max):
    """The launch that gives each 8-wave workgroup a whole (slot, head) block with 16 rows
    per lane (N x P = 32768 floats per head, at least 256 slot-heads): the same rounds
    against the oracle, in both orientations of N and P, with deferred and immediate
    write-back and the most drafts."""
    verify_rounds(dtype, shape, K, k_max)


def verify_rounds(dtype, shape, K, k_max):
    Bt, H, P, N, G = shape
    rng = np.random.default_rng(100 * K + Bt * H + P + N)
    layer, pre = make_layer_and_tokens(rng, Bt, 37, H, P, N, G, dtype)
    cache = SSMCache(Bt, H, P, N, G, k_max, dtype)
    A, D = dev_layer(layer)
    cache.prefill(*dev_tokens(pre), A, D, chunk=64, want_y=False)
    _, ref = oracle.prefill(pre.x.f64, pre.B.f64, pre.C.f64, pre.dt.f64, layer.A.f64, layer.D.f64)
    pos = np.full(Bt, 37)
    for r in range(4):
        drf = synth.draw_tokens(rng, Bt, K, H, P, N, G, dtype)
        j = synth.draw_accept_uniform(rng, Bt, K)
        if r == 1:
            j[:] = K
        if r == 2:
            j[:] = 0
        dx, dB, dC, ddt = dev_tokens(drf)
        yv = sync_np(cache.verify(dx, dB, dC, ddt, A, D))
        ry = oracle.verify(ref, drf.x.f64, drf.B.f64, drf.C.f64, drf.dt.f64, layer.A.f64, layer.D.f64)
        assert y_err(yv, ry) <= BOUND[dtype], r
        cache.commit(torch.from_numpy(j).cuda(), dx, dB, ddt, A, D, materialize=(r == 3))
        ref = oracle.commit(ref, drf.x.f64, drf.B.f64, drf.dt.f64, layer.A.f64, layer.D.f64, j)
        pos += j
    assert np.array_equal(cache.pos().cpu().numpy(), pos)
    assert state_err(logical_state(cache), ref) <= BOUND[dtype]


def _prefilled_cache(rng, Bt, H, P, N, G, k_max, dtype, L=50):
    layer, pre = make_layer_and_tokens(rng, Bt, L, H, P, N, G, dtype)
    cache = SSMCache(Bt, H, P, N, G, k_max, dtype)
    A, D = dev_layer(layer)
    cache.prefill(*dev_tokens(pre), A, D, chunk=64, want_y=False)
    return layer, pre, cache, A, D


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_rollback_is_bit_exact(dtype):
    """Keeping j of K drafts gives the same raw state bits as verifying only those j
    drafts, and as j single-token rounds (one state step, one order, everywhere)."""
    Bt, H, P, N, G, K = 1, 4, 128, 128, 2, 8
    for j in range(K + 1):
        states = []
        seed = 500 + j
        layer, _, _, _, _ = _prefilled_cache(np.random.default_rng(seed), Bt, H, P, N, G, K, dtype)
        drf = synth.draw_tokens(np.random.default_rng(seed + 1), Bt, K, H, P, N, G, dtype)
        for mode in ("all_K", "only_j", "single"):
            _, _, cache, A, D = _prefilled_cache(np.random.default_rng(seed), Bt, H, P, N, G, K, dtype)
            jj = torch.tensor([j], dtype=torch.int32, device="cuda")
            if mode == "all_K":
                dx, dB, dC, ddt = dev_tokens(drf)
                cache.verify(dx, dB, dC, ddt, A, D)
                cache.commit(jj, dx, dB, ddt, A, D, materialize=True)
            elif mode == "only_j" and j > 0:
                d = synth.slice_tokens(drf, 0, Bt, 0, j)
                dx, dB, dC, ddt = dev_tokens(d)
                cache.verify(dx, dB, dC, ddt, A, D)
                cache.commit(jj, dx, dB, ddt, A, D, materialize=True)
            elif mode == "single":
                one = torch.tensor([1], dtype=torch.int32, device="cuda")
                for i in range(j):
                    d = synth.slice_tokens(drf, 0, Bt, i, i + 1)
                    dx, dB, dC, ddt = dev_tokens(d)
                    cache.verify(dx, dB, dC, ddt, A, D)
                    cache.commit(one, dx, dB, ddt, A, D, materialize=(i == j - 1))
            torch.cuda.synchronize()
            states.append(cache.state().contiguous().view(torch.int32).cpu().numpy())
        assert np.array_equal(states[0], states[1]), j
        assert np.array_equal(states[0], states[2]), j


def test_commit_zero_then_same_drafts_gives_same_y():
    rng = np.random.default_rng(61)
    Bt, H, P, N, G, K = 2, 4, 128, 128, 2, 4
    layer, _, cache, A, D = _prefilled_cache(rng, Bt, H, P, N, G, K, synth.BF16)
    # leave pending rows so that the first verify has something to fold
    d0 = synth.draw_tokens(rng, Bt, K, H, P, N, G, synth.BF16)
    dx, dB, dC, ddt = dev_tokens(d0)
    cache.verify(dx, dB, dC, ddt, A, D)
    cache.commit(torch.tensor([3, 2], dtype=torch.int32, device="cuda"), dx, dB, ddt)
    d1 = synth.draw_tokens(rng, Bt, K, H, P, N, G, synth.BF16)
    dx, dB, dC, ddt = dev_tokens(d1)
    y1 = cache.verify(dx, dB, dC, ddt, A, D).clone()
    cache.commit(torch.zeros(Bt, dtype=torch.int32, device="cuda"), dx, dB, ddt)
    y2 = cache.verify(dx, dB, dC, ddt, A, D).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    cache.commit(torch.zeros(Bt, dtype=torch.int32, device="cuda"), dx, dB, ddt)


def test_repeated_runs_are_bitwise_equal():
    outs = []
    for _ in range(2):
        rng = np.random.default_rng(71)
        Bt, H, P, N, G, K = 2, 8, 128, 128, 2, 8
        layer, pre, cache, A, D = _prefilled_cache(rng, Bt, H, P, N, G, K, synth.BF16, L=700)
        y = cache.prefill(*dev_tokens(pre), A, D, chunk=256)
        d = synth.draw_tokens(rng, Bt, K, H, P, N, G, synth.BF16)
        yv = cache.verify(*dev_tokens(d), A, D)
        torch.cuda.synchronize()
        outs.append((y.cpu(), yv.cpu(), cache.state().contiguous().cpu()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_bad_accepted_length_sets_error_and_changes_nothing():
    rng = np.random.default_rng(81)
    Bt, H, P, N, G, K = 3, 4, 64, 32, 2, 4
    layer, pre, cache, A, D = _prefilled_cache(rng, Bt, H, P, N, G, K, synth.BF16)
    _, ref = oracle.prefill(pre.x.f64, pre.B.f64, pre.C.f64, pre.dt.f64, layer.A.f64, layer.D.f64)
    drf = synth.draw_tokens(rng, Bt, K, H, P, N, G, synth.BF16)
    dx, dB, dC, ddt = dev_tokens(drf)
    cache.verify(dx, dB, dC, ddt, A, D)
    j = np.array([K + 1, -1, 2], dtype=np.int32)
    cache.commit(torch.from_numpy(j).cuda(), dx, dB, ddt, A, D, materialize=True)
    assert cache.status() == 0
    assert cache.err().cpu().tolist() == [1, 1, 0]
    assert cache.pos().cpu().tolist() == [50, 50, 52]
    ref = oracle.commit(ref, drf.x.f64, drf.B.f64, drf.dt.f64, layer.A.f64, layer.D.f64, np.array([0, 0, 2]))
    assert state_err(logical_state(cache), ref) <= BOUND[synth.BF16]
    assert cache.status(clear=True) == 0
    assert cache.status() == -1
    # the protocol goes on
    cache.verify(dx, dB, dC, ddt, A, D)
    cache.commit(torch.zeros(Bt, dtype=torch.int32, device="cuda"), dx, dB, ddt)


@pytest.mark.parametrize("kind", ["commit", "commit_tree"])
def test_error_bits_accumulate(kind):
    """err is the OR of every device error a slot has seen: a bad accepted length (or node)
    adds MIL_DEVERR_ACCEPT to a bit set earlier and erases nothing."""
    from speculative_decode_amd._lib import MIL_DEVERR_ACCEPT, MIL_DEVERR_SCAN, MIL_DEVERR_TREE
    rng = np.random.default_rng(83)
    Bt, H, P, N, G, K = 3, 4, 64, 32, 2, 4
    layer, pre, cache, A, D = _prefilled_cache(rng, Bt, H, P, N, G, K, synth.BF16)
    cache.err().copy_(torch.tensor([MIL_DEVERR_SCAN, MIL_DEVERR_TREE, 0], dtype=torch.int32, device="cuda"))
    drf = synth.draw_tokens(rng, Bt, K, H, P, N, G, synth.BF16)
    dx, dB, dC, ddt = dev_tokens(drf)
    bad = np.array([K + 1, 2, -3], dtype=np.int32)  # slot 1 is fine
    if kind == "commit":
        cache.verify(dx, dB, dC, ddt, A, D)
        cache.commit(torch.from_numpy(bad).cuda(), dx, dB, ddt)
    else:
        parent = torch.from_numpy(np.tile(np.arange(-1, K - 1, dtype=np.int32), (Bt, 1))).cuda()
        cache.verify_tree(parent, dx, dB, dC, ddt, A, D)
        cache.commit_tree(parent, torch.from_numpy(np.array([K, 1, -2], dtype=np.int32)).cuda(), dx, dB, ddt)
    torch.cuda.synchronize()
    assert cache.err().cpu().tolist() == [MIL_DEVERR_SCAN | MIL_DEVERR_ACCEPT, MIL_DEVERR_TREE, MIL_DEVERR_ACCEPT]
    assert cache.pos().cpu().tolist() == [50, 52, 50]


def test_protocol_order_errors():
    from speculative_decode_amd._lib import MilError, MIL_E_ORDER
    rng = np.random.default_rng(91)
    Bt, H, P, N, G, K = 1, 2, 16, 16, 1, 4
    layer, pre, cache, A, D = _prefilled_cache(rng, Bt, H, P, N, G, K, synth.F32)
    d = synth.draw_tokens(rng, Bt, K, H, P, N, G, synth.F32)
    dx, dB, dC, ddt = dev_tokens(d)
    with pytest.raises(MilError) as e:
        cache.commit(torch.zeros(1, dtype=torch.int32, device="cuda"), dx, dB, ddt)
    assert e.value.status == MIL_E_ORDER
    cache.verify(dx, dB, dC, ddt, A, D)
    with pytest.raises(MilError) as e:
        cache.verify(dx, dB, dC, ddt, A, D)
    assert e.value.status == MIL_E_ORDER
    with pytest.raises(MilError) as e:
        cache.prefill(*dev_tokens(pre), A, D)
    assert e.value.status == MIL_E_ORDER
    with pytest.raises(TypeError):
        cache.commit(torch.zeros(1, dtype=torch.int32, device="cuda"), dx.to(torch.bfloat16), dB, ddt)
    cache.commit(torch.zeros(1, dtype=torch.int32, device="cuda"), dx, dB, ddt)
