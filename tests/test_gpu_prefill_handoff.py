"""The single-launch prefill's chunk-to-chunk handoff where its flags could be stale: a
prefill captured once in a HIP graph and replayed with new inputs, and prefills on an
attached byte copy of a cache whose handoff rows already hold flags from earlier calls.

Each handoff row keeps, beside its chunk flags, the epoch its last call raised them to;
a call waits for epoch + 1, so flags left by earlier calls, by earlier replays of the same
graph or by the prefills that wrote a copied buffer never pass for this call's.  Every
replay and every call on the copy is checked against the oracle; the layer's decays are
A = 0 and A = -1e-3, so the state a chunk receives matters to every later chunk."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import BOUND, dev_layer, dev_tokens, state_err, y_err
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache

pytestmark = pytest.mark.gpu

SCAN_BIT = 1 << 8  # MIL_TRACE_PREFILL_SCAN: the one-launch prefill
SHAPE = (2, 8, 128, 128, 2)  # batch, H, P, N, G
L_TOK = 1024                 # four chunks of 256


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from speculative_decode_amd import _lib
    _lib.lib()


def slow_layer(rng, H):
    """D as drawn; A = 0 on even heads and -1e-3 on odd ones (long memory)."""
    layer = synth.draw_layer(rng, H)
    A = np.where(np.arange(H) % 2 == 0, 0.0, -1e-3)
    return synth.Layer(synth.quantize(A, synth.F32), layer.D)


def stored_state(cache):
    torch.cuda.synchronize()
    assert int(cache.pending().max().item()) == 0
    return cache.state().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("cont", [False, True], ids=["fresh", "continue"])
def test_graph_replayed_prefill_matches_oracle(cont):
    rng = np.random.default_rng(515 + cont)
    Bt, H, P, N, G = SHAPE
    layer = slow_layer(rng, H)
    A, D = dev_layer(layer)
    cache = SSMCache(Bt, H, P, N, G, 4, synth.BF16)
    assert cache.prefill_kernels(Bt, L_TOK) == SCAN_BIT
    ref_state = np.zeros((Bt, H, N, P))
    pos = 0
    if cont:  # a context to continue from, prefilled eagerly
        pre = synth.draw_tokens(rng, Bt, 300, H, P, N, G, synth.BF16)
        cache.prefill(*dev_tokens(pre), A, D)
        _, ref_state = oracle.prefill(pre.x.f64, pre.B.f64, pre.C.f64, pre.dt.f64, layer.A.f64, layer.D.f64)
        pos = 300
    x = torch.empty((Bt, L_TOK, H, P), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((Bt, L_TOK, G, N), dtype=torch.bfloat16, device="cuda")
    C = torch.empty_like(B)
    dt = torch.empty((Bt, L_TOK, H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((Bt, L_TOK, H, P), dtype=torch.float32, device="cuda")
    ws = torch.empty(cache.workspace_bytes(Bt, L_TOK) + 256, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        cache.prefill(x, B, C, dt, A, D, y=y, ws=ws, cont=cont)
    torch.cuda.synchronize()
    for rnd in range(4):
        tok = synth.draw_tokens(rng, Bt, L_TOK, H, P, N, G, synth.BF16)
        for dst, src in zip((x, B, C, dt), dev_tokens(tok)):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ry, rs = oracle.prefill(tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, layer.A.f64, layer.D.f64,
                                h0=ref_state if cont else None)
        ey = y_err(y.cpu().numpy(), ry)
        es = state_err(stored_state(cache), rs)
        assert ey <= BOUND[synth.BF16] and es <= BOUND[synth.BF16], (rnd, ey, es)
        pos = pos + L_TOK if cont else L_TOK
        assert cache.pos().cpu().tolist() == [pos] * Bt
        assert cache.err().cpu().tolist() == [0] * Bt
        if cont:
            ref_state = rs
    # four calls of one row: its epoch moved by one per replay (plus the eager prefill)
    epochs = cache.scan_words().cpu().numpy()[..., SSMCache.SCAN_EPOCH]
    assert epochs.any() and np.all(epochs[epochs != 0] == 4 + cont)


def test_prefill_on_attached_copy_with_flags_from_earlier_calls():
    """A cache that has run prefills is copied byte for byte to another buffer and
    attached: the copy's flags already hold the values of those calls.  Prefills on the copy
    (fresh and continuing) must match the oracle.  Then the same with the copy's rows set
    to values by hand before a call: flags of epochs 1..8 under epoch 8 (a buffer whose
    launches used other chunk counts), and every flag and epoch at 1000 (a buffer written
    by a process that had run 1000 prefills)."""
    rng = np.random.default_rng(616)
    Bt, H, P, N, G = SHAPE
    layer = slow_layer(rng, H)
    A, D = dev_layer(layer)
    src = SSMCache(Bt, H, P, N, G, 4, synth.BF16)
    for _ in range(3):
        tok = synth.draw_tokens(rng, Bt, L_TOK, H, P, N, G, synth.BF16)
        src.prefill(*dev_tokens(tok), A, D)
    _, ref_state = oracle.prefill(tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, layer.A.f64, layer.D.f64)
    raw = torch.empty(src.layout.bytes + 256, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    torch.cuda.synchronize()
    raw[off:off + src.layout.bytes].copy_(src.buffer)
    copy = SSMCache(Bt, H, P, N, G, 4, synth.BF16, attach_to=raw[off:])
    assert copy.prefill_kernels(Bt, L_TOK) == SCAN_BIT
    torch.cuda.synchronize()
    assert np.array_equal(copy.scan_words().cpu().numpy(), src.scan_words().cpu().numpy())
    epochs = copy.scan_words().cpu().numpy()[..., SSMCache.SCAN_EPOCH]
    assert epochs.any() and np.all(epochs[epochs != 0] == 3)
    pos = L_TOK
    for rnd, (preset, cont) in enumerate([(False, True), (False, False), (True, True), (True, False)]):
        if preset:  # flags of epochs 1..8 under epoch 8, then every flag and epoch at 1000
            words = copy.scan_words()
            E = SSMCache.SCAN_EPOCH
            if cont:
                ep = torch.arange(E, dtype=torch.int32, device="cuda") % 8 + 1
                words[:, :, :, :E] = ep * 4 + 2  # (epoch << 2) | inclusive
                words[:, :, :, E] = 8
            else:
                words[:, :, :, :E] = 1000 * 4 + 2
                words[:, :, :, E] = 1000
        tok = synth.draw_tokens(rng, Bt, L_TOK, H, P, N, G, synth.BF16)
        y = copy.prefill(*dev_tokens(tok), A, D, cont=cont)
        ry, rs = oracle.prefill(tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, layer.A.f64, layer.D.f64,
                                h0=ref_state if cont else None)
        torch.cuda.synchronize()
        ey, es = y_err(y.cpu().numpy(), ry), state_err(stored_state(copy), rs)
        assert ey <= BOUND[synth.BF16] and es <= BOUND[synth.BF16], (rnd, ey, es)
        pos = pos + L_TOK if cont else L_TOK
        assert copy.pos().cpu().tolist() == [pos] * Bt
        assert copy.err().cpu().tolist() == [0] * Bt
        ref_state = rs
