"""mil_ssm_commit_greedy_noalloc (the greedy commit without a workspace argument: its
partial maxima go to the library's own per-GPU scratch) against mil_ssm_commit_greedy on
twin caches, through the C ABI.  Two rounds in a row, the second with a smaller input
(fewer drafts, a smaller vocabulary), so that the scratch still holds the first call's
keys when the second runs: accepted lengths, argmax tokens, counters, the state and the
next round's outputs must be identical.  Sizes over the scratch's limit are refused
before anything is enqueued."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, dev_layer, dev_tokens
from speculative_decode_amd import _lib as L
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.lib()


def test_noalloc_greedy_commit_matches_workspace_form():
    rng = np.random.default_rng(4321)
    Bt, H, P, N, G, kmax = 32, 8, 64, 64, 2, 16
    layer = synth.draw_layer(rng, H)
    A, D = dev_layer(layer)
    pre = synth.draw_tokens(rng, Bt, 40, H, P, N, G, synth.BF16)
    caches = []
    for _ in range(2):  # [0] workspace form, [1] no-alloc form
        c = SSMCache(Bt, H, P, N, G, kmax, synth.BF16)
        c.prefill(*dev_tokens(pre), A, D)
        caches.append(c)
    for rnd, (K, vocab, ldt) in enumerate([(16, 128256, synth.BF16), (4, 5000, synth.F32)]):
        drf = synth.draw_tokens(rng, Bt, K, H, P, N, G, synth.BF16)
        planted = synth.draw_accept_uniform(rng, Bt, K)
        dtok, lg = synth.draw_greedy(rng, Bt, K, vocab, ldt, planted, ties=True)
        j_ref, tok_ref = oracle.greedy_accept(dtok, lg.f64)
        x, B, C, dt = dev_tokens(drf)
        lgd, dtd = dev(lg), torch.from_numpy(dtok).cuda()
        ys, outs = [], []
        for i, c in enumerate(caches):
            ys.append(c.verify(x, B, C, dt, A, D))
            acc, tok = c.commit_greedy(dtd, lgd, x, B, dt, A, D, want_tokens=True, noalloc=(i == 1),
                                       materialize=(rnd == 1))
            outs.append((acc, tok))
        torch.cuda.synchronize()
        assert torch.equal(ys[0], ys[1])
        for acc, tok in outs:
            assert np.array_equal(acc.cpu().numpy(), j_ref), rnd
            assert np.array_equal(tok.cpu().numpy(), tok_ref), rnd
        assert torch.equal(caches[0].pos(), caches[1].pos())
        assert torch.equal(caches[0].pending(), caches[1].pending())
        assert torch.equal(caches[0].state(), caches[1].state())
        assert caches[1].err().cpu().tolist() == [0] * Bt
    # the rounds after: same outputs from both caches
    nxt = synth.draw_tokens(rng, Bt, 4, H, P, N, G, synth.BF16)
    y0, y1 = (c.verify(*dev_tokens(nxt), A, D) for c in caches)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_noalloc_greedy_commit_refuses_sizes_over_its_scratch():
    rng = np.random.default_rng(99)
    Bt, H, P, N, G, K, vocab = 64, 2, 32, 32, 1, 16, 100   # 64 x 16 = 1024 rows > 512
    assert Bt * K > L.MIL_GREEDY_NOALLOC_MAX_ROWS
    layer = synth.draw_layer(rng, H)
    A, D = dev_layer(layer)
    c = SSMCache(Bt, H, P, N, G, K, synth.BF16)
    drf = synth.draw_tokens(rng, Bt, K, H, P, N, G, synth.BF16)
    x, B, C, dt = dev_tokens(drf)
    c.verify(x, B, C, dt, A, D)
    dtok = torch.zeros((Bt, K), dtype=torch.int32, device="cuda")
    logits = torch.zeros((Bt, K, vocab), dtype=torch.bfloat16, device="cuda")
    acc = torch.full((Bt,), -7, dtype=torch.int32, device="cuda")
    P_ = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.lib().mil_ssm_commit_greedy_noalloc(ctypes.byref(c.desc), K, P_(dtok), P_(logits), vocab, L.MIL_BF16,
                                               P_(acc), None, P_(x), P_(B), P_(dt), None, None, 0, None)
    assert st == L.MIL_E_WORKSPACE
    assert c.phase() == L.PHASE_VERIFIED
    torch.cuda.synchronize()
    assert acc.cpu().tolist() == [-7] * Bt
    # the same cache with fewer drafts fits
    c.commit(torch.zeros(Bt, dtype=torch.int32, device="cuda"), x, B, dt)
    x4, B4, C4, dt4 = (t[:, :4].contiguous() for t in (x, B, C, dt))
    c.verify(x4, B4, C4, dt4, A, D)
    acc2, _ = c.commit_greedy(dtok[:, :4].contiguous(), logits[:, :4].contiguous(), x4, B4, dt4, noalloc=True)
    torch.cuda.synchronize()
    assert acc2.cpu().tolist() == [4] * Bt  # all-zero logits: token 0 (the lowest id) everywhere
