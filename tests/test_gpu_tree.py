"""GPU parity of tree-draft verification (mil_ssm_verify_tree, mil_ssm_commit_tree)
against the oracle's verify_tree / commit_tree, and the bitwise properties the kernel is
built to keep: a chain tree is exactly the flat verify and commit, and a node's output is
bit-identical to a flat verify of its root path's tokens (so rolling back to any branch is
as exact as rolling back a chain).  Rounds run after a flat round whose accepted rows are
still pending, so the fold in front of the tree readout is exercised too."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import BOUND, dev, dev_layer, dev_tokens, state_err, y_err
from speculative_decode_amd import _lib as L
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.lib()  # a missing library is a failure, not a skip


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def bits(t):
    return t.detach().contiguous().view(torch.int32).cpu().numpy()


def start(rng, shape, dtype, k_max, ncache=1):
    """Caches with a prefilled context and one flat round whose accepted rows are pending;
    returns the oracle's logical state after them too."""
    Bt, H, P, N, G = shape
    layer = synth.draw_layer(rng, H)
    ctx = synth.draw_tokens(rng, Bt, 24, H, P, N, G, dtype)
    r1 = synth.draw_tokens(rng, Bt, 3, H, P, N, G, dtype)
    j1 = synth.draw_accept_uniform(rng, Bt, 3)
    A, D = dev_layer(layer)
    caches = []
    for _ in range(ncache):
        c = SSMCache(Bt, H, P, N, G, k_max, dtype)
        c.prefill(*dev_tokens(ctx), A, D, chunk=64)
        x1, B1, C1, dt1 = dev_tokens(r1)
        c.verify(x1, B1, C1, dt1, A, D)
        c.commit(i32(j1), x1, B1, dt1)
        caches.append(c)
    Af, Df = layer.A.f64, layer.D.f64
    _, h = oracle.prefill(ctx.x.f64, ctx.B.f64, ctx.C.f64, ctx.dt.f64, Af, Df)
    h = oracle.commit(h, r1.x.f64, r1.B.f64, r1.dt.f64, Af, Df, j1)
    return layer, (A, D), caches, h


CASES = [
    ((2, 2, 16, 16, 1), synth.F32, 5, "random"),
    ((3, 4, 32, 64, 2), synth.BF16, 8, "random"),
    ((4, 32, 128, 128, 8), synth.BF16, 8, "binary"),
    ((2, 32, 128, 128, 8), synth.BF16, 16, "random"),
    ((2, 32, 128, 256, 8), synth.BF16, 4, "fan"),
    ((3, 8, 64, 128, 4), synth.F32, 16, "random"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0][1]}h_P{c[0][2]}_N{c[0][3]}_{c[1]}_K{c[2]}_{c[3]}" for c in CASES])
def test_tree_matches_oracle(case):
    shape, dtype, K, kind = case
    Bt, H, P, N, G = shape
    rng = np.random.default_rng(5000 + K + N)
    print(f"tree {shape} {dtype} K={K} {kind}", flush=True)
    layer, (A, D), (c,), h = start(rng, shape, dtype, max(K, 4))
    par = synth.draw_tree(rng, Bt, K, kind)
    drafts = synth.draw_tokens(rng, Bt, K, H, P, N, G, dtype)
    dx, dB, dC, ddt = dev_tokens(drafts)
    y = c.verify_tree(i32(par), dx, dB, dC, ddt, A, D)
    Af, Df = layer.A.f64, layer.D.f64
    y_ref = oracle.verify_tree(h, drafts.x.f64, drafts.B.f64, drafts.C.f64, drafts.dt.f64, Af, Df, par)
    assert y_err(y.cpu().numpy(), y_ref) <= BOUND[dtype]
    node = rng.integers(-1, K, size=Bt).astype(np.int32)
    pos0 = c.pos().cpu().numpy().copy()
    c.commit_tree(i32(par), i32(node), dx, dB, ddt, A, D, materialize=True)
    h_ref, lens = oracle.commit_tree(h, drafts.x.f64, drafts.B.f64, drafts.dt.f64, Af, Df, par, node)
    torch.cuda.synchronize()
    assert state_err(c.state().cpu().numpy(), h_ref) <= BOUND[dtype]
    assert np.array_equal(c.pos().cpu().numpy(), pos0 + lens)
    assert np.array_equal(c.pending().cpu().numpy(), np.zeros(Bt))
    assert c.status() == -1


def test_chain_tree_is_the_flat_round():
    shape, dtype, K = (3, 32, 128, 128, 8), synth.BF16, 6
    Bt, H, P, N, G = shape
    rng = np.random.default_rng(5100)
    print("tree chain == flat", flush=True)
    layer, (A, D), (ct, cf), _ = start(rng, shape, dtype, 8, ncache=2)
    drafts = synth.draw_tokens(rng, Bt, K, H, P, N, G, dtype)
    dx, dB, dC, ddt = dev_tokens(drafts)
    par = synth.draw_tree(rng, Bt, K, "chain")
    yt = ct.verify_tree(i32(par), dx, dB, dC, ddt, A, D)
    yf = cf.verify(dx, dB, dC, ddt, A, D)
    assert np.array_equal(bits(yt), bits(yf))
    node = np.array([-1, 2, 5], dtype=np.int32)
    ct.commit_tree(i32(par), i32(node), dx, dB, ddt, A, D, materialize=True)
    cf.commit(i32(node + 1), dx, dB, ddt, A, D, materialize=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(ct.state()), bits(cf.state()))
    assert np.array_equal(ct.pos().cpu().numpy(), cf.pos().cpu().numpy())


def test_node_is_bit_identical_to_a_flat_verify_of_its_path():
    shape, dtype, K = (2, 32, 128, 128, 8), synth.BF16, 8
    Bt, H, P, N, G = shape
    rng = np.random.default_rng(5200)
    print("tree node == flat path", flush=True)
    layer, (A, D), caches, _ = start(rng, shape, dtype, 8, ncache=2)
    ct, cf = caches
    # one tree shape for every slot, so that a node's path has the same length in all of them
    par = np.tile(synth.draw_tree(rng, 1, K, "random"), (Bt, 1))
    drafts = synth.draw_tokens(rng, Bt, K, H, P, N, G, dtype)
    dx, dB, dC, ddt = dev_tokens(drafts)
    yt = bits(ct.verify_tree(i32(par), dx, dB, dC, ddt, A, D))
    paths = oracle.tree_paths(par)
    for k in range(K):
        idx = torch.tensor(paths[0][k], device="cuda")
        xs, Bs, Cs, ds = (t.index_select(1, idx).contiguous() for t in (dx, dB, dC, ddt))
        yf = bits(cf.verify(xs, Bs, Cs, ds, A, D))
        cf.commit(i32(np.zeros(Bt)), xs, Bs, ds)  # nothing accepted: the logical state stays
        assert np.array_equal(yf[:, -1], yt[:, k]), k
    ct.commit_tree(i32(par), i32(np.full(Bt, -1)), dx, dB, ddt)


def test_bad_node_and_links_are_reported():
    shape, dtype, K = (3, 4, 32, 64, 2), synth.BF16, 4
    Bt, H, P, N, G = shape
    rng = np.random.default_rng(5300)
    print("tree errors", flush=True)
    layer, (A, D), (c,), _ = start(rng, shape, dtype, 4)
    drafts = synth.draw_tokens(rng, Bt, K, H, P, N, G, dtype)
    dx, dB, dC, ddt = dev_tokens(drafts)
    par = synth.draw_tree(rng, Bt, K, "binary")
    c.verify_tree(i32(par), dx, dB, dC, ddt, A, D)
    pos0 = c.pos().cpu().numpy().copy()
    node = np.array([K, 1, -2], dtype=np.int32)   # out of range, fine, out of range
    c.commit_tree(i32(par), i32(node), dx, dB, ddt)
    torch.cuda.synchronize()
    err = c.err().cpu().numpy()
    assert err[0] == L.MIL_DEVERR_ACCEPT and err[1] == 0 and err[2] == L.MIL_DEVERR_ACCEPT
    pos = c.pos().cpu().numpy()
    assert pos[0] == pos0[0] and pos[2] == pos0[2] and pos[1] == pos0[1] + 2
    assert c.status(clear=True) == 0
    # a link that is not to an earlier node is reported by both calls
    bad = par.copy()
    bad[1, 3] = 3
    c.verify_tree(i32(bad), dx, dB, dC, ddt, A, D)
    torch.cuda.synchronize()
    assert c.err().cpu().numpy().tolist() == [0, L.MIL_DEVERR_TREE, 0]
    c.status(clear=True)
    c.commit_tree(i32(bad), i32(np.array([3, 3, 0])), dx, dB, ddt)
    torch.cuda.synchronize()
    assert c.err().cpu().numpy().tolist() == [0, L.MIL_DEVERR_TREE, 0]
    assert c.pending().cpu().numpy().tolist()[1] == 0
