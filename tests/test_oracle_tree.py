"""Pins of the oracle's tree-draft verify and commit (oracle.verify_tree, commit_tree)
against things other than themselves: the independent brute-force quadratic form run on
each node's root path (tests/brute.py), the one-step closed form when every node hangs off
the committed state, and the chain special case, which must reduce to the flat verify and
commit.  Planted mistakes in copies of the functions must be caught by these checks."""
from __future__ import annotations

import inspect
import math
import textwrap

import numpy as np
import pytest

import oracle
from brute import quadratic_form
from speculative_decode_amd import synth

SHAPE = (2, 4, 2, 3, 2)  # batch, H, P, N, G (tiny: the brute force is pure Python)


def random_parents(rng, batch, K):
    par = np.zeros((batch, K), dtype=np.int32)
    for b in range(batch):
        for k in range(K):
            par[b, k] = rng.integers(-1, k)  # -1..k-1
    return par


def setup(seed, K, parent=None):
    rng = np.random.default_rng(seed)
    Bt, H, P, N, G = SHAPE
    layer = synth.draw_layer(rng, H)
    h0 = rng.normal(size=(Bt, H, N, P))
    tok = synth.draw_tokens(rng, Bt, K, H, P, N, G, synth.F32)
    par = random_parents(rng, Bt, K) if parent is None else np.array(parent, dtype=np.int32)
    return layer, h0, tok, par


def root_path(par_row, k):
    """Walk up the parent links (the reverse of how the oracle builds paths)."""
    out = []
    while k >= 0:
        out.append(k)
        k = int(par_row[k])
    return out[::-1]


def check_brute_force_paths(vt, ct):
    for seed in range(3):
        layer, h0, tok, par = setup(40 + seed, 6)
        A, D = layer.A.f64, layer.D.f64
        y = vt(h0, tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, A, D, par)
        for b in range(SHAPE[0]):
            for k in range(6):
                idx = root_path(par[b], k)
                yb, _ = quadratic_form(tok.x.f64[b:b + 1, idx], tok.B.f64[b:b + 1, idx], tok.C.f64[b:b + 1, idx],
                                       tok.dt.f64[b:b + 1, idx], A, D, h0[b:b + 1])
                assert np.allclose(y[b, k], yb[0, -1], rtol=1e-11, atol=1e-12), (seed, b, k)
        acc = np.array([3, 5])
        hs, lens = ct(h0, tok.x.f64, tok.B.f64, tok.dt.f64, A, D, par, acc)
        for b in range(SHAPE[0]):
            idx = root_path(par[b], int(acc[b]))
            assert lens[b] == len(idx)
            _, hb = quadratic_form(tok.x.f64[b:b + 1, idx], tok.B.f64[b:b + 1, idx], tok.C.f64[b:b + 1, idx],
                                   tok.dt.f64[b:b + 1, idx], A, D, h0[b:b + 1])
            assert np.allclose(hs[b], hb[0], rtol=1e-11, atol=1e-12), (seed, b)


def check_all_branches_from_the_state(vt, ct):
    # every node follows the committed state: one step each, closed form
    K = 5
    layer, h0, tok, par = setup(50, K, parent=np.full((SHAPE[0], K), -1))
    A, D = layer.A.f64, layer.D.f64
    y = vt(h0, tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, A, D, par)
    Bt, H, P, N, G = SHAPE
    for b in range(Bt):
        for k in range(K):
            for h in range(H):
                g = h // (H // G)
                dtv = tok.dt.f64[b, k, h]
                h1 = math.exp(dtv * A[h]) * h0[b, h] + dtv * np.outer(tok.B.f64[b, k, g], tok.x.f64[b, k, h])
                want = tok.C.f64[b, k, g] @ h1 + D[h] * tok.x.f64[b, k, h]
                assert np.allclose(y[b, k, h], want, rtol=1e-13, atol=1e-14), (b, k, h)
    hs, lens = ct(h0, tok.x.f64, tok.B.f64, tok.dt.f64, A, D, par, np.array([-1, 2]))
    assert np.array_equal(hs[0], h0[0]) and lens.tolist() == [0, 1]


def check_chain_is_the_flat_path(vt, ct):
    K = 6
    Bt = SHAPE[0]
    layer, h0, tok, par = setup(60, K, parent=np.tile(np.arange(-1, K - 1), (Bt, 1)))
    A, D = layer.A.f64, layer.D.f64
    y = vt(h0, tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, A, D, par)
    yf = oracle.verify(h0, tok.x.f64, tok.B.f64, tok.C.f64, tok.dt.f64, A, D)
    assert np.array_equal(y, yf)
    acc = np.array([2, 5])
    hs, lens = ct(h0, tok.x.f64, tok.B.f64, tok.dt.f64, A, D, par, acc)
    hf = oracle.commit(h0, tok.x.f64, tok.B.f64, tok.dt.f64, A, D, acc + 1)
    assert np.array_equal(hs, hf) and lens.tolist() == (acc + 1).tolist()


CHECKS = [check_brute_force_paths, check_all_branches_from_the_state, check_chain_is_the_flat_path]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_tree_oracle_pin(check, oracle_lib):
    check(oracle.verify_tree, oracle.commit_tree)


def test_tree_parents_are_checked():
    with pytest.raises(ValueError):
        oracle.tree_paths(np.array([[0, -1]]))   # a node cannot be its own parent
    with pytest.raises(ValueError):
        oracle.tree_paths(np.array([[-1, 2, 0]]))  # parents come before children
    with pytest.raises(ValueError):
        oracle.commit_tree(np.zeros((1, 1, 1, 1)), np.zeros((1, 2, 1, 1)), np.zeros((1, 2, 1, 1)),
                           np.zeros((1, 2, 1)), np.zeros(1), np.zeros(1), np.array([[-1, 0]]), np.array([2]))


MUTANTS = [
    ("path taken leaf-first", "tree_paths",
     "row.append((row[p] if p >= 0 else []) + [k])", "row.append([k] + (row[p] if p >= 0 else []))"),
    ("every earlier node on the path", "tree_paths",
     "row.append((row[p] if p >= 0 else []) + [k])", "row.append(list(range(k + 1)))"),
    ("grandparent link", "tree_paths",
     "row.append((row[p] if p >= 0 else []) + [k])",
     "row.append((row[int(par[b, p])] if p >= 0 and int(par[b, p]) >= 0 else []) + [k])"),
    ("accepted node itself left out", "commit_tree",
     "idx = paths[b][int(acc[b])]", "idx = paths[b][int(acc[b])][:-1]"),
    ("first nodes by index instead of the path", "commit_tree",
     "idx = paths[b][int(acc[b])]", "idx = list(range(len(paths[b][int(acc[b])])))"),
]


@pytest.mark.parametrize("i", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_tree_planted_mistakes_are_caught(i, oracle_lib):
    desc, fname, old, new = MUTANTS[i]
    ns = {"np": np, "verify": oracle.verify, "scan": oracle.scan, "tree_paths": oracle.tree_paths}
    for name in ("tree_paths", "verify_tree", "commit_tree"):
        src = textwrap.dedent(inspect.getsource(getattr(oracle, name)))
        if name == fname:
            assert src.count(old) == 1, desc
            src = src.replace(old, new)
        exec(src, ns)
    caught = 0
    for check in CHECKS:
        try:
            check(ns["verify_tree"], ns["commit_tree"])
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, desc
