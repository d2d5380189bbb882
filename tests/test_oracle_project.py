"""Pins of the oracle's input projections (oracle.project) against things other than
itself: one-hot weights that select known input columns (which output block comes from
which weight, and that a weight row is one output feature), row sums of integer weights,
brute force on a tiny case, linearity, and closed-form softplus values
(softplus(0) = ln 2, softplus(log(e^c - 1)) = c, softplus(z) - softplus(-z) = z).
Planted mistakes in a copy of the function must be caught by these checks."""
from __future__ import annotations

import inspect
import math
import textwrap

import numpy as np
import pytest

import oracle

H, P, G, N = 2, 4, 1, 8
D_MODEL = 16


def one_hot_rows(cols, d):
    w = np.zeros((len(cols), d))
    w[np.arange(len(cols)), cols] = 1.0
    return w


def check_one_hot_blocks(fn):
    rng = np.random.default_rng(21)
    u = rng.integers(-5, 6, size=(3, D_MODEL)).astype(np.float64)
    kx = rng.permutation(D_MODEL)[:H * P]
    kb = rng.permutation(D_MODEL)[:G * N]
    kc = rng.permutation(D_MODEL)[:G * N]
    kd = np.array([2, 9])
    x, B, C, dt = fn(u, one_hot_rows(kx, D_MODEL), one_hot_rows(kb, D_MODEL), one_hot_rows(kc, D_MODEL),
                     one_hot_rows(kd, D_MODEL))
    assert np.array_equal(x, u[:, kx])
    assert np.array_equal(B, u[:, kb])
    assert np.array_equal(C, u[:, kc])
    # the step size goes through softplus: checked at values with a closed form
    u2 = np.zeros((4, D_MODEL))
    cs = [1.0, 2.0, 3.0, 0.25]
    for t, c in enumerate(cs):
        u2[t, 2] = math.log(math.expm1(c))   # softplus of this is c
    u2[:, 9] = 0.0                            # softplus(0) = ln 2
    _, _, _, dt2 = fn(u2, one_hot_rows(kx, D_MODEL), one_hot_rows(kb, D_MODEL), one_hot_rows(kc, D_MODEL),
                      one_hot_rows(kd, D_MODEL))
    assert np.allclose(dt2[:, 0], cs, rtol=1e-14, atol=0)
    assert np.allclose(dt2[:, 1], math.log(2.0), rtol=1e-15, atol=0)


def check_row_sums(fn):
    # all-ones input: every output is the sum of its weight row (integers, so exact)
    rng = np.random.default_rng(22)
    w = [rng.integers(-3, 4, size=(r, D_MODEL)).astype(np.float64) for r in (H * P, G * N, G * N, H)]
    u = np.ones((2, D_MODEL))
    x, B, C, dt = fn(u, *w)
    for out, wi in ((x, w[0]), (B, w[1]), (C, w[2])):
        assert np.array_equal(out, np.tile(wi.sum(axis=1), (2, 1)))


def check_brute_force(fn):
    rng = np.random.default_rng(23)
    T = 3
    u = rng.normal(size=(T, D_MODEL))
    w = [rng.normal(size=(r, D_MODEL)) for r in (H * P, G * N, G * N, H)]
    bias = rng.normal(size=H)
    outs = fn(u, *w, dt_bias=bias)
    for i, (out, wi) in enumerate(zip(outs, w)):
        for t in range(T):
            for n in range(wi.shape[0]):
                acc = 0.0
                for k in range(D_MODEL):
                    acc += u[t, k] * wi[n, k]
                if i == 3:
                    acc = math.log1p(math.exp(acc + bias[n]))
                assert abs(out[t, n] - acc) <= 1e-12 * (1 + abs(acc)), (i, t, n)


def check_linearity(fn):
    rng = np.random.default_rng(24)
    u1, u2 = rng.normal(size=(2, 5, D_MODEL))
    w = [rng.normal(size=(r, D_MODEL)) for r in (H * P, G * N, G * N, H)]
    a, b = 0.75, -1.5
    o1, o2, o12 = fn(u1, *w), fn(u2, *w), fn(a * u1 + b * u2, *w)
    for i in range(3):
        assert np.allclose(o12[i], a * o1[i] + b * o2[i], rtol=1e-12, atol=1e-12)
    # the step size is softplus of a linear function: log(e^dt - 1) is linear in u (a
    # planted mistake may give step sizes that overflow here; the check then fails)
    with np.errstate(over="ignore", invalid="ignore"):
        z = [np.log(np.expm1(o[3])) for o in (o1, o2, o12)]
    assert np.allclose(z[2], a * z[0] + b * z[1], rtol=1e-9, atol=1e-9)


def check_softplus_and_bias(fn):
    w = [np.zeros((r, D_MODEL)) for r in (H * P, G * N, G * N, H)]
    u = np.ones((2, D_MODEL))
    # zero step-size weights: dt is softplus of the bias alone, per head
    cs = np.array([0.5, 4.0])
    _, _, _, dt = fn(u, *w, dt_bias=np.log(np.expm1(cs)))
    assert np.allclose(dt, np.tile(cs, (2, 1)), rtol=1e-14, atol=0)
    _, _, _, dt0 = fn(u, *w)
    assert np.allclose(dt0, math.log(2.0), rtol=1e-15, atol=0)
    # far tails: softplus(40) = 40 + e^-40, softplus(-40) = e^-40 (relative)
    _, _, _, dtt = fn(u, *w, dt_bias=np.array([40.0, -40.0]))
    assert abs(dtt[0, 0] - 40.0) <= 1e-14 * 40.0
    assert abs(dtt[0, 1] - math.exp(-40.0)) <= 1e-12 * math.exp(-40.0)
    # softplus(z) - softplus(-z) = z
    zs = np.array([-7.0, 0.3])
    _, _, _, dp = fn(u, *w, dt_bias=zs)
    _, _, _, dm = fn(u, *w, dt_bias=-zs)
    assert np.allclose(dp[0] - dm[0], zs, rtol=0, atol=1e-14)


CHECKS = [check_one_hot_blocks, check_row_sums, check_brute_force, check_linearity, check_softplus_and_bias]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_project_oracle_pin(check):
    check(oracle.project)


MUTANTS = [
    ("key and query projections swapped", "B = u @ np.asarray(w_B, dtype=np.float64).T",
     "B = u @ np.asarray(w_C, dtype=np.float64).T"),
    ("value rows taken as columns", "x = u @ np.asarray(w_x, dtype=np.float64).T",
     "x = (np.asarray(w_x, dtype=np.float64) @ u.T).T[:, ::-1]"),
    ("exp in place of softplus", "return x, B, C, softplus(z)", "return x, B, C, np.exp(z)"),
    ("bias added after softplus", "return x, B, C, softplus(z)",
     "return x, B, C, softplus(z - (0 if dt_bias is None else np.asarray(dt_bias)[None, :])) + "
     "(0 if dt_bias is None else np.asarray(dt_bias)[None, :])"),
    ("bias ignored", "z = z + np.asarray(dt_bias, dtype=np.float64)[None, :]", "z = z"),
    ("step-size sign flipped", "z = u @ np.asarray(w_dt, dtype=np.float64).T",
     "z = -(u @ np.asarray(w_dt, dtype=np.float64).T)"),
    ("last input column dropped", "u = np.asarray(u, dtype=np.float64)",
     "u = np.asarray(u, dtype=np.float64).copy(); u[:, -1] = 0"),
]


@pytest.mark.parametrize("i", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_project_planted_mistakes_are_caught(i):
    desc, old, new = MUTANTS[i]
    src = textwrap.dedent(inspect.getsource(oracle.project))
    assert src.count(old) == 1, desc
    ns = {"np": np, "softplus": oracle.softplus}
    exec(src.replace(old, new), ns)
    mutant = ns["project"]
    caught = 0
    for check in CHECKS:
        try:
            check(mutant)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, desc
