"""Pins of the oracle's greedy acceptance (oracle.greedy_accept) against things other than
itself: an explicit scan on small inputs full of ties, and planted structures whose
answer is known by construction.  Planted mistakes in a copy of the function must be
caught by these checks."""
from __future__ import annotations

import inspect
import textwrap

import numpy as np
import pytest

import oracle
from speculative_decode_amd import synth


def scan_argmax(row):
    """Brute force: walk the row, keep the first index of the largest value."""
    best, bi = row[0], 0
    for i in range(1, len(row)):
        if row[i] > best:
            best, bi = row[i], i
    return bi


def check_brute_force(fn):
    rng = np.random.default_rng(11)
    for trial in range(40):
        batch, K, V = rng.integers(1, 4), rng.integers(1, 6), rng.integers(1, 9)
        logits = rng.integers(-2, 3, size=(batch, K, V)).astype(np.float64)  # many ties
        tokens = np.array([[scan_argmax(logits[b, k]) for k in range(K)] for b in range(batch)])
        drafts = np.where(rng.random((batch, K)) < 0.7, tokens, rng.integers(0, V, size=(batch, K)))
        j, t = fn(drafts, logits)
        assert np.array_equal(t, tokens), trial
        for b in range(batch):
            lead = 0
            while lead < K and drafts[b, lead] == tokens[b, lead]:
                lead += 1
            assert j[b] == lead, (trial, b)


def check_planted(fn):
    rng = np.random.default_rng(12)
    for dtype in (synth.F32, synth.BF16):
        for K in (1, 4, 8):
            planted = rng.integers(0, K + 1, size=7).astype(np.int32)
            planted[0], planted[1] = 0, K  # first draft rejected; every draft accepted
            drafts, lg = synth.draw_greedy(rng, 7, K, 300, dtype, planted)
            j, t = fn(drafts, lg.f64)
            assert np.array_equal(j, planted), (dtype, K)
            for b in range(7):
                assert np.array_equal(t[b, :planted[b]], drafts[b, :planted[b]])


def check_ties_lowest_index(fn):
    # two equal maxima: the lower id wins, whichever side the draft is on
    logits = np.zeros((2, 1, 10))
    logits[:, 0, [3, 7]] = 5.0
    j, t = fn(np.array([[3], [7]]), logits)
    assert t.tolist() == [[3], [3]] and j.tolist() == [1, 0]


def check_signed_zero_and_nan(fn):
    """Hand-worked rows for the two cases numbers alone leave open (the rule stated in
    oracle.greedy_accept): -0 and +0 are one value, so the lower id wins; every NaN,
    whatever its sign, ranks above every number, and the first NaN wins."""
    nan, inf = float("nan"), float("inf")
    rows = [
        ([-1.0, -0.0, 0.0, -2.0], 1),       # -0 at id 1 ties +0 at id 2
        ([0.0, -0.0], 0),
        ([-0.0, 0.0], 0),
        ([-3.0, -0.0, -0.0, 0.0], 1),
        ([1.0, -nan, nan, 5.0], 1),         # a negative NaN is a NaN too
        ([5.0, inf, nan], 2),               # NaN above +inf
        ([nan, inf], 0),
        ([-inf, -inf, -inf], 0),
        ([nan, nan, nan], 0),
        ([2.0, 7.0, -nan], 2),
    ]
    for vals, want in rows:
        lg = np.array(vals, dtype=np.float64).reshape(1, 1, -1)
        j, t = fn(np.array([[want]]), lg)
        assert t.tolist() == [[want]], (vals, t)
        assert j.tolist() == [1]
        j, t = fn(np.array([[want + 1]]), lg)
        assert j.tolist() == [0]


CHECKS = [check_brute_force, check_planted, check_ties_lowest_index, check_signed_zero_and_nan]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_greedy_oracle_pin(check):
    check(oracle.greedy_accept)


# (description, [(text in the oracle, replacement), ...])
MUTANTS = [
    ("ties go to the highest id", [("np.flatnonzero(row == np.max(row))[0]", "np.flatnonzero(row == np.max(row))[-1]")]),
    ("every match counted, not the leading run",
     [("        while j < K and drafts[b, j] == tokens[b, j]:\n            j += 1",
       "        j = int(np.sum(drafts[b] == tokens[b]))")]),
    ("last draft never accepted", [("while j < K and drafts", "while j < K - 1 and drafts")]),
    ("draft compared with the next position", [("drafts[b, j] == tokens[b, j]",
                                                "drafts[b, j] == tokens[b, min(j + 1, K - 1)]")]),
    ("argmin instead of argmax", [("np.max(row)", "np.min(row)")]),
    ("NaN ignored", [("if nan.size:", "if False:"), ("np.max(row)", "np.nanmax(row)")]),
    ("last NaN wins", [("tokens[b, k] = nan[0]", "tokens[b, k] = nan[-1]")]),
    ("-0 ranked below +0 (sign bit read as part of the value)",
     [("np.flatnonzero(row == np.max(row))[0]",
       "np.argmax(np.where(row == 0, np.copysign(1e-300, row), row))")]),
    ("a NaN with the sign bit set ranked below every number",
     [("nan = np.flatnonzero(np.isnan(row))", "nan = np.flatnonzero(np.isnan(row) & ~np.signbit(row))"),
      ("np.max(row)", "np.max(np.where(np.isnan(row), -np.inf, row))")]),
]


@pytest.mark.parametrize("i", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_greedy_planted_mistakes_are_caught(i):
    desc, edits = MUTANTS[i]
    src = textwrap.dedent(inspect.getsource(oracle.greedy_accept))
    for old, new in edits:
        assert src.count(old) >= 1, desc
        src = src.replace(old, new)
    ns = {"np": np}
    exec(src, ns)
    mutant = ns["greedy_accept"]
    caught = 0
    for check in CHECKS:
        try:
            check(mutant)
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught > 0, desc
