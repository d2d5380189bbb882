"""Pins for the CPU oracle, checked against things other than the oracle itself.

Each check cites what fixes the expected value:
  * hand-worked fixtures in tests/golden/ (the pages print no numbers, so these
    are worked from the layer's definition);
  * closed forms (causal linear attention at A = 0, dt = 1; a geometric series);
  * an independent brute force of the quadratic form (tests/brute.py);
  * a textbook library routine (a numpy matmul for the A = 0, dt = 1 case);
  * invariants the speculative protocol of the QbitAI article's walkthrough
    implies (roll-back to the last accepted token equals never having taken
    the rejected ones; no intermediate state needed).
`test_planted_mistakes_are_caught` rebuilds the oracle with one deliberate
error at a time and asserts that at least one of these checks fails.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from brute import causal_linear_attention_int, quadratic_form

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand_case(rng, Bt, T, H, P, N, G, a_lo=-3.0, a_hi=-0.1, with_h0=True):
    x = rng.normal(size=(Bt, T, H, P))
    B = rng.normal(size=(Bt, T, G, N))
    C = rng.normal(size=(Bt, T, G, N))
    dt = rng.uniform(0.05, 1.5, size=(Bt, T, H))
    A = rng.uniform(a_lo, a_hi, size=H)
    D = rng.normal(size=H)
    h0 = rng.normal(size=(Bt, H, N, P)) if with_h0 else None
    return x, B, C, dt, A, D, h0


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ----------------------------------------------------------------------------
# checks (each takes the oracle library so that planted-mistake builds reuse them)
# ----------------------------------------------------------------------------

def check_golden(lib):
    """Hand-worked fixtures (tests/golden/*.txt)."""
    files = sorted(glob.glob(os.path.join(HERE, "golden", "*.txt")))
    assert files
    for f in files:
        kv = {}
        for line in open(f):
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *vals = line.split()
            kv[k] = [float(v) for v in vals]
        T, H, G, P, N = (int(kv[k][0]) for k in ("T", "H", "G", "P", "N"))
        x = np.array(kv["x"]).reshape(1, T, H, P)
        B = np.array(kv["B"]).reshape(1, T, G, N)
        C = np.array(kv["C"]).reshape(1, T, G, N)
        dt = np.array(kv["dt"]).reshape(1, T, H)
        A = np.broadcast_to(np.array(kv["A"]), (H,)).copy()
        D = np.broadcast_to(np.array(kv["D"]), (H,)).copy()
        h0 = np.array(kv["h0"]).reshape(1, H, N, P)
        y, hT = oracle.prefill(x, B, C, dt, A, D, h0=h0, lib=lib)
        tol = kv["tol"][0]
        ey = np.array(kv["y"]).reshape(1, T, H, P)
        eh = np.array(kv["hT"]).reshape(1, H, N, P)
        assert np.max(np.abs(y - ey)) <= tol * max(1.0, np.max(np.abs(ey))), (f, y.ravel(), ey.ravel())
        assert np.max(np.abs(hT - eh)) <= tol * max(1.0, np.max(np.abs(eh))), (f, hT.ravel(), eh.ravel())


def check_p1_linear_attention_exact(lib):
    """P1: A = 0, dt = 1 reduces the layer to causal linear attention; with small
    integers every value is an exact double, so the match must be exact."""
    rng = np.random.default_rng(11)
    Bt, T, H, P, N, G = 2, 7, 4, 3, 5, 2
    x = rng.integers(-2, 3, size=(Bt, T, H, P)).astype(np.float64)
    B = rng.integers(-2, 3, size=(Bt, T, G, N)).astype(np.float64)
    C = rng.integers(-2, 3, size=(Bt, T, G, N)).astype(np.float64)
    D = rng.integers(-3, 4, size=H).astype(np.float64)
    D[D == 0] = 2.0
    dt = np.ones((Bt, T, H))
    A = np.zeros(H)
    y, hT = oracle.prefill(x, B, C, dt, A, D, lib=lib)
    ey, eh = causal_linear_attention_int(x, B, C, D)
    assert np.array_equal(y, np.array(ey, dtype=np.float64))
    assert np.array_equal(hT, np.array(eh, dtype=np.float64))


def check_p2_quadratic_form(lib):
    """P2: the unrolled (attention-like) form, written independently, on tiny shapes,
    with a non-zero starting state and G < H."""
    rng = np.random.default_rng(12)
    for (Bt, T, H, P, N, G) in [(1, 5, 2, 3, 4, 1), (2, 4, 4, 2, 3, 2), (1, 6, 3, 2, 2, 3)]:
        x, B, C, dt, A, D, h0 = _rand_case(rng, Bt, T, H, P, N, G)
        y, hT = oracle.prefill(x, B, C, dt, A, D, h0=h0, lib=lib)
        ey, eh = quadratic_form(x, B, C, dt, A, D, h0=h0)
        assert _rel(y, ey) < 1e-12
        assert _rel(hT, eh) < 1e-12


def check_p3_geometric_series(lib):
    """P3: N = P = 1 with constant decay a = exp(dt A) and constant input:
    h_t = a^t h_0 + dt B x (1 - a^t)/(1 - a), y_t = C h_t + D x."""
    T, dtv, Av, Bv, Cv, xv, Dv, h0v = 40, 0.37, -0.8, 1.3, -0.7, 0.9, 0.25, 2.0
    x = np.full((1, T, 1, 1), xv)
    B = np.full((1, T, 1, 1), Bv)
    C = np.full((1, T, 1, 1), Cv)
    dt = np.full((1, T, 1), dtv)
    y, hT = oracle.prefill(x, B, C, dt, np.array([Av]), np.array([Dv]),
                           h0=np.full((1, 1, 1, 1), h0v), lib=lib)
    a = np.exp(dtv * Av)
    t = np.arange(1, T + 1)
    h = a ** t * h0v + dtv * Bv * xv * (1 - a ** t) / (1 - a)
    assert _rel(y[0, :, 0, 0], Cv * h + Dv * xv) < 1e-13
    assert abs(hT[0, 0, 0, 0] - h[-1]) / abs(h[-1]) < 1e-13


def check_p4_rollback_equals_prefix(lib):
    """P4: verify K drafts then keep j is the same as never having seen the rejected
    drafts: the state equals a prefill of prefix + j drafts (bitwise: same loop,
    same order), and verify's y_k equals the prefill's y at position L + k."""
    rng = np.random.default_rng(14)
    Bt, L, K, H, P, N, G = 3, 9, 5, 4, 3, 4, 2
    x, B, C, dt, A, D, _ = _rand_case(rng, Bt, L + K, H, P, N, G, with_h0=False)
    pre = lambda a: np.ascontiguousarray(a[:, :L])
    drf = lambda a: np.ascontiguousarray(a[:, L:])
    _, hc = oracle.prefill(pre(x), pre(B), pre(C), pre(dt), A, D, lib=lib)
    yv = oracle.verify(hc, drf(x), drf(B), drf(C), drf(dt), A, D, lib=lib)
    yfull, _ = oracle.prefill(x, B, C, dt, A, D, lib=lib)
    assert np.array_equal(yv, yfull[:, L:])
    for j in range(K + 1):
        hj = oracle.commit(hc, drf(x), drf(B), drf(dt), A, D, [j] * Bt, lib=lib)
        cut = lambda a: np.ascontiguousarray(a[:, :L + j])
        _, ref = oracle.prefill(cut(x), cut(B), cut(C), cut(dt), A, D, lib=lib)
        assert np.array_equal(hj, ref), j
    # ragged accepted lengths per sequence
    jb = [0, K, 2]
    hj = oracle.commit(hc, drf(x), drf(B), drf(dt), A, D, jb, lib=lib)
    for b, j in enumerate(jb):
        sl = lambda a: np.ascontiguousarray(a[b:b + 1, :L + j])
        _, ref = oracle.prefill(sl(x), sl(B), sl(C), sl(dt), A, D, lib=lib)
        assert np.array_equal(hj[b:b + 1], ref)


def check_p5_split_invariance(lib):
    """P5: prefill(L1 + L2) equals prefill(L2) started from the state after L1."""
    rng = np.random.default_rng(15)
    x, B, C, dt, A, D, _ = _rand_case(rng, 2, 13, 2, 3, 4, 1, with_h0=False)
    y, h = oracle.prefill(x, B, C, dt, A, D, lib=lib)
    for L1 in (1, 6, 12):
        a = lambda v: np.ascontiguousarray(v[:, :L1])
        b = lambda v: np.ascontiguousarray(v[:, L1:])
        y1, h1 = oracle.prefill(a(x), a(B), a(C), a(dt), A, D, lib=lib)
        y2, h2 = oracle.prefill(b(x), b(B), b(C), b(dt), A, D, h0=h1, lib=lib)
        assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
        assert np.array_equal(h2, h)


def check_p6_special_cases(lib):
    """P6: x = 0 leaves only the decay, h_T = exp(A sum dt) h_0; dt = 0 leaves the state
    unchanged and y = C^T h_0 + D x; accepting j = 0 leaves the state bitwise."""
    rng = np.random.default_rng(16)
    Bt, T, H, P, N, G = 2, 6, 2, 3, 4, 2
    x, B, C, dt, A, D, h0 = _rand_case(rng, Bt, T, H, P, N, G)
    _, hT = oracle.prefill(np.zeros_like(x), B, C, dt, A, D, h0=h0, lib=lib)
    decay = np.exp(A[None, :] * dt.sum(axis=1))  # [Bt][H]
    assert _rel(hT, decay[:, :, None, None] * h0) < 1e-13
    y, hT = oracle.prefill(x, B, C, np.zeros_like(dt), A, D, h0=h0, lib=lib)
    assert np.array_equal(hT, h0)
    hpg = H // G
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            ey = C[b, :, g, :] @ h0[b, h] + D[h] * x[b, :, h, :]
            assert _rel(y[b, :, h, :], ey) < 1e-13
    h1 = oracle.commit(h0, x, B, dt, A, D, [0] * Bt, lib=lib)
    assert np.array_equal(h1, h0)


def check_p7_linearity(lib):
    """P7: outputs are linear in (x, h_0) jointly (dt, A, B, C, D fixed)."""
    rng = np.random.default_rng(17)
    x1, B, C, dt, A, D, h01 = _rand_case(rng, 1, 8, 2, 3, 3, 1)
    x2 = rng.normal(size=x1.shape)
    h02 = rng.normal(size=h01.shape)
    ya, ha = oracle.prefill(x1, B, C, dt, A, D, h0=h01, lib=lib)
    yb, hb = oracle.prefill(x2, B, C, dt, A, D, h0=h02, lib=lib)
    yc, hc = oracle.prefill(2.0 * x1 - 3.0 * x2, B, C, dt, A, D, h0=2.0 * h01 - 3.0 * h02, lib=lib)
    assert _rel(yc, 2.0 * ya - 3.0 * yb) < 1e-12
    assert _rel(hc, 2.0 * ha - 3.0 * hb) < 1e-12


def check_p8_gqa_equivalence(lib):
    """P8: G shared groups give the same result as G = H with B and C repeated per
    head in the contiguous order h -> h // (H/G)."""
    rng = np.random.default_rng(18)
    Bt, T, H, P, N, G = 2, 5, 6, 2, 3, 2
    x, B, C, dt, A, D, h0 = _rand_case(rng, Bt, T, H, P, N, G)
    y, hT = oracle.prefill(x, B, C, dt, A, D, h0=h0, lib=lib)
    Br = np.repeat(B, H // G, axis=2)
    Cr = np.repeat(C, H // G, axis=2)
    y2, h2 = oracle.prefill(x, Br, Cr, dt, A, D, h0=h0, lib=lib)
    assert np.array_equal(y, y2)
    assert np.array_equal(hT, h2)


def check_p9_matmul(lib):
    """P9: at A = 0, dt = 1 the prefill is Y = tril(C B^T) X + D X per head (numpy matmul)."""
    rng = np.random.default_rng(19)
    Bt, T, H, P, N, G = 2, 11, 4, 5, 6, 2
    x, B, C, _, _, D, _ = _rand_case(rng, Bt, T, H, P, N, G)
    y, _ = oracle.prefill(x, B, C, np.ones((Bt, T, H)), np.zeros(H), D, lib=lib)
    for b in range(Bt):
        for h in range(H):
            g = h // (H // G)
            M = np.tril(C[b, :, g, :] @ B[b, :, g, :].T)
            ey = M @ x[b, :, h, :] + D[h] * x[b, :, h, :]
            assert _rel(y[b, :, h, :], ey) < 1e-12


ALL_CHECKS = [check_golden, check_p1_linear_attention_exact, check_p2_quadratic_form,
              check_p3_geometric_series, check_p4_rollback_equals_prefix,
              check_p5_split_invariance, check_p6_special_cases, check_p7_linearity,
              check_p8_gqa_equivalence, check_p9_matmul]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check, oracle_lib):
    check(oracle_lib)


def test_threads_do_not_change_results(oracle_lib):
    rng = np.random.default_rng(20)
    x, B, C, dt, A, D, h0 = _rand_case(rng, 3, 7, 4, 3, 5, 2)
    y1, h1 = oracle.prefill(x, B, C, dt, A, D, h0=h0, nthreads=1, lib=oracle_lib)
    y8, h8 = oracle.prefill(x, B, C, dt, A, D, h0=h0, nthreads=8, lib=oracle_lib)
    assert np.array_equal(y1, y8) and np.array_equal(h1, h8)


def test_commit_rejects_out_of_range(oracle_lib):
    z = np.zeros((1, 2, 1, 1))
    with pytest.raises(ValueError):
        oracle.commit(np.zeros((1, 1, 1, 1)), z, z, np.zeros((1, 2, 1)), np.zeros(1), np.zeros(1), [3],
                      lib=oracle_lib)


# (description, exact text in ssm_oracle.c, replacement): one plausible mistake each
MUTANTS = [
    ("skip term D*x dropped", "y[p] = acc + D * x[p];", "y[p] = acc;"),
    ("decay exponent sign flipped", "exp(dt * A)", "exp(-dt * A)"),
    ("step size missing on B", "const double bn = dt * b[n];", "const double bn = b[n];"),
    ("step size missing in decay", "exp(dt * A)", "exp(A)"),
    ("decay applied after the input", "row[p] = abar * row[p] + bn * x[p];",
     "row[p] = abar * (row[p] + bn * x[p]);"),
    ("readout uses B instead of C", "acc += c[n] * h", "acc += b[n] * h"),
    ("state read transposed", "acc += c[n] * h[(size_t)n * P + p];",
     "acc += c[n] * h[(size_t)p * N + n];"),
    ("group map h % G", "g = h / heads_per_group", "g = h % j->G"),
    ("B taken from the previous token", "const double *bb = j->B + (bt * j->G + g) * j->N;",
     "const double *bb = j->B + ((t > 0 ? bt - 1 : bt) * j->G + g) * j->N;"),
    ("D of head 0 for every head", "j->D[h]", "j->D[0]"),
    ("readout before the update", "    if (!y)\n        return;\n    for (int p = 0; p < P; ++p) {\n        double acc",
     "    if (!y)\n        return;\n    for (int p = 0; p < P; ++p) {\n        double acc"),
]


def _build_mutant(tmp_path, i, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ssm_oracle.c")).read()
    assert src.count(old) >= 1, old
    if i == len(MUTANTS) - 1:
        # move the readout loop ahead of the update loop: y reads h_{t-1}
        upd_start = src.index("    for (int n = 0; n < N; ++n) {\n        const double bn")
        read_start = src.index("    if (!y)\n        return;")
        read_end = src.index("        y[p] = acc + D * x[p];\n    }\n") + len("        y[p] = acc + D * x[p];\n    }\n")
        upd = src[upd_start:read_start]
        read = src[read_start:read_end].replace("    if (!y)\n        return;\n", "    if (y)\n")
        src = src[:upd_start] + read + upd + src[read_end:]
    else:
        src = src.replace(old, new, 1)
    d = tmp_path / f"m{i}"
    d.mkdir()
    c = d / "ssm_oracle.c"
    c.write_text(src)
    return oracle.build(str(c), str(d / "libm.so"))


@pytest.mark.parametrize("i", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_planted_mistakes_are_caught(i, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc missing")
    desc, old, new = MUTANTS[i]
    lib = oracle.load(_build_mutant(tmp_path, i, old, new))
    failed = []
    for check in ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"planted mistake '{desc}' passed every pin"
