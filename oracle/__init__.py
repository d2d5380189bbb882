"""CPU oracle for the SSM layer -- TEST INFRASTRUCTURE ONLY.

A double-precision reference for the recurrence of the Mamba layer that "The
Mamba in the Llama" distils from attention, and for the speculative verify /
roll-back protocol of the QbitAI article's speculative-decoding walkthrough.
Only `tests/`, `__graft_entry__.smoke()` and the bench's `cpu_baseline` leg
may import this package.  It shares no code with the GPU library.

Besides the recurrence (`scan`, `prefill`, `verify`, `commit`) it holds the two steps
on either side of it, the input projections (`project`) and greedy acceptance
(`greedy_accept`), and the tree-draft forms of verify and commit (`verify_tree`,
`commit_tree`).

All arrays are float64 numpy arrays in the token-row layouts
  x [batch][T][H][P], B and C [batch][T][G][N], dt [batch][T][H], A and D [H],
  state [batch][H][N][P], y [batch][T][H][P].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "libssm_oracle.so")
# no contraction, no fast math: the loops run exactly as written
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99"]


def build(src: str = _SRC, out: str = _LIB, extra: list[str] | None = None) -> str:
    cmd = ["gcc", *CFLAGS, *(extra or []), "-o", out, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str | None = None):
    """Load (building first if needed) the oracle library; `path` loads a specific build."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.ssm_oracle_scan.argtypes = [ctypes.c_int] * 6 + [dp] * 6 + [ip, dp, dp, ctypes.c_int]
    lib.ssm_oracle_scan.restype = ctypes.c_int
    return lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _dptr(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def scan(x, B, C, dt, A, D, state, ntok=None, want_y=True, nthreads=None, lib=None):
    """Advance `state` in place over tokens [0, ntok[b]) of each sequence; return y or None."""
    lib = lib or load()
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert B.shape == (Bt, T, G, N) and dt.shape == (Bt, T, H)
    assert state.shape == (Bt, H, N, P)
    x, B, dt = (np.ascontiguousarray(v, dtype=np.float64) for v in (x, B, dt))
    C = None if C is None else np.ascontiguousarray(C, dtype=np.float64)
    A = np.ascontiguousarray(A, dtype=np.float64)
    D = np.ascontiguousarray(D, dtype=np.float64)
    y = np.zeros((Bt, T, H, P)) if want_y else None
    nt = None
    if ntok is not None:
        nt = np.ascontiguousarray(np.broadcast_to(np.asarray(ntok, dtype=np.int32), (Bt,)))
    rc = lib.ssm_oracle_scan(Bt, T, H, P, N, G, _dptr(x), _dptr(B), _dptr(C), _dptr(dt),
                             _dptr(A), _dptr(D),
                             None if nt is None else nt.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
                             _dptr(state), _dptr(y), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return y


def prefill(x, B, C, dt, A, D, h0=None, nthreads=None, lib=None):
    """Full-sequence scan from zeros (or from h0): returns (y, final state)."""
    Bt, T, H, P = x.shape
    N = B.shape[3]
    state = np.zeros((Bt, H, N, P)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)
    y = scan(x, B, C, dt, A, D, state, nthreads=nthreads, lib=lib)
    return y, state


def verify(state, x, B, C, dt, A, D, nthreads=None, lib=None):
    """y for K draft tokens from the committed state; the state is left as it was."""
    work = np.array(state, dtype=np.float64, copy=True)
    return scan(x, B, C, dt, A, D, work, nthreads=nthreads, lib=lib)


def commit(state, x, B, dt, A, D, accepted, nthreads=None, lib=None):
    """State after the first accepted[b] draft tokens of each sequence (a new array)."""
    K = x.shape[1]
    acc = np.asarray(accepted, dtype=np.int32)
    if np.any(acc < 0) or np.any(acc > K):
        raise ValueError("accepted length outside 0..K")
    out = np.array(state, dtype=np.float64, copy=True)
    scan(x, B, None, dt, A, D, out, ntok=acc, want_y=False, nthreads=nthreads, lib=lib)
    return out


def greedy_accept(draft_tokens, logits):
    """Greedy acceptance (the QbitAI walkthrough's keep-until-the-first-rejection, with a
    draft taken as correct when it is the verifier's most likely token at its position).

    draft_tokens [batch][K] int, logits [batch][K][vocab] (the exact values the GPU gets,
    widened to float64).  Returns (accepted [batch] int32, verifier_tokens [batch][K]
    int32): the argmax token of every position and the number of leading positions whose
    draft equals it.

    The argmax rule (the pages fix none; this is the reading the GPU kernel follows too):
      * the largest value wins, and among equal values the lowest token id;
      * +0 and -0 are the same value (they compare equal);
      * a NaN, of either sign and any payload, counts as larger than every number, and
        among NaNs the lowest token id wins.
    """
    drafts = np.asarray(draft_tokens)
    lg = np.asarray(logits, dtype=np.float64)
    batch, K = drafts.shape
    tokens = np.zeros((batch, K), dtype=np.int32)
    for b in range(batch):
        for k in range(K):
            row = lg[b, k]
            nan = np.flatnonzero(np.isnan(row))
            if nan.size:
                tokens[b, k] = nan[0]
                continue
            # equal maxima (including -0 and +0) all satisfy row == max; take the first
            tokens[b, k] = np.flatnonzero(row == np.max(row))[0]
    accepted = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        j = 0
        while j < K and drafts[b, j] == tokens[b, j]:
            j += 1
        accepted[b] = j
    return accepted, tokens


def softplus(z):
    """log(1 + e^z) in float64 (numpy's logaddexp, which neither overflows for large z
    nor loses the tail for very negative z)."""
    return np.logaddexp(0.0, np.asarray(z, dtype=np.float64))


def project(u, w_x, w_B, w_C, w_dt, dt_bias=None):
    """The layer's per-token inputs from its input rows (the step before the recurrence).

    "The Mamba in the Llama" builds the layer from an attention layer's own linear
    projection weights (arXiv abstract, as on the chatpaper.ai and pith.science pages;
    skycaiji.com summary, method paragraph: the modified Mamba is initialised from the
    attention module).  Reading used here: x comes from the value projection, B from the
    key projection, C from the query projection, and the step size from one more
    projection per head through softplus (plus an optional per-head bias), so that dt > 0.

    u [T][d]; w_x [H*P][d]; w_B, w_C [G*N][d]; w_dt [H][d]; dt_bias [H] or None; every
    weight row is one output feature.  Returns float64 (x [T][H*P], B [T][G*N],
    C [T][G*N], dt [T][H]) before any rounding to a storage type.
    """
    u = np.asarray(u, dtype=np.float64)
    x = u @ np.asarray(w_x, dtype=np.float64).T
    B = u @ np.asarray(w_B, dtype=np.float64).T
    C = u @ np.asarray(w_C, dtype=np.float64).T
    z = u @ np.asarray(w_dt, dtype=np.float64).T
    if dt_bias is not None:
        z = z + np.asarray(dt_bias, dtype=np.float64)[None, :]
    return x, B, C, softplus(z)


def tree_paths(parent):
    """Root-first node list of every node of every sequence's draft tree.

    Tree drafts (the pages name tree-organised candidates among speculative decoding
    variants; skycaiji.com summary, related-work paragraph): K candidate tokens per
    sequence, node k following node parent[b][k] (-1: the committed state itself), with
    parents numbered before their children.  A node's path is the chain of tokens from the
    committed state to it, which is what the recurrence must run through for that node.
    """
    par = np.asarray(parent)
    batch, K = par.shape
    paths = []
    for b in range(batch):
        row = []
        for k in range(K):
            p = int(par[b, k])
            if p < -1 or p >= k:
                raise ValueError("parent[b][k] must lie in -1..k-1")
            row.append((row[p] if p >= 0 else []) + [k])
        paths.append(row)
    return paths


def verify_tree(state, x, B, C, dt, A, D, parent, nthreads=None, lib=None):
    """y[b][k] for every node of a draft tree: the plain recurrence run from a copy of the
    committed state along node k's root path, read out at node k.  The state is left as
    it was (every branch starts from the same cached state)."""
    paths = tree_paths(parent)
    batch, K = np.asarray(parent).shape
    H, P = x.shape[2], x.shape[3]
    y = np.zeros((batch, K, H, P))
    for b in range(batch):
        for k in range(K):
            idx = paths[b][k]
            yk = verify(state[b:b + 1], x[b:b + 1, idx], B[b:b + 1, idx], C[b:b + 1, idx], dt[b:b + 1, idx], A, D,
                        nthreads=nthreads, lib=lib)
            y[b, k] = yk[0, -1]
    return y


def commit_tree(state, x, B, dt, A, D, parent, accepted_node, nthreads=None, lib=None):
    """State after the accepted branch: the tokens on the root path of accepted_node[b]
    (-1: none accepted, state unchanged), in root-first order.  Returns (new state,
    accepted path lengths)."""
    paths = tree_paths(parent)
    batch, K = np.asarray(parent).shape
    acc = np.asarray(accepted_node, dtype=np.int64)
    if np.any(acc < -1) or np.any(acc >= K):
        raise ValueError("accepted node outside -1..K-1")
    out = np.array(state, dtype=np.float64, copy=True)
    lengths = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        if acc[b] < 0:
            continue
        idx = paths[b][int(acc[b])]
        lengths[b] = len(idx)
        sub = out[b:b + 1].copy()
        scan(x[b:b + 1, idx], B[b:b + 1, idx], None, dt[b:b + 1, idx], A, D, sub, want_y=False,
             nthreads=nthreads, lib=lib)
        out[b] = sub[0]
    return out, lengths
