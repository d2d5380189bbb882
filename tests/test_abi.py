"""Host-side checks of the C ABI (no GPU needed: nothing here enqueues device work).

The library is loaded; every function include/mil_ssm.h declares must be exported;
the cache layout must be the head-major, 256-B aligned fp32 layout; every argument
and protocol check must return its status before any launch.  Fake device addresses
are never dereferenced on the host: each call below fails its checks first.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest
from hypothesis import given, settings, strategies as st

from speculative_decode_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-B aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "mil_ssm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mil_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(L.EXPORTS) == names


def test_status_strings(lib):
    for s in range(7):
        assert lib.mil_status_string(s).decode() not in ("", "unknown status")
    assert lib.mil_status_string(99).decode() == "unknown status"


def dims(batch=2, H=32, P=128, N=128, G=8):
    return L.Dims(batch, H, P, N, G)


@pytest.mark.parametrize("shape", [(1, 2, 16, 16, 1), (16, 32, 128, 128, 8), (32, 32, 128, 256, 8),
                                   (3, 4, 32, 64, 2), (2, 8, 256, 16, 4)])
@pytest.mark.parametrize("dtype", [L.MIL_F32, L.MIL_BF16])
@pytest.mark.parametrize("k_max", [1, 4, 8, 16])
def test_layout_is_head_major_and_aligned(lib, shape, dtype, k_max):
    d = L.Dims(*shape)
    lay = L.Layout()
    assert lib.mil_ssm_cache_layout(ctypes.byref(d), k_max, dtype, ctypes.byref(lay)) == L.MIL_OK
    Bt, H, P, N, G = shape
    e = 2 if dtype == L.MIL_BF16 else 4
    offs = [lay.state_off, lay.pend_x_off, lay.pend_B_off, lay.pend_dt_off, lay.pos_off,
            lay.pending_off, lay.err_off, lay.scan_off, lay.append_off, lay.bytes]
    assert all(o % 256 == 0 for o in offs)
    assert lay.state_head_stride % 256 == 0 and lay.state_head_stride >= N * P * 4
    assert lay.state_head_stride < N * P * 4 + 256
    # regions in order, each big enough, no overlap; the prefill handoff words are
    # [slot][head][8 column slabs][64 chunk flags, the row's epoch, 3 spare words]
    sizes = [Bt * H * lay.state_head_stride, Bt * k_max * H * P * e, Bt * k_max * G * N * e,
             Bt * k_max * H * e, Bt * 4, Bt * 4, Bt * 4, Bt * H * 8 * (64 + 4) * 4, Bt * 4]
    for a, b, sz in zip(offs, offs[1:], sizes):
        assert b - a >= sz
    assert lib.mil_ssm_cache_bytes(ctypes.byref(d), k_max, dtype) == lay.bytes


@settings(max_examples=300, deadline=None)
@given(batch=st.integers(1, 4096), G=st.sampled_from([1, 2, 4, 8, 16]), rep=st.integers(1, 8),
       P=st.sampled_from([16, 32, 64, 128, 256]), N=st.sampled_from([16, 32, 64, 128, 256]),
       k_max=st.integers(1, 16), dtype=st.sampled_from([L.MIL_F32, L.MIL_BF16]))
def test_layout_regions_over_random_shapes(lib, batch, G, rep, P, N, k_max, dtype):
    """Any supported shape: every region starts on a 256-B boundary, after the end of the
    one before it, and the cache size covers the last; the two size queries agree."""
    H = G * rep
    d = L.Dims(batch, H, P, N, G)
    lay = L.Layout()
    assert lib.mil_ssm_cache_layout(ctypes.byref(d), k_max, dtype, ctypes.byref(lay)) == L.MIL_OK
    e = 2 if dtype == L.MIL_BF16 else 4
    regions = [(lay.state_off, batch * H * lay.state_head_stride),
               (lay.pend_x_off, batch * k_max * H * P * e), (lay.pend_B_off, batch * k_max * G * N * e),
               (lay.pend_dt_off, batch * k_max * H * e), (lay.pos_off, batch * 4),
               (lay.pending_off, batch * 4), (lay.err_off, batch * 4),
               (lay.scan_off, batch * H * 8 * (64 + 4) * 4), (lay.append_off, batch * 4)]
    end = 0
    for off, size in regions:
        assert off % 256 == 0 and off >= end
        end = off + size
    assert lay.bytes >= end and lay.bytes % 256 == 0 and lay.bytes - end < 256
    assert lay.state_head_stride == -(-N * P * 4 // 256) * 256
    assert lib.mil_ssm_cache_bytes(ctypes.byref(d), k_max, dtype) == lay.bytes


def test_supported_shapes(lib):
    ok = [(1, 2, 16, 16, 1), (1, 32, 128, 128, 8), (4, 32, 128, 256, 8), (1, 1, 256, 256, 1),
          (1, 4, 32, 16, 4), (1, 4, 64, 32, 2)]
    for s in ok:
        for dt in (L.MIL_F32, L.MIL_BF16):
            assert lib.mil_ssm_supported(ctypes.byref(L.Dims(*s)), dt) == L.MIL_OK, s
    assert lib.mil_ssm_supported(ctypes.byref(L.Dims(1, 32, 96, 128, 8)), 0) == L.MIL_E_UNSUPPORTED
    assert lib.mil_ssm_supported(ctypes.byref(L.Dims(1, 32, 128, 512, 8)), 0) == L.MIL_E_UNSUPPORTED
    assert lib.mil_ssm_supported(ctypes.byref(L.Dims(1, 30, 128, 128, 8)), 0) == L.MIL_E_INVALID
    assert lib.mil_ssm_supported(ctypes.byref(L.Dims(0, 32, 128, 128, 8)), 0) == L.MIL_E_INVALID
    assert lib.mil_ssm_supported(ctypes.byref(L.Dims(1, 32, 128, 128, 8)), 7) == L.MIL_E_INVALID
    assert lib.mil_ssm_supported(None, 0) == L.MIL_E_INVALID


def test_layout_rejects_bad_k_max(lib):
    lay = L.Layout()
    for k in (0, -1, L.MIL_KMAX_LIMIT + 1):
        assert lib.mil_ssm_cache_layout(ctypes.byref(dims()), k, 1, ctypes.byref(lay)) == L.MIL_E_INVALID
    assert lib.mil_ssm_cache_bytes(ctypes.byref(dims()), 0, 1) == 0


def test_workspace_bytes(lib):
    d = dims(batch=1)
    w = lib.mil_ssm_prefill_workspace_bytes(ctypes.byref(d), 1, 8192, 256)
    # one fp32 N x P state per chunk and head, plus one decay total each
    assert w >= 32 * 32 * 128 * 128 * 4 + 32 * 32 * 4
    assert w % 256 == 0
    assert lib.mil_ssm_prefill_workspace_bytes(ctypes.byref(d), 1, 8192, 100) == 0
    assert lib.mil_ssm_prefill_workspace_bytes(ctypes.byref(d), 0, 8192, 256) == 0
    assert lib.mil_ssm_prefill_workspace_bytes(ctypes.byref(d), 1, 0, 256) == 0


def attached(lib, k_max=8, dtype=L.MIL_BF16, d=None):
    d = d or dims()
    c = L.CacheDesc()
    nbytes = lib.mil_ssm_cache_bytes(ctypes.byref(d), k_max, dtype)
    assert lib.mil_ssm_cache_attach(ctypes.byref(c), ctypes.byref(d), k_max, dtype,
                                    ctypes.c_void_p(FAKE), nbytes) == L.MIL_OK
    return c


def test_attach_and_init_checks(lib):
    d = dims()
    c = L.CacheDesc()
    n = lib.mil_ssm_cache_bytes(ctypes.byref(d), 8, 1)
    assert lib.mil_ssm_cache_phase(ctypes.byref(c)) == L.PHASE_UNINIT
    assert lib.mil_ssm_cache_attach(ctypes.byref(c), ctypes.byref(d), 8, 1, None, n) == L.MIL_E_INVALID
    assert lib.mil_ssm_cache_attach(ctypes.byref(c), ctypes.byref(d), 8, 1, ctypes.c_void_p(FAKE + 128), n) \
        == L.MIL_E_ALIGN
    assert lib.mil_ssm_cache_attach(ctypes.byref(c), ctypes.byref(d), 8, 1, ctypes.c_void_p(FAKE), n - 1) \
        == L.MIL_E_INVALID
    assert lib.mil_ssm_cache_init(ctypes.byref(c), ctypes.byref(d), 8, 1, ctypes.c_void_p(FAKE + 64), n, None) \
        == L.MIL_E_ALIGN
    assert lib.mil_ssm_cache_init(ctypes.byref(c), ctypes.byref(L.Dims(1, 32, 96, 128, 8)), 8, 1,
                                  ctypes.c_void_p(FAKE), n, None) == L.MIL_E_UNSUPPORTED
    assert lib.mil_ssm_cache_phase(ctypes.byref(c)) == L.PHASE_UNINIT
    c = attached(lib)
    assert lib.mil_ssm_cache_phase(ctypes.byref(c)) == L.PHASE_READY


def P(v=FAKE):
    return ctypes.c_void_p(v)


def test_verify_argument_checks(lib):
    c = attached(lib, k_max=8)
    f = lib.mil_ssm_verify
    ok = [P(), P(), P(), P(), P(), P(), P()]
    assert f(None, 4, *ok, None) == L.MIL_E_INVALID
    assert f(ctypes.byref(L.CacheDesc()), 4, *ok, None) == L.MIL_E_INVALID  # never initialised
    assert f(ctypes.byref(c), 0, *ok, None) == L.MIL_E_INVALID
    assert f(ctypes.byref(c), 9, *ok, None) == L.MIL_E_INVALID  # K > k_max
    for i in range(7):
        args = list(ok)
        args[i] = None
        assert f(ctypes.byref(c), 4, *args, None) == L.MIL_E_INVALID, i
    args = list(ok)
    args[0] = P(FAKE + 1)  # bf16 x must be 2-B aligned
    assert f(ctypes.byref(c), 4, *args, None) == L.MIL_E_ALIGN
    args = list(ok)
    args[6] = P(FAKE + 2)  # fp32 y must be 4-B aligned
    assert f(ctypes.byref(c), 4, *args, None) == L.MIL_E_ALIGN
    assert lib.mil_ssm_cache_phase(ctypes.byref(c)) == L.PHASE_READY


def test_commit_before_verify_is_out_of_order(lib):
    c = attached(lib)
    assert lib.mil_ssm_commit(ctypes.byref(c), 4, P(), P(), P(), P(), P(), P(), 0, None) == L.MIL_E_ORDER
    assert lib.mil_ssm_cache_phase(ctypes.byref(c)) == L.PHASE_READY


def test_prefill_argument_checks(lib):
    c = attached(lib, d=dims(batch=2))
    d = dims(batch=2)
    need = lib.mil_ssm_prefill_workspace_bytes(ctypes.byref(d), 1, 100, 256)
    f = lib.mil_ssm_prefill

    def call(slot0=0, nseq=1, Lt=100, chunk=256, ws=P(), ws_bytes=need, flags=0, x=P(), y=P()):
        return f(ctypes.byref(c), slot0, nseq, Lt, chunk, x, P(), P(), P(), P(), P(), y, ws, ws_bytes, flags, None)

    assert call(slot0=2) == L.MIL_E_INVALID
    assert call(slot0=1, nseq=2) == L.MIL_E_INVALID
    assert call(slot0=-1) == L.MIL_E_INVALID
    assert call(Lt=0) == L.MIL_E_INVALID
    assert call(chunk=100) == L.MIL_E_INVALID
    assert call(flags=4) == L.MIL_E_INVALID
    assert call(x=None) == L.MIL_E_INVALID
    assert call(x=P(FAKE + 1)) == L.MIL_E_ALIGN
    assert call(y=P(FAKE + 2)) == L.MIL_E_ALIGN
    assert call(ws=None) == L.MIL_E_WORKSPACE
    assert call(ws_bytes=need - 1) == L.MIL_E_WORKSPACE
    assert call(ws=P(FAKE + 16)) == L.MIL_E_ALIGN


def test_cache_status_checks(lib):
    bad = ctypes.c_int32()
    assert lib.mil_ssm_cache_status(None, ctypes.byref(bad), 0, None) == L.MIL_E_INVALID
    c = attached(lib)
    assert lib.mil_ssm_cache_status(ctypes.byref(c), None, 0, None) == L.MIL_E_INVALID


def test_largest_state_with_most_drafts_is_accepted(lib):
    """N = P = 256 with k_max = 16 needs more LDS than one whole-row workgroup has; the
    verify launch then splits the columns, so init and attach accept the shape."""
    d = L.Dims(1, 1, 256, 256, 1)
    for dtype in (L.MIL_F32, L.MIL_BF16):
        c = L.CacheDesc()
        n = lib.mil_ssm_cache_bytes(ctypes.byref(d), L.MIL_KMAX_LIMIT, dtype)
        assert lib.mil_ssm_cache_attach(ctypes.byref(c), ctypes.byref(d), L.MIL_KMAX_LIMIT, dtype,
                                        ctypes.c_void_p(FAKE), n) == L.MIL_OK


def test_greedy_workspace_bytes(lib):
    d = dims(batch=16)
    w = lib.mil_ssm_greedy_workspace_bytes(ctypes.byref(d), 8, 128256)
    assert w >= 16 * 8 * 8 and w % 256 == 0
    assert lib.mil_ssm_greedy_workspace_bytes(ctypes.byref(d), 0, 128256) == 0
    assert lib.mil_ssm_greedy_workspace_bytes(ctypes.byref(d), L.MIL_KMAX_LIMIT + 1, 128256) == 0
    assert lib.mil_ssm_greedy_workspace_bytes(ctypes.byref(d), 8, 0) == 0


def test_commit_greedy_checks(lib):
    c = attached(lib, k_max=8)
    f = lib.mil_ssm_commit_greedy
    need = lib.mil_ssm_greedy_workspace_bytes(ctypes.byref(dims()), 4, 1000)

    def call(cache=c, K=4, draft=P(), logits=P(), vocab=1000, ldt=L.MIL_BF16, acc=P(), tok=None, ws=P(),
             ws_bytes=need, flags=0):
        return f(ctypes.byref(cache), K, draft, logits, vocab, ldt, acc, tok, P(), P(), P(), None, None, ws,
                 ws_bytes, flags, None)

    assert call() == L.MIL_E_ORDER  # no verify before it (the checks after a verify are GPU tests)
    assert call(cache=L.CacheDesc()) == L.MIL_E_INVALID  # never initialised
    assert lib.mil_ssm_cache_phase(ctypes.byref(c)) == L.PHASE_READY


def test_project_workspace_bytes(lib):
    d = dims(batch=1, H=32, P=128, N=128, G=8)
    ncols = 32 * 128 + 2 * 8 * 128 + 32
    # a decode round's rows (few): the inputs are split, so partial sums need room
    w = lib.mil_ssm_project_workspace_bytes(ctypes.byref(d), 128, 4096)
    assert w >= 2 * 128 * ncols * 4 and w % 256 == 0
    assert lib.mil_ssm_project_workspace_bytes(ctypes.byref(d), 4, 4096) >= 2 * 4 * ncols * 4
    # a long prompt fills the GPU without a split: no workspace
    assert lib.mil_ssm_project_workspace_bytes(ctypes.byref(d), 8192, 4096) == 0
    # unsupported widths and bad sizes report 0
    assert lib.mil_ssm_project_workspace_bytes(ctypes.byref(d), 128, 100) == 0
    assert lib.mil_ssm_project_workspace_bytes(ctypes.byref(d), 0, 4096) == 0


def test_project_argument_checks(lib):
    d = dims(batch=1, H=32, P=128, N=128, G=8)
    f = lib.mil_ssm_project
    need = lib.mil_ssm_project_workspace_bytes(ctypes.byref(d), 128, 4096)

    def call(dd=d, T=128, dm=4096, u=P(), wx=P(), bias=None, odt=L.MIL_BF16, x=P(), ws=P(), ws_bytes=need):
        return f(ctypes.byref(dd), T, dm, u, wx, P(), P(), P(), bias, odt, x, P(), P(), P(), ws, ws_bytes, None)

    assert call(u=None) == L.MIL_E_INVALID
    assert call(wx=None) == L.MIL_E_INVALID
    assert call(x=None) == L.MIL_E_INVALID
    assert call(T=0) == L.MIL_E_INVALID
    assert call(odt=7) == L.MIL_E_INVALID
    assert call(dm=100) == L.MIL_E_UNSUPPORTED
    assert call(ws=None) == L.MIL_E_WORKSPACE
    assert call(ws_bytes=need - 1) == L.MIL_E_WORKSPACE
    assert call(u=P(8)) == L.MIL_E_ALIGN
    assert call(x=P(1)) == L.MIL_E_ALIGN
    assert call(bias=P(2)) == L.MIL_E_ALIGN
    assert call(dd=dims(batch=1, H=3, P=128, N=128, G=2)) == L.MIL_E_INVALID  # H % G != 0


def test_tree_call_checks(lib):
    c = attached(lib, k_max=8)
    vt, ct = lib.mil_ssm_verify_tree, lib.mil_ssm_commit_tree

    def verify(cache=c, K=4, parent=P(), y=P()):
        return vt(ctypes.byref(cache), K, parent, P(), P(), P(), P(), P(), P(), y, None)

    def commit(cache=c, K=4, parent=P(), node=P(), flags=0):
        return ct(ctypes.byref(cache), K, parent, node, P(), P(), P(), None, None, flags, None)

    assert commit() == L.MIL_E_ORDER  # no verify before it
    assert verify(parent=None) == L.MIL_E_INVALID
    assert verify(K=0) == L.MIL_E_INVALID
    assert verify(K=9) == L.MIL_E_INVALID  # above k_max
    assert verify(parent=P(FAKE + 2)) == L.MIL_E_ALIGN
    assert verify(cache=L.CacheDesc()) == L.MIL_E_INVALID
    assert lib.mil_ssm_cache_phase(ctypes.byref(c)) == L.PHASE_READY


def test_commit_layers_checks(lib):
    """Every check of the multi-layer commit that returns before anything is enqueued."""
    f = lib.mil_ssm_commit_layers
    a, b = attached(lib), attached(lib)
    other = attached(lib, d=dims(batch=4))

    def call(cs, n=None, accepted=P(), ptrs=None):
        n = len(cs) if n is None else n
        arr = (ctypes.POINTER(L.CacheDesc) * max(len(cs), 1))(*[ctypes.pointer(c) for c in cs])
        ptrs = ptrs or [P()] * max(len(cs), 1)
        vp = (ctypes.c_void_p * len(ptrs))(*ptrs)
        return f(arr, n, 4, accepted, vp, vp, vp, None)

    assert f(None, 2, 4, P(), None, None, None, None) == L.MIL_E_INVALID
    assert call([a, b], n=0) == L.MIL_E_INVALID
    assert call([a, b], accepted=None) == L.MIL_E_INVALID
    assert call([a, b], ptrs=[P(), None]) == L.MIL_E_INVALID  # a null draft pointer
    assert call([a, a]) == L.MIL_E_INVALID                    # a cache twice
    assert call([a, other]) == L.MIL_E_INVALID                # shapes differ
    assert call([a, L.CacheDesc()]) == L.MIL_E_INVALID        # not a cache
    assert call([a, b]) == L.MIL_E_ORDER                      # no verify before it
    for c in (a, b, other):
        assert lib.mil_ssm_cache_phase(ctypes.byref(c)) == L.PHASE_READY


def test_debug_mode_reports_failed_calls():
    """MIL_SSM_DEBUG=1: a failing call names itself and its status on stderr; unset, the
    library prints nothing."""
    import os
    import subprocess
    import sys
    prog = (
        "import ctypes, sys\n"
        f"sys.path.insert(0, {os.path.dirname(os.path.dirname(os.path.abspath(__file__)))!r})\n"
        "from speculative_decode_amd import _lib as L\n"
        "lib = L.lib()\n"
        "d = L.Dims(2, 32, 128, 128, 8)\n"
        "c = L.CacheDesc()\n"
        "st = lib.mil_ssm_verify(ctypes.byref(c), 4, None, None, None, None, None, None, None, None)\n"
        "print(st)\n"
    )
    for env, expect in (({"MIL_SSM_DEBUG": "1"}, True), ({"MIL_SSM_DEBUG": "0"}, False), ({}, False)):
        e = {k: v for k, v in os.environ.items() if k != "MIL_SSM_DEBUG"}
        e.update(env)
        r = subprocess.run([sys.executable, "-c", prog], capture_output=True, text=True, env=e, timeout=120)
        assert r.returncode == 0, r.stderr
        assert r.stdout.strip() == str(L.MIL_E_INVALID)
        said = "mil_ssm debug: mil_ssm_verify returned" in r.stderr
        assert said == expect, (env, r.stderr)
