"""GPU parity of the input projections (mil_ssm_project) against the oracle's project().

Bounds, from the arithmetic: the products of bf16 values are exact in fp32 and are summed
in fp32, so an output may differ from the exact sum by at most a small multiple of the
unit roundoff times sum_k |u_k w_k| (1e-6 of it is used: about 16 ulp of that sum, which
covers the fp32 summation of up to a few thousand terms with a wide margin); a bf16 output
adds one rounding to nearest, at most 2^-8 of its value; softplus is 1-Lipschitz, so the
step size inherits the same bound plus a few ulp of its own evaluation.  With small
integer inputs every partial sum is an exact fp32 integer, so x, B and C are bit-exact
(fp32), or the round-to-nearest-even of the exact value (bf16).  The rows cover several
column tiles and ragged ends in both directions (T and the dt block's 32 columns), the
unsplit and the split-input forms (a few rows), and the full decode-round sizes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import BOUND, TOL, dev, dev_layer, y_err
from speculative_decode_amd import _lib as L
from speculative_decode_amd import synth
from speculative_decode_amd.ssm import SSMCache, project, project_workspace_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.lib()  # a missing library is a failure, not a skip


def run(pr: synth.Projection, H, P, N, G, out_dtype, bias=True):
    u = dev(pr.u)
    outs = project(u, dev(pr.w_x), dev(pr.w_B), dev(pr.w_C), dev(pr.w_dt), H, P, N, G,
                   dt_bias=dev(pr.bias) if bias else None, out_dtype=out_dtype)
    torch.cuda.synchronize()
    T = pr.u.store.shape[0]
    return [o.float().cpu().numpy().astype(np.float64).reshape(T, -1) for o in outs]


def reference(pr: synth.Projection, bias=True):
    return oracle.project(pr.u.f64, pr.w_x.f64, pr.w_B.f64, pr.w_C.f64, pr.w_dt.f64,
                          pr.bias.f64 if bias else None)


def magnitude(pr: synth.Projection, bias=True):
    """sum_k |u_k w_k| per output element (the scale of fp32 summation error)."""
    au = np.abs(pr.u.f64)
    return [au @ np.abs(w.f64).T for w in (pr.w_x, pr.w_B, pr.w_C, pr.w_dt)]


def check(gpu, ref, mag, bf16_out):
    for i, (g, r, m) in enumerate(zip(gpu, ref, mag)):
        tol = 1e-6 * m + (2.0 ** -8 * np.abs(r) if bf16_out else 0.0)
        if i == 3:
            tol = tol + 1e-6 * np.abs(r)
        bad = np.abs(g - r) > tol
        assert not bad.any(), (["x", "B", "C", "dt"][i], int(bad.sum()), float(np.max(np.abs(g - r) - tol)))


CASES = [
    # (T, d_model, (H, P, N, G)) -- several column tiles, ragged T, short and long d
    (1, 64, (2, 16, 16, 1)),
    (3, 192, (2, 16, 16, 1)),      # 3 input blocks: the ring's guarded tail
    (33, 256, (4, 32, 64, 2)),
    (100, 640, (4, 32, 64, 2)),    # 10 blocks
    (300, 192, (8, 64, 32, 4)),    # three 128-row tiles, ragged
    (4, 4096, (32, 128, 128, 8)),  # split inputs, one verify round of a single sequence
    (70, 1024, (32, 128, 128, 8)),
]


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_d{c[1]}_H{c[2][0]}" for c in CASES])
def test_project_matches_oracle(case, out_dtype):
    T, d, (H, P, N, G) = case
    rng = np.random.default_rng(3000 + T + d)
    pr = synth.draw_projection(rng, T, d, H, P, N, G)
    print(f"project T={T} d={d} H={H} P={P} N={N} G={G} out={out_dtype}", flush=True)
    gpu = run(pr, H, P, N, G, out_dtype)
    check(gpu, reference(pr), magnitude(pr), out_dtype == torch.bfloat16)


@pytest.mark.parametrize("case", [(128, 4096, (32, 128, 128, 8)), (128, 4096, (32, 128, 256, 8))],
                         ids=["batched_8b", "hybrid_n256"])
def test_project_full_decode_round(case):
    # the decode-round sizes of the batched (16 x 8 drafts) and hybrid (32 x 4) workloads
    T, d, (H, P, N, G) = case
    pr = synth.draw_projection(np.random.default_rng(3100 + N), T, d, H, P, N, G)
    print(f"project full T={T} d={d} N={N}", flush=True)
    gpu = run(pr, H, P, N, G, torch.bfloat16)
    check(gpu, reference(pr), magnitude(pr), True)


@pytest.mark.parametrize("case", [(5, 4096, (32, 128, 128, 8)), (130, 192, (4, 32, 64, 2))],
                         ids=["split", "unsplit"])
def test_project_integers_are_exact(case):
    T, d, (H, P, N, G) = case
    pr = synth.integer_projection(np.random.default_rng(3200 + T), T, d, H, P, N, G)
    ref = reference(pr, bias=False)
    print(f"project integers T={T} d={d}", flush=True)
    g32 = run(pr, H, P, N, G, torch.float32, bias=False)
    for i in range(3):
        assert np.array_equal(g32[i], ref[i]), i
    g16 = run(pr, H, P, N, G, torch.bfloat16, bias=False)
    for i in range(3):
        want = synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(ref[i].astype(np.float32)))
        assert np.array_equal(g16[i], want), i


def test_project_is_deterministic_and_bias_optional():
    T, d, (H, P, N, G) = 16, 2048, (32, 128, 128, 8)
    pr = synth.draw_projection(np.random.default_rng(3300), T, d, H, P, N, G)
    print("project determinism", flush=True)
    a = run(pr, H, P, N, G, torch.float32)
    b = run(pr, H, P, N, G, torch.float32)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.int64), y.view(np.int64))
    nb = run(pr, H, P, N, G, torch.float32, bias=False)
    check(nb, reference(pr, bias=False), magnitude(pr), False)
    assert project_workspace_bytes(H, P, N, G, T, d) > 0


def test_project_feeds_verify():
    """Projections straight into verify: the GPU chain (project, prefill, verify) against
    the oracle's prefill and verify on exactly the tokens the device projected (the layer's
    bound), and against the oracle's whole chain (project in float64, rounded to bf16 as
    the device stores it, then prefill and verify): there a product summed in fp32 may round
    to the neighbouring bf16 value on a boundary, which moves y by up to ~1e-3 of its scale,
    so that comparison takes the stated bf16 tolerance."""
    Bt, K, H, P, N, G, d = 4, 4, 32, 128, 128, 8, 1024
    rng = np.random.default_rng(3400)
    layer = synth.draw_layer(rng, H)
    ctx = synth.draw_projection(rng, Bt * 32, d, H, P, N, G)
    drafts = synth.draw_projection(rng, Bt * K, d, H, P, N, G)
    drafts.w_x, drafts.w_B, drafts.w_C, drafts.w_dt, drafts.bias = ctx.w_x, ctx.w_B, ctx.w_C, ctx.w_dt, ctx.bias
    A, D = dev_layer(layer)
    print("project -> prefill -> verify", flush=True)

    def gpu_tokens(pr, T):
        w = [dev(t) for t in (pr.w_x, pr.w_B, pr.w_C, pr.w_dt)]
        x, B, C, dt = project(dev(pr.u).view(Bt, T, d), *w, H, P, N, G, dt_bias=dev(pr.bias))
        return x, B, C, dt

    cache = SSMCache(Bt, H, P, N, G, 8, synth.BF16)
    ctx_dev = gpu_tokens(ctx, 32)
    drf_dev = gpu_tokens(drafts, K)
    cache.prefill(*ctx_dev, A, D, chunk=64)
    y = cache.verify(*drf_dev, A, D)
    torch.cuda.synchronize()

    # the oracle on exactly the tokens the device projected: the layer's own bound
    def as_f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    _, h_dev = oracle.prefill(*(as_f64(t) for t in ctx_dev), layer.A.f64, layer.D.f64)
    y_same = oracle.verify(h_dev, *(as_f64(t) for t in drf_dev), layer.A.f64, layer.D.f64)
    err_same = y_err(y.cpu().numpy(), y_same)
    print(f"verify on the projected tokens: y err {err_same:.3e}", flush=True)
    assert err_same <= BOUND[synth.BF16]

    def ref_tokens(pr, T):
        x, B, C, dt = reference(pr)
        r = [synth.quantize(v, synth.BF16).f64 for v in (x, B, C, dt)]
        return (r[0].reshape(Bt, T, H, P), r[1].reshape(Bt, T, G, N), r[2].reshape(Bt, T, G, N),
                r[3].reshape(Bt, T, H))

    cx, cB, cC, cdt = ref_tokens(ctx, 32)
    _, h = oracle.prefill(cx, cB, cC, cdt, layer.A.f64, layer.D.f64)
    dx, dB, dC, ddt = ref_tokens(drafts, K)
    y_ref = oracle.verify(h, dx, dB, dC, ddt, layer.A.f64, layer.D.f64)
    err = y_err(y.cpu().numpy(), y_ref)
    print(f"project -> verify y err {err:.3e}", flush=True)
    assert err <= TOL[synth.BF16]
