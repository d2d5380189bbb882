"""Seeded synthetic inputs for the SSM layer, shared by tests, the bench and smoke.

This module draws random numbers and rounds them to the storage dtype. It holds
none of the layer's arithmetic: no discretisation, no recurrence, no readout.
Both the GPU path and the CPU oracle receive exactly the arrays made here.

Recipe (the layer of "The Mamba in the Llama", with x from the V projection,
B from K, C from Q; the pages give no trained weights, so every tensor is drawn):
  * per layer:   A_h = -exp(U(0, ln 16))  (so A in [-16, -1]),  D_h ~ N(0, 1)
  * per token:   x ~ N(0,1)/4 [T][H][P],  B ~ N(0,1)/4 [T][G][N],
                 C ~ N(0,1)/4 [T][G][N],  dt = softplus(z), z ~ N(-1, 0.5) [T][H]
  * draw order:  x, B, C, z for each block of tokens, sequences in order
  * rounding:    fp64 -> fp32 (round to nearest), then for bf16 inputs
                 fp32 -> bf16 with round-to-nearest-even on the bit pattern.
A and D always stay fp32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    u = b.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Tensor:
    """One input tensor: `store` is what the device receives (float32, or uint16 bf16
    bits), `f64` is the same values widened exactly to double for the oracle."""

    store: np.ndarray
    f64: np.ndarray
    dtype: str


def quantize(v64: np.ndarray, dtype: str) -> Tensor:
    v32 = v64.astype(np.float32)
    if dtype == F32:
        return Tensor(v32, v32.astype(np.float64), F32)
    if dtype == BF16:
        bits = f32_to_bf16_bits(v32)
        return Tensor(bits, bf16_bits_to_f64(bits), BF16)
    raise ValueError(f"unknown dtype {dtype}")


@dataclasses.dataclass
class Layer:
    A: Tensor  # [H] fp32
    D: Tensor  # [H] fp32


@dataclasses.dataclass
class Tokens:
    """Per-token projected inputs for `batch` sequences of `T` tokens."""

    x: Tensor   # [batch][T][H][P]
    B: Tensor   # [batch][T][G][N]
    C: Tensor   # [batch][T][G][N]
    dt: Tensor  # [batch][T][H]

    @property
    def T(self) -> int:
        return self.x.store.shape[1]


def softplus(z: np.ndarray) -> np.ndarray:
    # numerically safe log(1 + e^z) in fp64; part of the input recipe, not of the layer
    return np.logaddexp(0.0, z)


def draw_layer(rng: np.random.Generator, H: int) -> Layer:
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=H))
    D = rng.normal(0.0, 1.0, size=H)
    return Layer(quantize(A, F32), quantize(D, F32))


def draw_tokens(rng: np.random.Generator, batch: int, T: int, H: int, P: int, N: int,
                G: int, dtype: str) -> Tokens:
    x = rng.normal(0.0, 1.0, size=(batch, T, H, P)) / 4.0
    B = rng.normal(0.0, 1.0, size=(batch, T, G, N)) / 4.0
    C = rng.normal(0.0, 1.0, size=(batch, T, G, N)) / 4.0
    z = rng.normal(-1.0, 0.5, size=(batch, T, H))
    return Tokens(quantize(x, dtype), quantize(B, dtype), quantize(C, dtype),
                  quantize(softplus(z), dtype))


@dataclasses.dataclass
class Projection:
    """Layer input rows and the four projection weight blocks (all bf16) plus the fp32
    step-size bias, for the input step before the layer."""

    u: Tensor      # [T][d]
    w_x: Tensor    # [H*P][d]  value rows
    w_B: Tensor    # [G*N][d]  key rows
    w_C: Tensor    # [G*N][d]  query rows
    w_dt: Tensor   # [H][d]
    bias: Tensor   # [H] fp32


def draw_projection(rng: np.random.Generator, T: int, d: int, H: int, P: int, N: int, G: int) -> Projection:
    """Seeded stand-ins for trained weights (none are available): u ~ N(0, 1); the x, B, C
    rows ~ N(0, 1/(16 d)) and the step-size rows ~ N(0, 1/(4 d)) with bias -1, so that the
    projected values have about the per-token distributions of the recipe above
    (N(0,1)/4, and softplus of N(-1, 0.5)).  Draw order: u, w_x, w_B, w_C, w_dt."""
    u = rng.normal(0.0, 1.0, size=(T, d))
    sx = 0.25 / math.sqrt(d)
    w_x = rng.normal(0.0, sx, size=(H * P, d))
    w_B = rng.normal(0.0, sx, size=(G * N, d))
    w_C = rng.normal(0.0, sx, size=(G * N, d))
    w_dt = rng.normal(0.0, 0.5 / math.sqrt(d), size=(H, d))
    return Projection(quantize(u, BF16), quantize(w_x, BF16), quantize(w_B, BF16), quantize(w_C, BF16),
                      quantize(w_dt, BF16), quantize(np.full(H, -1.0), F32))


def integer_projection(rng: np.random.Generator, T: int, d: int, H: int, P: int, N: int, G: int,
                       lo: int = -2, hi: int = 2) -> Projection:
    """Small integers (exact in bf16, and every sum of products exact in fp32 while
    d * max|u| * max|w| < 2^24), no bias."""
    def ints(shape):
        return rng.integers(lo, hi + 1, size=shape).astype(np.float64)
    return Projection(quantize(ints((T, d)), BF16), quantize(ints((H * P, d)), BF16),
                      quantize(ints((G * N, d)), BF16), quantize(ints((G * N, d)), BF16),
                      quantize(ints((H, d)), BF16), quantize(np.zeros(H), F32))


def draw_tree(rng: np.random.Generator, batch: int, K: int, kind: str = "random") -> np.ndarray:
    """Draft-tree links parent [batch][K] int32 (-1..k-1; -1 = the committed state):
    "random": parent[b][k] ~ U{-1..k-1}; "chain": k-1; "binary": node 0 follows the state
    and node k >= 1 follows node (k-1)//2; "fan": every node follows the state."""
    if kind == "chain":
        return np.tile(np.arange(-1, K - 1, dtype=np.int32), (batch, 1))
    if kind == "binary":
        row = np.array([-1] + [(k - 1) // 2 for k in range(1, K)], dtype=np.int32)
        return np.tile(row, (batch, 1))
    if kind == "fan":
        return np.full((batch, K), -1, dtype=np.int32)
    par = np.zeros((batch, K), dtype=np.int32)
    for b in range(batch):
        for k in range(K):
            par[b, k] = rng.integers(-1, k)
    return par


def draw_accept_uniform(rng: np.random.Generator, batch: int, K: int) -> np.ndarray:
    """Accepted lengths j ~ U{0..K} (inclusive), int32."""
    return rng.integers(0, K + 1, size=batch).astype(np.int32)


def draw_accept_geometric(rng: np.random.Generator, batch: int, K: int, p: float = 0.3) -> np.ndarray:
    """Accepted lengths j = min(Geom(p) - 1, K): P(j=k) = p (1-p)^k for k < K."""
    return np.minimum(rng.geometric(p, size=batch) - 1, K).astype(np.int32)


def draw_greedy(rng: np.random.Generator, batch: int, K: int, vocab: int, dtype: str,
                planted: np.ndarray, ties: bool = False):
    """Verifier logits [batch][K][vocab] ~ N(0,1) and draft tokens [batch][K] ~ U{0..vocab-1},
    with a structure planted so that greedy verification accepts planted[b] drafts: at
    positions k < planted[b] the draft's logit is set to 16 (far above every N(0,1) draw),
    at k = planted[b] to -16.  With ties=True, some planted maxima get a second 16 at
    another id (lower or higher than the draft), which makes the tie rule decide.
    Returns (draft_tokens int32, logits Tensor)."""
    draft = rng.integers(0, vocab, size=(batch, K)).astype(np.int32)
    lg = rng.standard_normal((batch, K, vocab))
    for b in range(batch):
        for k in range(K):
            if k < planted[b]:
                lg[b, k, draft[b, k]] = 16.0
                if ties and rng.random() < 0.5:
                    other = int(rng.integers(0, vocab))
                    if other != draft[b, k]:
                        lg[b, k, other] = 16.0
            elif k == planted[b]:
                lg[b, k, draft[b, k]] = -16.0
    return draft, quantize(lg, dtype)


def integer_tokens(rng: np.random.Generator, batch: int, T: int, H: int, P: int, N: int,
                   G: int, dtype: str, lo: int = -1, hi: int = 1) -> Tokens:
    """Small-integer x, B, C with dt = 1: every product and partial sum of the
    causal-linear-attention special case is exact in fp32 and bf16."""
    x = rng.integers(lo, hi + 1, size=(batch, T, H, P)).astype(np.float64)
    B = rng.integers(lo, hi + 1, size=(batch, T, G, N)).astype(np.float64)
    C = rng.integers(lo, hi + 1, size=(batch, T, G, N)).astype(np.float64)
    dt = np.ones((batch, T, H))
    return Tokens(quantize(x, dtype), quantize(B, dtype), quantize(C, dtype), quantize(dt, dtype))


def concat_tokens(parts: list[Tokens]) -> Tokens:
    """Join token blocks along the token axis (same batch and shapes)."""
    def cat(name):
        ts = [getattr(p, name) for p in parts]
        return Tensor(np.concatenate([t.store for t in ts], axis=1),
                      np.concatenate([t.f64 for t in ts], axis=1), ts[0].dtype)
    return Tokens(cat("x"), cat("B"), cat("C"), cat("dt"))


def slice_tokens(t: Tokens, b0: int, b1: int, t0: int, t1: int) -> Tokens:
    def sl(v: Tensor) -> Tensor:
        return Tensor(np.ascontiguousarray(v.store[b0:b1, t0:t1]),
                      np.ascontiguousarray(v.f64[b0:b1, t0:t1]), v.dtype)
    return Tokens(sl(t.x), sl(t.B), sl(t.C), sl(t.dt))


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload (a Llama-3-8B-derived hybrid layer or a tiny case)."""

    name: str
    batch: int
    H: int
    P: int
    N: int
    G: int
    dtype: str
    K: int = 0            # drafts per verify round
    L: int = 0            # prefill length (fixed) or 0 when ctx_range is used
    ctx_range: tuple = () # (lo, hi) inclusive per-sequence prefill lengths
    chunk: int = 256
    layers: int = 1
    accept: str = "uniform"  # or "geometric", or "greedy" (decided on the device from verifier logits)
    vocab: int = 0           # vocabulary size of the verifier logits ("greedy")
    d_model: int = 0         # > 0: the drafts' x, B, C, dt are projected on the device from
                             # layer input rows of this width (the step before the layer)
    tree: str = ""           # draft-tree shape (draw_tree kinds); accept "tree" takes one node
    kmax: int = 0            # pending rows a cache holds (0: K); above K, accepted rows collect
                             # over rounds and a verify writes the state back only when full
    seed: int = 1000


WORKLOADS = {
    # tiny fp32 case: every step cheap enough for the oracle at once
    "tiny_f32": Workload("tiny_f32", batch=1, H=2, P=16, N=16, G=1, dtype=F32, K=4, L=64,
                         chunk=256, seed=1001),
    # one Llama-3-8B-shaped sequence: 32 heads, P=N=128, 8 B/C groups
    "llama8b_single": Workload("llama8b_single", batch=1, H=32, P=128, N=128, G=8, dtype=BF16,
                               K=4, L=1024, seed=1002),
    # batched verify: 16 sequences with prior contexts U{256..4096}
    "llama8b_batched": Workload("llama8b_batched", batch=16, H=32, P=128, N=128, G=8,
                                dtype=BF16, K=8, ctx_range=(256, 4096), seed=1003),
    # the batched round with its acceptance decided on the device: greedy verification
    # against bf16 verifier logits over the Llama-3 vocabulary (128256 tokens)
    "llama8b_batched_greedy": Workload("llama8b_batched_greedy", batch=16, H=32, P=128, N=128, G=8,
                                       dtype=BF16, K=8, ctx_range=(256, 4096), accept="greedy",
                                       vocab=128256, seed=1006),
    # the batched round from the layer's input rows: the drafts' x, B, C, dt projected on
    # the device (Llama-3-8B width 4096; seeded stand-in weights) before verify and commit
    "llama8b_batched_project": Workload("llama8b_batched_project", batch=16, H=32, P=128, N=128, G=8,
                                        dtype=BF16, K=8, ctx_range=(256, 4096), d_model=4096, seed=1007),
    # the batched round with tree drafts: 8 candidate tokens per sequence in a random tree
    # (parent ~ U{-1..k-1}), one accepted node ~ U{-1..7} whose root path is kept
    "llama8b_batched_tree": Workload("llama8b_batched_tree", batch=16, H=32, P=128, N=128, G=8, dtype=BF16,
                                     K=8, ctx_range=(256, 4096), accept="tree", tree="random", seed=1008),
    # one long prefill scan
    "llama8b_long_prefill": Workload("llama8b_long_prefill", batch=1, H=32, P=128, N=128, G=8,
                                     dtype=BF16, L=8192, chunk=256, seed=1004),
    # hybrid decode step: 24 SSM layers, batch 32, expanded state N=256
    "hybrid_decode": Workload("hybrid_decode", batch=32, H=32, P=128, N=256, G=8, dtype=BF16,
                              K=4, L=1024, layers=24, accept="geometric", kmax=8, seed=1005),
}
