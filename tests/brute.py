"""Independent brute force of the SSM layer in its quadratic ("attention") form.

Unrolling the recurrence of the Mamba layer in "The Mamba in the Llama" (the
layer the abstract says is distilled from attention) gives, for one sequence
and head, with S(u, v) = sum_{r=u+1..v} dt_r:

  y_t = sum_{s<=t} exp(A S(s,t)) dt_s (C_t . B_s) x_s
        + exp(A S(0,t)) C_t^T h_0 + D x_t
  h_T = exp(A S(0,T)) h_0 + sum_{s<=T} exp(A S(s,T)) dt_s B_s x_s^T

With A = 0 and dt = 1 this is causal linear attention with C as queries and B
as keys.  This file writes that form out with explicit Python loops, for tiny
shapes only; it never calls the oracle.
"""
from __future__ import annotations

import math

import numpy as np


def quadratic_form(x, B, C, dt, A, D, h0=None):
    """x [Bt][T][H][P], B/C [Bt][T][G][N], dt [Bt][T][H], A/D [H], h0 [Bt][H][N][P] or None.
    Returns (y [Bt][T][H][P], h_T [Bt][H][N][P]) in float64."""
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    y = np.zeros((Bt, T, H, P))
    hT = np.zeros((Bt, H, N, P))
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            a = float(A[h])
            for t in range(T):
                for p in range(P):
                    acc = 0.0
                    for s in range(t + 1):
                        seg = sum(float(dt[b, r, h]) for r in range(s + 1, t + 1))
                        cb = sum(float(C[b, t, g, n]) * float(B[b, s, g, n]) for n in range(N))
                        acc += math.exp(a * seg) * float(dt[b, s, h]) * cb * float(x[b, s, h, p])
                    if h0 is not None:
                        seg0 = sum(float(dt[b, r, h]) for r in range(0, t + 1))
                        ch = sum(float(C[b, t, g, n]) * float(h0[b, h, n, p]) for n in range(N))
                        acc += math.exp(a * seg0) * ch
                    y[b, t, h, p] = acc + float(D[h]) * float(x[b, t, h, p])
            for n in range(N):
                for p in range(P):
                    acc = 0.0
                    for s in range(T):
                        seg = sum(float(dt[b, r, h]) for r in range(s + 1, T))
                        acc += math.exp(a * seg) * float(dt[b, s, h]) * float(B[b, s, g, n]) * float(x[b, s, h, p])
                    if h0 is not None:
                        seg0 = sum(float(dt[b, r, h]) for r in range(T))
                        acc += math.exp(a * seg0) * float(h0[b, h, n, p])
                    hT[b, h, n, p] = acc
    return y, hT


def causal_linear_attention_int(x, B, C, D):
    """Exact integer closed form at A = 0, dt = 1 (Python ints, no rounding at all):
    y_t = sum_{s<=t} (C_t . B_s) x_s + D x_t, h_T = sum_s B_s x_s^T."""
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    y = [[[[0] * P for _ in range(H)] for _ in range(T)] for _ in range(Bt)]
    hT = [[[[0] * P for _ in range(N)] for _ in range(H)] for _ in range(Bt)]
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            for t in range(T):
                for p in range(P):
                    v = 0
                    for s in range(t + 1):
                        cb = sum(int(C[b, t, g, n]) * int(B[b, s, g, n]) for n in range(N))
                        v += cb * int(x[b, s, h, p])
                    y[b][t][h][p] = v + int(D[h]) * int(x[b, t, h, p])
            for n in range(N):
                for p in range(P):
                    hT[b][h][n][p] = sum(int(B[b, s, g, n]) * int(x[b, s, h, p]) for s in range(T))
    return y, hT
