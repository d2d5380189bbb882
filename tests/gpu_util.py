"""Helpers for the GPU parity tests: moving seeded inputs to the device and the
error metric used against the oracle.

Metric (the reading used throughout): for each (sequence, head) slice, the normwise
relative error max|gpu - ref| / max|ref|, maximised over slices.  A purely elementwise
relative error has no bound where ref crosses zero, so it is reported, not judged.
Bounds: 1e-5 for fp32 token inputs, 2e-3 for bf16 token inputs.
"""
from __future__ import annotations

import numpy as np
import torch

from speculative_decode_amd import synth

TOL = {synth.F32: 1e-5, synth.BF16: 2e-3}


def dev(t: synth.Tensor, device="cuda") -> torch.Tensor:
    if t.dtype == synth.BF16:
        return torch.from_numpy(np.ascontiguousarray(t.store).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.store)).to(device)


def dev_tokens(tok: synth.Tokens, device="cuda"):
    return dev(tok.x, device), dev(tok.B, device), dev(tok.C, device), dev(tok.dt, device)


def dev_layer(layer: synth.Layer, device="cuda"):
    return dev(layer.A, device), dev(layer.D, device)


def slice_err(gpu: np.ndarray, ref: np.ndarray, head_axis: int) -> float:
    """Max over (sequence, head) slices of max|g - r| / max|r|.  Arrays are
    [seq][...][H][...] with the head axis given."""
    g = np.moveaxis(np.asarray(gpu, dtype=np.float64), head_axis, 1)
    r = np.moveaxis(np.asarray(ref, dtype=np.float64), head_axis, 1)
    S, H = g.shape[0], g.shape[1]
    g = g.reshape(S, H, -1)
    r = r.reshape(S, H, -1)
    num = np.max(np.abs(g - r), axis=2)
    den = np.max(np.abs(r), axis=2)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def y_err(gpu_y, ref_y) -> float:
    return slice_err(gpu_y, ref_y, head_axis=2)       # y [seq][T][H][P]


def state_err(gpu_s, ref_s) -> float:
    return slice_err(gpu_s, ref_s, head_axis=1)       # state [seq][H][N][P]


def head_slice(tok: synth.Tokens, layer: synth.Layer, h: int, H: int, G: int):
    """Inputs of one head as a one-head, one-group problem (float64), for sampled checks."""
    g = h // (H // G)
    x = np.ascontiguousarray(tok.x.f64[:, :, h:h + 1])
    B = np.ascontiguousarray(tok.B.f64[:, :, g:g + 1])
    C = np.ascontiguousarray(tok.C.f64[:, :, g:g + 1])
    dt = np.ascontiguousarray(tok.dt.f64[:, :, h:h + 1])
    A = layer.A.f64[h:h + 1].copy()
    D = layer.D.f64[h:h + 1].copy()
    return x, B, C, dt, A, D
