"""Oracle for the per-layer DP clip-and-accumulate step of one linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only the tests, the package's smoke check and the benchmark's CPU
baseline call it.  It shares no code with the GPU library.

What it computes (FlashDP: Private Training Large Language Models with
Efficient DP-SGD, Abstract: per-layer DP-SGD with per-sample gradient
clipping, whose result must match standard per-layer clipped DP-SGD;
Memory-Efficient Differentially Private Training with Gradient Random
Projection, English explainer, Problem Statement: each sample's gradient is
clipped before noise is added):

1. X~_i, G~_i: the rows of sample i whose token mask is 0 are *selected* to
   zero (never multiplied, so NaN in a padded row cannot leak).
2. g_i = G~_i^T X~_i, shape [dout, din], materialised one sample at a time
   in float64 (the explicit, Opacus-style method the FlashDP abstract
   contrasts with).
3. n_i = ||g_i||_F.
4. c_i = 1 if n_i <= C else C / n_i   (clip to norm C; no epsilon).
5. S = sum_i c_i g_i, summed in sample order.
6. out = (S + sigma * C * xi) / B, xi_e the Philox/Box-Muller normal of the
   row-major element index e (see oracle.philox), B = number of samples in
   the call including fully masked ones.

Projected variant (DP-GRAPE explainer, Methodology, "Order of Operations":
project the raw per-sample gradient first, then clip and add noise):
h_i = G~_i^T (X~_i P), shape [dout, r], with P [din, r]; steps 3-6 then run
on h_i.  Y_i = X~_i P is kept in float64.

Inputs are the exact values the GPU sees: bf16 bit patterns or float32,
widened to float64.  The readings taken where the pages are silent (gradient
orientation, clip rule, noise law and generator, denominator) are listed in
the repository's design notes.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import philox


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """bf16 bits (uint16) or float32 -> float64, exactly."""
    a = np.asarray(a)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 inputs are passed as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def select_active(rows: np.ndarray, mask_row: Optional[np.ndarray]) -> np.ndarray:
    """Rows whose mask entry is 0 become exactly 0 (selection, not a product)."""
    if mask_row is None:
        return rows
    keep = np.asarray(mask_row).astype(bool)
    return np.where(keep[:, None], rows, 0.0)


def per_sample_grad(Xi: np.ndarray, Gi: np.ndarray) -> np.ndarray:
    """g_i = G_i^T X_i for one sample: [T, dout]^T @ [T, din] -> [dout, din]."""
    return Gi.T @ Xi


def clip_factor(n: float, C: float) -> float:
    return 1.0 if n <= C else C / n


def noise_matrix(seed: int, offset: int, shape: Tuple[int, int]) -> np.ndarray:
    rows, cols = shape
    return philox.gaussian(seed, offset, rows * cols).reshape(rows, cols)


def clip_accumulate(per_sample, C: float):
    """Steps 3-5 over an iterable of per-sample gradients; returns (S, norms, c)."""
    S = None
    norms, factors = [], []
    for g in per_sample:
        n = float(np.sqrt(np.sum(g * g)))
        c = clip_factor(n, C)
        norms.append(n)
        factors.append(c)
        S = c * g if S is None else S + c * g
    return S, np.array(norms), np.array(factors)


def oracle_linear(X, G, mask, C: float, sigma: float, seed: int, offset: int,
                  dtype: str = "bf16", with_noise: bool = True, denom=None, out0=None):
    """Dense variant.  Returns (out [dout, din] f64, norms [B] f64, c [B] f64).

    out = (S + sigma C xi) / denom, denom = B unless given; with out0 (the
    buffer's previous contents) the result is added to it.  Each sample is
    still clipped on its own (FlashDP abstract: per-layer clipping of each
    sample's gradient), so the calls on the parts of a batch, each with the
    whole batch's size as denom and the noise in one of them, add up to the
    call on the whole batch."""
    Xw = widen(X, dtype)
    Gw = widen(G, dtype)
    B = Xw.shape[0]
    d = float(B if denom is None else denom)

    def grads():
        for i in range(B):
            m = None if mask is None else mask[i]
            yield per_sample_grad(select_active(Xw[i], m), select_active(Gw[i], m))

    S, norms, c = clip_accumulate(grads(), C)
    out = S.copy()
    if with_noise and sigma != 0.0:
        out = out + sigma * C * noise_matrix(seed, offset, S.shape)
    out = out / d
    if out0 is not None:
        out = np.asarray(out0, dtype=np.float64) + out
    return out, norms, c


def oracle_linear_bias(X, G, mask, C: float, sigma: float, seed: int, offset: int,
                       dtype: str = "bf16", with_noise: bool = True):
    """Dense variant for a linear with a bias, y = x W^T + b.

    The per-layer clipping of the FlashDP abstract applies to the layer's
    whole gradient, here the pair (g_i, gb_i) with gb_i = sum of the active
    rows of G_i (the weight gradient of a constant-one input).  Steps 3-5 run
    on the pair flattened into one vector.  Noise: the weight's xi from
    `offset`, the bias's continuing the stream at offset + ceil(dout*din/4).

    Returns (out_W [dout, din], out_b [dout], norms [B], c [B]), all float64."""
    Xw = widen(X, dtype)
    Gw = widen(G, dtype)
    B, din, dout = Xw.shape[0], Xw.shape[2], Gw.shape[2]

    def flat_grads():
        for i in range(B):
            m = None if mask is None else mask[i]
            Gi = select_active(Gw[i], m)
            g = per_sample_grad(select_active(Xw[i], m), Gi)
            yield np.concatenate([g.ravel(), Gi.sum(axis=0)])

    S, norms, c = clip_accumulate(flat_grads(), C)
    out_w = S[:dout * din].reshape(dout, din).copy()
    out_b = S[dout * din:].copy()
    if with_noise and sigma != 0.0:
        out_w = out_w + sigma * C * noise_matrix(seed, offset, (dout, din))
        out_b = out_b + sigma * C * philox.gaussian(seed, offset + (dout * din + 3) // 4, dout)
    return out_w / B, out_b / B, norms, c


def oracle_group(linears, mask, C: float, sigma: float, seed: int, offsets,
                 dtype: str = "bf16", with_noise: bool = True):
    """Group (joint) clipping over linears that see the same samples.

    The FlashDP abstract frames the method as per-layer clipping; clipping
    over a group of layers is the same procedure with sample i's gradient
    taken as the tuple (g_i^1, ..., g_i^L) of its per-layer gradients, whose
    norm is that of the tuple flattened into one vector -- standard (flat)
    DP-SGD restricted to those layers.  Steps 3-5 run on that vector; the
    sum is split back per linear, and linear l gets the noise of
    (seed, offsets[l]).

    linears: list of (X, G) pairs in the storage dtype, same B and T.
    Returns ([out_l [dout_l, din_l] f64], norms [B] f64, c [B] f64)."""
    widened = [(widen(X, dtype), widen(G, dtype)) for X, G in linears]
    B = widened[0][0].shape[0]
    shapes = [(Gw.shape[2], Xw.shape[2]) for Xw, Gw in widened]

    def flat_grads():
        for i in range(B):
            m = None if mask is None else mask[i]
            yield np.concatenate([
                per_sample_grad(select_active(Xw[i], m), select_active(Gw[i], m)).ravel()
                for Xw, Gw in widened])

    S, norms, c = clip_accumulate(flat_grads(), C)
    outs, at = [], 0
    for l, shape in enumerate(shapes):
        n = shape[0] * shape[1]
        o = S[at:at + n].reshape(shape).copy()
        at += n
        if with_noise and sigma != 0.0:
            o = o + sigma * C * noise_matrix(seed, offsets[l], shape)
        outs.append(o / B)
    return outs, norms, c


def projection_matrix(seed: int, offset: int, din: int, r: int, scale: float,
                      dtype: str = "bf16") -> np.ndarray:
    """P[d, j] = scale * xi_{d*r+j}(seed, offset) in the storage dtype (bf16
    bits rounded to nearest even, or float32): the seeded projection of the
    DP-GRAPE explainer (Methodology, random projections drawn again from their
    seed rather than stored).  The normals are this module's float64 ones
    rounded to float32 and scaled in float32, so a float32 generator may round
    a few entries to the neighbouring bf16 value; comparisons against one use
    a tolerance."""
    v = (np.float32(scale) * philox.gaussian(seed, offset, din * r).astype(np.float32))
    v = v.astype(np.float32).reshape(din, r)
    if dtype == "f32":
        return v
    u = v.view(np.uint32)
    out = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16))
    return out.astype(np.uint16)


def project_rows(Xi: np.ndarray, Pw: np.ndarray) -> np.ndarray:
    """Y_i = X~_i P (float64)."""
    return Xi @ Pw


def oracle_projected(X, G, mask, P, C: float, sigma: float, seed: int, offset: int,
                     dtype: str = "bf16", with_noise: bool = True):
    """Projected variant.  P is [din, r] in the inputs' storage dtype.

    Returns (out [dout, r] f64, norms [B] f64, c [B] f64)."""
    Xw = widen(X, dtype)
    Gw = widen(G, dtype)
    Pw = widen(P, dtype)
    B = Xw.shape[0]

    def grads():
        for i in range(B):
            m = None if mask is None else mask[i]
            Yi = project_rows(select_active(Xw[i], m), Pw)
            yield per_sample_grad(Yi, select_active(Gw[i], m))

    S, norms, c = clip_accumulate(grads(), C)
    out = S.copy()
    if with_noise and sigma != 0.0:
        out = out + sigma * C * noise_matrix(seed, offset, S.shape)
    return out / B, norms, c


def oracle_norms(X, G, mask, dtype: str = "bf16", samples=None) -> np.ndarray:
    """Pre-clip per-sample norms n_i only (for sampled checks at large sizes)."""
    Xw = widen(X, dtype) if samples is None else None
    B = X.shape[0]
    idx = range(B) if samples is None else samples
    out = []
    for i in idx:
        xi = widen(X[i], dtype) if Xw is None else Xw[i]
        gi = widen(G[i], dtype)
        m = None if mask is None else mask[i]
        g = per_sample_grad(select_active(xi, m), select_active(gi, m))
        out.append(float(np.sqrt(np.sum(g * g))))
    return np.array(out)


def oracle_entries(X, G, mask, c, rows, cols, sigma: float, C: float, seed: int,
                   offset: int, dtype: str = "bf16") -> np.ndarray:
    """Sampled output entries out[o, a] given the clip factors c (one by one).

    out[o, a] = (sum_i c_i sum_t G~[i,t,o] X~[i,t,a] + sigma C xi_{o*din+a}) / B.
    """
    B, _, din = X.shape
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    acc = np.zeros(len(rows), dtype=np.float64)
    for i in range(B):
        m = None if mask is None else mask[i]
        xi = select_active(widen(X[i][:, cols], dtype), m)      # [T, k]
        gi = select_active(widen(G[i][:, rows], dtype), m)      # [T, k]
        acc += c[i] * np.sum(gi * xi, axis=0)
    if sigma != 0.0:
        e = rows.astype(np.uint64) * np.uint64(din) + cols.astype(np.uint64)
        acc = acc + sigma * C * philox.gaussian_at(seed, offset, e)
    return acc / B


def brute_force_linear(X, G, mask, C: float):
    """Steps 2-5 as explicit loops in pure Python (tiny inputs only).

    X, G are nested lists / arrays of Python floats already widened.
    Returns (S as list of lists, norms list).
    """
    B = len(X)
    T = len(X[0])
    din = len(X[0][0])
    dout = len(G[0][0])
    S = [[0.0] * din for _ in range(dout)]
    norms = []
    for i in range(B):
        g = [[0.0] * din for _ in range(dout)]
        for o in range(dout):
            for a in range(din):
                s = 0.0
                for t in range(T):
                    if mask is not None and not mask[i][t]:
                        continue
                    s += float(G[i][t][o]) * float(X[i][t][a])
                g[o][a] = s
        n = 0.0
        for o in range(dout):
            for a in range(din):
                n += g[o][a] * g[o][a]
        n = n ** 0.5
        c = 1.0 if n <= C else C / n
        norms.append(n)
        for o in range(dout):
            for a in range(din):
                S[o][a] += c * g[o][a]
    return S, norms
