"""Seeded synthetic inputs for the per-layer DP clip-and-accumulate step.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds no arithmetic of the method itself: it only draws activations,
output gradients, token masks and the like with numpy's PCG64 generator,
and rounds float32 draws to bfloat16 bit patterns (round to nearest even).

The shapes and value laws follow the workloads the FlashDP and DP-GRAPE
pages train on (Llama-13B layer widths 5120/13824, GPT-2-small 768/3072,
RoBERTa-large 1024/4096 at an SST-2-like length of 128).  No dataset or
trained weight is used: every tensor is Gaussian noise of the right shape.

Arrays are returned as numpy: float32 for fp32 workloads, uint16 bit
patterns for bf16 workloads (``dtype == "bf16"``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Linear", "Workload", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "dense_inputs", "config_c1", "config_c2", "config_c3", "config_c4",
    "config_c5", "C3_LINEARS", "C4_LINEARS", "C5_LINEARS", "LLAMA13B_HIDDEN",
    "LLAMA13B_FFN",
]

LLAMA13B_HIDDEN = 5120
LLAMA13B_FFN = 13824

# (name, din, dout) of the seven linears of one Llama-13B decoder layer.
C3_LINEARS: List[Tuple[str, int, int]] = [
    ("q", LLAMA13B_HIDDEN, LLAMA13B_HIDDEN),
    ("k", LLAMA13B_HIDDEN, LLAMA13B_HIDDEN),
    ("v", LLAMA13B_HIDDEN, LLAMA13B_HIDDEN),
    ("o", LLAMA13B_HIDDEN, LLAMA13B_HIDDEN),
    ("gate", LLAMA13B_HIDDEN, LLAMA13B_FFN),
    ("up", LLAMA13B_HIDDEN, LLAMA13B_FFN),
    ("down", LLAMA13B_FFN, LLAMA13B_HIDDEN),
]
C4_LINEARS = C3_LINEARS
# RoBERTa-large: d = 1024, d_ff = 4096.
C5_LINEARS: List[Tuple[str, int, int]] = [
    ("q", 1024, 1024), ("k", 1024, 1024), ("v", 1024, 1024), ("o", 1024, 1024),
    ("fc1", 1024, 4096), ("fc2", 4096, 1024),
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Linear:
    """One linear layer's inputs for one call."""
    name: str
    X: np.ndarray                 # [B, T, din]  float32 or uint16 (bf16 bits)
    G: np.ndarray                 # [B, T, dout] float32 or uint16 (bf16 bits)
    mask: Optional[np.ndarray]    # [B, T] uint8 or None
    C: float
    sigma: float
    seed: int
    offset: int
    dtype: str                    # "f32" or "bf16"

    @property
    def B(self) -> int:
        return int(self.X.shape[0])

    @property
    def T(self) -> int:
        return int(self.X.shape[1])

    @property
    def din(self) -> int:
        return int(self.X.shape[2])

    @property
    def dout(self) -> int:
        return int(self.G.shape[2])

    def active_tokens(self) -> int:
        if self.mask is None:
            return self.B * self.T
        return int(np.count_nonzero(self.mask))


@dataclass
class Workload:
    name: str
    linears: List[Linear]
    extra: Dict[str, object] = field(default_factory=dict)


def dense_inputs(rng: np.random.Generator, B: int, T: int, din: int, dout: int,
                 lognormal_sigma: float = 1.0, g_scale: float = 1e-3,
                 dtype: str = "bf16", s: Optional[np.ndarray] = None):
    """X ~ N(0,1); G_i = Z_i * s_i * g_scale with s_i = exp(lognormal_sigma * N(0,1)).

    Draw order: X, then Z, then s (unless ``s`` is given).  Returns (X, G) in
    the requested storage dtype.
    """
    X = rng.standard_normal((B, T, din), dtype=np.float32)
    Z = rng.standard_normal((B, T, dout), dtype=np.float32)
    if s is None:
        s = rng.lognormal(0.0, lognormal_sigma, B)
    scale = (np.asarray(s, dtype=np.float64) * g_scale).astype(np.float32)
    Z *= scale[:, None, None]
    if dtype == "bf16":
        return f32_to_bf16_bits(X), f32_to_bf16_bits(Z)
    return X, Z


def config_c1(sigma: float = 0.0) -> Workload:
    """Single fp32 linear: B=4, T=16, din=64, dout=32; X ~ N(0,1), G ~ N(0, 0.1^2), seed 0."""
    rng = np.random.default_rng(0)
    X = rng.standard_normal((4, 16, 64), dtype=np.float32)
    G = (0.1 * rng.standard_normal((4, 16, 32), dtype=np.float32)).astype(np.float32)
    lin = Linear("c1", X, G, None, 1.0, sigma, 0, 0, "f32")
    return Workload("c1_fp32_4x16x64to32", [lin])


def config_c2(sigma: float = 0.8, B: int = 32, T: int = 512) -> Workload:
    """GPT-2-small MLP up-projection 768 -> 3072, bf16, per-sample lognormal(0,1) G scale."""
    rng = np.random.default_rng(0)
    X, G = dense_inputs(rng, B, T, 768, 3072, 1.0)
    lin = Linear("up", X, G, None, 1.0, sigma, 0, 0, "bf16")
    return Workload("c2_gpt2_up_768x3072", [lin])


def config_c3_linear(index: int, B: int = 8, T: int = 2048, sigma: float = 1.0) -> Linear:
    """One Llama-13B-shaped linear (index into C3_LINEARS), numpy seed = index."""
    name, din, dout = C3_LINEARS[index]
    rng = np.random.default_rng(index)
    X, G = dense_inputs(rng, B, T, din, dout, 1.0)
    return Linear(name, X, G, None, 1.0, sigma, 0, 0, "bf16")


def config_c3(B: int = 8, T: int = 2048, which: Optional[List[int]] = None) -> Workload:
    which = list(range(len(C3_LINEARS))) if which is None else which
    return Workload("c3_llama13b_layer_B8_T2048",
                    [config_c3_linear(i, B, T) for i in which])


def ragged_lengths(B: int = 16, T: int = 2048, lo: int = 128):
    """T_i ~ Uniform{lo..T} (inclusive), prefix mask t < T_i, and the lognormal(0,2) scales."""
    rng = np.random.default_rng(0)
    lengths = rng.integers(lo, T + 1, B)
    s = rng.lognormal(0.0, 2.0, B)
    mask = (np.arange(T)[None, :] < lengths[:, None]).astype(np.uint8)
    return lengths, mask, s


def config_c4_linear(index: int, B: int = 16, T: int = 2048, lo: int = 128,
                     dims: Optional[Tuple[int, int]] = None) -> Linear:
    """One linear of the ragged Llama-13B decoder layer.

    Padded rows hold random non-zero values so that the mask is exercised.
    Per-linear numpy seed = 1000 + index; Philox offsets advance through the
    seven linears by ceil(din*dout/4) blocks each.
    """
    lengths, mask, s = ragged_lengths(B, T, lo)
    name, din, dout = C4_LINEARS[index]
    if dims is not None:
        din, dout = dims
    rng = np.random.default_rng(1000 + index)
    X, G = dense_inputs(rng, B, T, din, dout, s=s)
    offset = 0
    for j in range(index):
        _, dj, oj = C4_LINEARS[j]
        if dims is not None:
            dj, oj = dims
        offset += (dj * oj + 3) // 4
    return Linear(name, X, G, mask, 0.5, 1.2, 0, offset, "bf16")


def config_c4(B: int = 16, T: int = 2048, which: Optional[List[int]] = None) -> Workload:
    which = list(range(len(C4_LINEARS))) if which is None else which
    return Workload("c4_llama13b_ragged_B16_T2048",
                    [config_c4_linear(i, B, T) for i in which])


def config_c5_linear(index: int, B: int = 32, T: int = 128) -> Linear:
    """One RoBERTa-large linear for the projected variant (r = 256), numpy seed = index."""
    name, din, dout = C5_LINEARS[index]
    rng = np.random.default_rng(index)
    X, G = dense_inputs(rng, B, T, din, dout, 1.0)
    return Linear(name, X, G, None, 1.0, 1.0, 0, 0, "bf16")


def config_c5(B: int = 32, T: int = 128, which: Optional[List[int]] = None) -> Workload:
    which = list(range(len(C5_LINEARS))) if which is None else which
    return Workload("c5_roberta_large_projected_r256",
                    [config_c5_linear(i, B, T) for i in which],
                    extra={"r": 256, "proj_seed": 7, "proj_offset": 0})
