"""Per-layer DP-SGD clip-and-accumulate for linear layers on AMD MI355X.

Python binding of libdpfused (include/dpfused.h).  This module only
marshals arguments: torch tensors provide device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.

    grad, norms = linear_clip_accumulate(X, G, mask=None, C=1.0, sigma=1.0,
                                         seed=0, offset=0)

computes, for X [B, T, din] and G [B, T, dout] (bf16 or fp32, on the GPU),
grad = (sum_i c_i G~_i^T X~_i + sigma C xi) / B with c_i = min(1, C/||g_i||),
and the pre-clip per-sample norms.  See include/dpfused.h for the contract.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

from . import _lib
from ._lib import DpfAct, DpfError, DPF_BF16, DPF_F32  # noqa: F401

__all__ = [
    "linear_clip_accumulate", "linear_clip_accumulate_noalloc", "linear_clip_accumulate_projected",
    "linear_clip_accumulate_projected_seeded", "linear_clip_accumulate_bias", "project",
    "group_clip_accumulate", "consecutive_offsets", "projected_adam_step",
    "linear_clip_accumulate_projected_many",
    "per_sample_sqnorms",
    "clip_factors", "scaled_accumulate", "philox4x32_10", "gaussian_fill", "noise_blocks",
    "set_option", "get_option", "timing_reset", "timing_collect", "DpfError", "load",
]


def load():
    """Load libdpfused (raises ImportError if it has not been built)."""
    return _lib.lib()


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DPF_BF16
    if t.dtype == torch.float32:
        return DPF_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _act(t) -> DpfAct:
    if t.dim() != 3:
        raise ValueError("activations must be [B, T, D]")
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if t.stride(2) != 1:
        raise ValueError("the last dimension must be contiguous")
    B, T, D = t.shape
    return DpfAct(t.data_ptr(), _dtype_code(t), 0, B, T, D, t.stride(0), t.stride(1))


def _stream(t, stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _mask_ptr(mask, B, T, device=None) -> Optional[int]:
    if mask is None:
        return None
    torch = _torch()
    if mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError("mask must be uint8 or bool")
    if tuple(mask.shape) != (B, T) or not mask.is_contiguous() or not mask.is_cuda:
        raise ValueError("mask must be a contiguous [B, T] GPU tensor")
    if device is not None and mask.device != device:
        raise ValueError(f"mask is on {mask.device}, the activations on {device}")
    return mask.data_ptr()


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _same_device(t, device, name: str) -> None:
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the activations on {device}")


def _check_out(t, shape, name: str, device, dtype=None) -> None:
    """A caller-supplied output: a contiguous tensor of exactly ``shape`` and
    ``dtype`` (float32 unless given) on ``device``.  The library writes it
    through a raw pointer, so anything else would be written out of bounds or
    in the wrong layout."""
    torch = _torch()
    dtype = torch.float32 if dtype is None else dtype
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the activations on {device}")


def _pair(X, G):
    """Descriptors of X [B, T, din] and G [B, T, dout] on one device."""
    xa, ga = _act(X), _act(G)
    _same_device(G, X.device, "G")
    return xa, ga


def linear_clip_accumulate(X, G, mask=None, C: float = 1.0, sigma: float = 0.0, seed: int = 0,
                           offset: int = 0, grad_out=None, norms_out=None, stream=None,
                           want_norms: bool = True, denom: Optional[float] = None,
                           accumulate: bool = False) -> Tuple[object, object]:
    """Fused per-layer DP step; returns (grad_out [dout, din] fp32, norms [B] fp32 or None).

    denom (default B) divides the noisy clipped sum; accumulate=True adds the
    result into grad_out (which must then be given) instead of overwriting it."""
    torch = _torch()
    xa, ga = _pair(X, G)
    B, T = X.shape[0], X.shape[1]
    if accumulate and grad_out is None:
        raise ValueError("accumulate=True needs grad_out")
    if grad_out is None:
        grad_out = torch.empty((G.shape[2], X.shape[2]), dtype=torch.float32, device=X.device)
    _check_out(grad_out, (G.shape[2], X.shape[2]), "grad_out", X.device)
    if norms_out is None and want_norms:
        norms_out = torch.empty((B,), dtype=torch.float32, device=X.device)
    if norms_out is not None:
        _check_out(norms_out, (B,), "norms_out", X.device)
    mp = _mask_ptr(mask, B, T, X.device)
    if denom is None and not accumulate:
        st = _lib.lib().dpfused_linear_clip_accumulate(
            ctypes.byref(xa), ctypes.byref(ga), mp, float(C), float(sigma),
            int(seed), int(offset), grad_out.data_ptr(), _ptr(norms_out), _stream(X, stream))
    else:
        st = _lib.lib().dpfused_linear_clip_accumulate_ex(
            ctypes.byref(xa), ctypes.byref(ga), mp, float(C), float(sigma),
            int(seed), int(offset), float(B if denom is None else denom), int(bool(accumulate)),
            grad_out.data_ptr(), _ptr(norms_out), _stream(X, stream))
    _lib.check(st)
    return grad_out, norms_out


def linear_clip_accumulate_noalloc(X, G, grad_out, mask=None, C: float = 1.0,
                                   sigma: float = 0.0, seed: int = 0, offset: int = 0,
                                   norms_out=None, stream=None):
    """linear_clip_accumulate without any device allocation, for code under graph
    capture or loops that must not allocate: the library works in its static per-GPU
    scratch, and this wrapper allocates nothing either (grad_out [dout, din] fp32 must
    be given; norms_out [B] fp32 or None).  Calls that overlap in time on one GPU race
    on the scratch: keep them ordered."""
    xa, ga = _pair(X, G)
    B, T = X.shape[0], X.shape[1]
    _check_out(grad_out, (G.shape[2], X.shape[2]), "grad_out", X.device)
    if norms_out is not None:
        _check_out(norms_out, (B,), "norms_out", X.device)
    st = _lib.lib().dpfused_linear_clip_accumulate_noalloc(
        ctypes.byref(xa), ctypes.byref(ga), _mask_ptr(mask, B, T, X.device), float(C),
        float(sigma), int(seed), int(offset), grad_out.data_ptr(), _ptr(norms_out),
        _stream(X, stream))
    _lib.check(st)
    return grad_out, norms_out


def linear_clip_accumulate_projected(X, G, P, mask=None, C: float = 1.0, sigma: float = 0.0,
                                     seed: int = 0, offset: int = 0, grad_out=None,
                                     norms_out=None, stream=None, want_norms: bool = True):
    """Projected variant: clip/sum/noise of G~_i^T (X~_i P); returns ([dout, r], norms)."""
    torch = _torch()
    xa, ga = _pair(X, G)
    B, T = X.shape[0], X.shape[1]
    if P.dim() != 2 or not P.is_contiguous() or P.shape[0] != X.shape[2] or P.dtype != X.dtype:
        raise ValueError("P must be a contiguous [din, r] tensor of X's dtype")
    _same_device(P, X.device, "P")
    r = P.shape[1]
    if grad_out is None:
        grad_out = torch.empty((G.shape[2], r), dtype=torch.float32, device=X.device)
    _check_out(grad_out, (G.shape[2], r), "grad_out", X.device)
    if norms_out is None and want_norms:
        norms_out = torch.empty((B,), dtype=torch.float32, device=X.device)
    if norms_out is not None:
        _check_out(norms_out, (B,), "norms_out", X.device)
    st = _lib.lib().dpfused_linear_clip_accumulate_projected(
        ctypes.byref(xa), ctypes.byref(ga), _mask_ptr(mask, B, T, X.device), P.data_ptr(), int(r),
        float(C), float(sigma), int(seed), int(offset), grad_out.data_ptr(), _ptr(norms_out),
        _stream(X, stream))
    _lib.check(st)
    return grad_out, norms_out


def linear_clip_accumulate_projected_many(Xs, Gs, Ps, masks=None, C: float = 1.0,
                                          sigma: float = 0.0, seed: int = 0, offsets=None,
                                          grad_outs=None, norms_outs=None, stream=None,
                                          want_norms: bool = True):
    """Several independent projected calls (each linear clipped on its own) queued
    together on the library's streams, so that their launches overlap; each result is
    bitwise that of linear_clip_accumulate_projected.  Ps are [din_l, r] (one r for
    all); returns ([grad_out per call], [norms per call]).

    offsets (Philox block offsets, one per call) default to consecutive disjoint ranges
    from 0: offsets[l] = sum over k < l of noise_blocks(dout_k * r)."""
    torch = _torch()
    n = len(Xs)
    if n < 1 or len(Gs) != n or len(Ps) != n:
        raise ValueError("Xs, Gs and Ps must be non-empty lists of the same length")
    dev = Xs[0].device
    pairs = [_pair(x, g) for x, g in zip(Xs, Gs)]
    for x, g in zip(Xs, Gs):
        _same_device(x, dev, "every X")
        _same_device(g, dev, "every G")
    r = Ps[0].shape[1] if Ps[0].dim() == 2 else -1
    for l, (x, P) in enumerate(zip(Xs, Ps)):
        if P.dim() != 2 or not P.is_contiguous() or P.shape[0] != x.shape[2] or P.dtype != x.dtype \
                or P.shape[1] != r:
            raise ValueError(f"Ps[{l}] must be a contiguous [din, r] tensor of X's dtype, "
                             "with the same r for every call")
        _same_device(P, dev, f"Ps[{l}]")
    masks = [None] * n if masks is None else list(masks)
    if len(masks) != n:
        raise ValueError(f"masks must have one entry per call ({n}), got {len(masks)}")
    if offsets is None:
        offsets = consecutive_offsets([(int(g.shape[2]), int(r)) for g in Gs])
    offsets = list(offsets)
    if len(offsets) != n:
        raise ValueError(f"offsets must have one entry per call ({n}), got {len(offsets)}")
    if grad_outs is None:
        grad_outs = [torch.empty((g.shape[2], r), dtype=torch.float32, device=dev) for g in Gs]
    grad_outs = list(grad_outs)
    if len(grad_outs) != n:
        raise ValueError(f"grad_outs must have one tensor per call ({n}), got {len(grad_outs)}")
    for l, (o, g) in enumerate(zip(grad_outs, Gs)):
        _check_out(o, (g.shape[2], r), f"grad_outs[{l}]", dev)
    if norms_outs is None:
        norms_outs = [torch.empty((x.shape[0],), dtype=torch.float32, device=dev) if want_norms
                      else None for x in Xs]
    norms_outs = list(norms_outs)
    if len(norms_outs) != n:
        raise ValueError(f"norms_outs must have one entry per call ({n}), got {len(norms_outs)}")
    for l, (nrm, x) in enumerate(zip(norms_outs, Xs)):
        if nrm is not None:
            _check_out(nrm, (x.shape[0],), f"norms_outs[{l}]", dev)
    acts = (DpfAct * n)(*[a for a, _ in pairs])
    gacts = (DpfAct * n)(*[b for _, b in pairs])
    mptrs = (ctypes.c_void_p * n)(*[_mask_ptr(m, x.shape[0], x.shape[1], dev)
                                    for m, x in zip(masks, Xs)])
    pptrs = (ctypes.c_void_p * n)(*[P.data_ptr() for P in Ps])
    offs = (ctypes.c_uint64 * n)(*[int(o) for o in offsets])
    outs = (ctypes.c_void_p * n)(*[o.data_ptr() for o in grad_outs])
    nptrs = (ctypes.c_void_p * n)(*[_ptr(nrm) for nrm in norms_outs])
    st = _lib.lib().dpfused_linear_clip_accumulate_projected_many(
        n, acts, gacts, mptrs, pptrs, int(r), float(C), float(sigma), int(seed), offs, outs, nptrs,
        _stream(Xs[0], stream))
    _lib.check(st)
    return grad_outs, norms_outs


def project(X, P, mask=None, out=None, stream=None):
    """The projection step alone: Y = X~ P ([B, T, r], X's dtype; masked rows zero),
    as the projected calls form it."""
    torch = _torch()
    xa = _act(X)
    B, T = X.shape[0], X.shape[1]
    if P.dim() != 2 or not P.is_contiguous() or P.shape[0] != X.shape[2] or P.dtype != X.dtype:
        raise ValueError("P must be a contiguous [din, r] tensor of X's dtype")
    _same_device(P, X.device, "P")
    r = P.shape[1]
    if out is None:
        out = torch.empty((B, T, r), dtype=X.dtype, device=X.device)
    _check_out(out, (B, T, r), "out", X.device, dtype=X.dtype)
    st = _lib.lib().dpfused_project(ctypes.byref(xa), _mask_ptr(mask, B, T, X.device), P.data_ptr(),
                                    int(r), out.data_ptr(), _stream(X, stream))
    _lib.check(st)
    return out


def linear_clip_accumulate_projected_seeded(X, G, r: int, mask=None, p_seed: int = 0,
                                            p_offset: int = 0, p_scale=None, C: float = 1.0,
                                            sigma: float = 0.0, seed: int = 0, offset: int = 0,
                                            grad_out=None, norms_out=None, stream=None,
                                            want_norms: bool = True):
    """Projected variant with P[d, j] = p_scale * xi_{d*r+j}(p_seed, p_offset) drawn in the
    call and not kept (see the "p_in_kernels" option).  p_scale=None lets the library
    take the method's default, 1/sqrt(r).  With sigma > 0 the noise (seed, offset) must
    not draw P's Philox blocks: the library rejects an overlap under one seed."""
    torch = _torch()
    xa, ga = _pair(X, G)
    B, T = X.shape[0], X.shape[1]
    if p_scale is None:
        p_scale = math.nan
    if grad_out is None:
        grad_out = torch.empty((G.shape[2], r), dtype=torch.float32, device=X.device)
    _check_out(grad_out, (G.shape[2], r), "grad_out", X.device)
    if norms_out is None and want_norms:
        norms_out = torch.empty((B,), dtype=torch.float32, device=X.device)
    if norms_out is not None:
        _check_out(norms_out, (B,), "norms_out", X.device)
    st = _lib.lib().dpfused_linear_clip_accumulate_projected_seeded(
        ctypes.byref(xa), ctypes.byref(ga), _mask_ptr(mask, B, T, X.device), int(r), int(p_seed),
        int(p_offset), float(p_scale), float(C), float(sigma), int(seed), int(offset),
        grad_out.data_ptr(), _ptr(norms_out), _stream(X, stream))
    _lib.check(st)
    return grad_out, norms_out


def linear_clip_accumulate_bias(X, G, mask=None, C: float = 1.0, sigma: float = 0.0,
                                seed: int = 0, offset: int = 0, grad_out=None, bias_grad_out=None,
                                norms_out=None, stream=None, want_norms: bool = True):
    """Dense step for a linear with a bias: weight and bias gradients clipped together;
    returns (grad_out [dout, din], bias_grad_out [dout], norms [B])."""
    torch = _torch()
    xa, ga = _pair(X, G)
    B, T = X.shape[0], X.shape[1]
    if grad_out is None:
        grad_out = torch.empty((G.shape[2], X.shape[2]), dtype=torch.float32, device=X.device)
    _check_out(grad_out, (G.shape[2], X.shape[2]), "grad_out", X.device)
    if bias_grad_out is None:
        bias_grad_out = torch.empty((G.shape[2],), dtype=torch.float32, device=X.device)
    _check_out(bias_grad_out, (G.shape[2],), "bias_grad_out", X.device)
    if norms_out is None and want_norms:
        norms_out = torch.empty((B,), dtype=torch.float32, device=X.device)
    if norms_out is not None:
        _check_out(norms_out, (B,), "norms_out", X.device)
    st = _lib.lib().dpfused_linear_clip_accumulate_bias(
        ctypes.byref(xa), ctypes.byref(ga), _mask_ptr(mask, B, T, X.device), float(C), float(sigma),
        int(seed), int(offset), grad_out.data_ptr(), bias_grad_out.data_ptr(), _ptr(norms_out),
        _stream(X, stream))
    _lib.check(st)
    return grad_out, bias_grad_out, norms_out


def consecutive_offsets(shapes, start: int = 0):
    """Philox offsets that give each output of ``shapes`` ([(rows, cols), ...]) its own
    consecutive block range: offsets[l] = start + sum over k < l of ceil(rows_k cols_k / 4)
    (four normals per block), so that no two outputs share noise."""
    out, at = [], int(start)
    for rows, cols in shapes:
        out.append(at)
        at += (int(rows) * int(cols) + 3) // 4
    return out


def group_clip_accumulate(Xs, Gs, mask=None, C: float = 1.0, sigma: float = 0.0, seed: int = 0,
                          offsets=None, grad_outs=None, norms_out=None, stream=None,
                          want_norms: bool = True):
    """Joint clipping over linears that see the same samples: one c_i from the norm of
    sample i's gradient over all of them; returns ([grad_out per linear], norms).

    offsets (Philox block offsets, one per linear) default to consecutive disjoint ranges
    from 0: offsets[l] = sum over k < l of noise_blocks(dout_k * din_k), so that no two
    linears share noise."""
    torch = _torch()
    n = len(Xs)
    if n < 1 or len(Gs) != n:
        raise ValueError("Xs and Gs must be non-empty lists of the same length")
    dev = Xs[0].device
    for x, g in zip(Xs, Gs):
        _same_device(x, dev, "every X")
        _same_device(g, dev, "every G")
    acts = (DpfAct * n)(*[_act(x) for x in Xs])
    gacts = (DpfAct * n)(*[_act(g) for g in Gs])
    B, T = Xs[0].shape[0], Xs[0].shape[1]
    if offsets is None:
        offsets = consecutive_offsets([(int(g.shape[2]), int(x.shape[2])) for x, g in zip(Xs, Gs)])
    offsets = list(offsets)
    if len(offsets) != n:
        raise ValueError(f"offsets must have one entry per linear ({n}), got {len(offsets)}")
    if grad_outs is None:
        grad_outs = [torch.empty((g.shape[2], x.shape[2]), dtype=torch.float32, device=x.device)
                     for x, g in zip(Xs, Gs)]
    grad_outs = list(grad_outs)
    if len(grad_outs) != n:
        raise ValueError(f"grad_outs must have one tensor per linear ({n}), got {len(grad_outs)}")
    for l, (o, x, g) in enumerate(zip(grad_outs, Xs, Gs)):
        _check_out(o, (g.shape[2], x.shape[2]), f"grad_outs[{l}]", dev)
    if norms_out is None and want_norms:
        norms_out = torch.empty((B,), dtype=torch.float32, device=dev)
    if norms_out is not None:
        _check_out(norms_out, (B,), "norms_out", dev)
    offs = (ctypes.c_uint64 * n)(*[int(o) for o in offsets])
    outs = (ctypes.c_void_p * n)(*[o.data_ptr() for o in grad_outs])
    st = _lib.lib().dpfused_group_clip_accumulate(
        n, acts, gacts, _mask_ptr(mask, B, T, dev), float(C), float(sigma), int(seed), offs, outs,
        _ptr(norms_out), _stream(Xs[0], stream))
    _lib.check(st)
    return grad_outs, norms_out


def projected_adam_step(grad, m, v, W, step: int, lr: float, beta1: float = 0.9,
                        beta2: float = 0.999, eps: float = 1e-8, P=None, p_seed: int = 0,
                        p_offset: int = 0, p_scale=None, p_dtype=None, stream=None):
    """One projected Adam step: m, v ([dout, r] fp32) and W ([dout, din] fp32) are updated
    in place from the privatised projected gradient ``grad`` [dout, r]; P [din, r], or
    None to draw it from (p_seed, p_offset, p_scale) in p_dtype (default bf16)."""
    torch = _torch()
    dout, r = grad.shape
    din = W.shape[1]
    for t, name in ((grad, "grad"), (m, "m"), (v, "v"), (W, "W")):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    if tuple(m.shape) != (dout, r) or tuple(v.shape) != (dout, r) or W.shape[0] != dout:
        raise ValueError("m and v must be [dout, r] and W [dout, din]")
    for t, name in ((m, "m"), (v, "v"), (W, "W")):
        _same_device(t, grad.device, name)
    if P is not None:
        if P.dim() != 2 or tuple(P.shape) != (din, r) or not P.is_contiguous():
            raise ValueError("P must be a contiguous [din, r] tensor")
        _same_device(P, grad.device, "P")
        pdt = _dtype_code(P)
        pptr = P.data_ptr()
    else:
        pdt = _dtype_code(torch.empty(0, dtype=p_dtype or torch.bfloat16))
        pptr = None
    # None: the library's default for a seeded P, 1/sqrt(r)
    scale = math.nan if p_scale is None else float(p_scale)
    st = _lib.lib().dpfused_projected_adam_step(
        grad.data_ptr(), m.data_ptr(), v.data_ptr(), W.data_ptr(), int(dout), int(din), int(r),
        int(step), float(lr), float(beta1), float(beta2), float(eps), pptr, int(pdt),
        int(p_seed), int(p_offset), scale, _stream(grad, stream))
    _lib.check(st)
    return m, v, W


def per_sample_sqnorms(X, G, mask=None, out=None, accumulate: bool = False, stream=None):
    """||G~_i^T X~_i||^2 per sample (fp64 [B]); with accumulate=True, added into ``out``."""
    torch = _torch()
    xa, ga = _pair(X, G)
    B, T = X.shape[0], X.shape[1]
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an out tensor")
        out = torch.empty((B,), dtype=torch.float64, device=X.device)
    _check_out(out, (B,), "out", X.device, torch.float64)
    st = _lib.lib().dpfused_per_sample_sqnorms(ctypes.byref(xa), ctypes.byref(ga),
                                               _mask_ptr(mask, B, T, X.device), out.data_ptr(),
                                               1 if accumulate else 0, _stream(X, stream))
    _lib.check(st)
    return out


def clip_factors(sqnorms, C: float, c_out=None, norms_out=None, stream=None):
    """c = min(1, C / sqrt(sqnorms)) (fp32) and the norms, from fp64 squared norms."""
    torch = _torch()
    if sqnorms.dtype != torch.float64 or not sqnorms.is_contiguous() or not sqnorms.is_cuda:
        raise ValueError("sqnorms must be a contiguous float64 GPU tensor")
    n = sqnorms.numel()
    if c_out is None:
        c_out = torch.empty((n,), dtype=torch.float32, device=sqnorms.device)
    _check_out(c_out, (n,), "c_out", sqnorms.device)
    if norms_out is not None:
        _check_out(norms_out, (n,), "norms_out", sqnorms.device)
    st = _lib.lib().dpfused_clip_factors(sqnorms.data_ptr(), int(n), float(C), c_out.data_ptr(),
                                         _ptr(norms_out), _stream(sqnorms, stream))
    _lib.check(st)
    return c_out, norms_out


def scaled_accumulate(X, G, c, mask=None, noise_std: float = 0.0, seed: int = 0, offset: int = 0,
                      grad_out=None, stream=None):
    """(sum_i c_i G~_i^T X~_i + noise_std xi) / B for given fp32 factors c [B]."""
    torch = _torch()
    xa, ga = _pair(X, G)
    B, T = X.shape[0], X.shape[1]
    _check_out(c, (B,), "c", X.device)
    if grad_out is None:
        grad_out = torch.empty((G.shape[2], X.shape[2]), dtype=torch.float32, device=X.device)
    _check_out(grad_out, (G.shape[2], X.shape[2]), "grad_out", X.device)
    st = _lib.lib().dpfused_scaled_accumulate(ctypes.byref(xa), ctypes.byref(ga),
                                              _mask_ptr(mask, B, T, X.device), c.data_ptr(),
                                              float(noise_std), int(seed), int(offset),
                                              grad_out.data_ptr(), _stream(X, stream))
    _lib.check(st)
    return grad_out


def philox4x32_10(seed: int, offset: int, nblocks: int, out=None, device="cuda", stream=None):
    """Raw Philox4x32-10 words as an int32 tensor [nblocks, 4] (bit patterns of uint32)."""
    torch = _torch()
    if out is None:
        out = torch.empty((max(nblocks, 0), 4), dtype=torch.int32, device=device)
    if not out.is_cuda:
        raise ValueError("out must be a GPU tensor")
    _check_out(out, (max(nblocks, 0), 4), "out", out.device, torch.int32)
    st = _lib.lib().dpfused_philox4x32_10(int(seed), int(offset), int(nblocks), out.data_ptr(),
                                          _stream(out, stream))
    _lib.check(st)
    return out


def gaussian_fill(seed: int, offset: int, n: int, scale: float = 1.0, dtype=None, out=None,
                  device="cuda", stream=None):
    """scale * xi_e for e < n, as float32 or bfloat16 (rounded from the fp32 product)."""
    torch = _torch()
    dtype = torch.float32 if dtype is None else dtype
    if out is None:
        out = torch.empty((max(n, 0),), dtype=dtype, device=device)
    if not out.is_cuda:
        raise ValueError("out must be a GPU tensor")
    if out.dtype not in (torch.float32, torch.bfloat16) or not out.is_contiguous() \
            or out.numel() < max(n, 0):
        raise ValueError("out must be a contiguous float32 or bfloat16 tensor of at least n values")
    st = _lib.lib().dpfused_gaussian_fill(int(seed), int(offset), int(n), float(scale),
                                          _dtype_code(out), out.data_ptr(), _stream(out, stream))
    _lib.check(st)
    return out


def noise_blocks(n_elements: int) -> int:
    return int(_lib.lib().dpfused_noise_blocks(int(n_elements)))


def set_option(name: str, value: int) -> None:
    _lib.check(_lib.lib().dpfused_set_option(name.encode(), int(value)))


def get_option(name: str) -> int:
    return int(_lib.lib().dpfused_get_option(name.encode()))


def timing_reset() -> None:
    _lib.lib().dpfused_timing_reset()


def timing_collect() -> dict:
    """{kernel name: (total ms, launches)} of the event pairs recorded since the last reset."""
    L = _lib.lib()
    n = L.dpfused_timing_collect()
    return {L.dpfused_timing_name(k).decode(): (L.dpfused_timing_total_ms(k),
                                                 int(L.dpfused_timing_launches(k)))
            for k in range(n)}
