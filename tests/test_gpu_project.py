"""GPU parity of the projection step alone, Y = X~ P (dpfused_project), the
first step of the projected variant -- against the oracle's fp64 product.

Bar, element by element: the GPU forms each entry as an fp32 sum of din
exact bf16 x bf16 products (any order) and rounds it once to bf16, so

    |Y - Y_ref| <= 2^-8 |Y_ref| + din 2^-23 (|X~| |P|)[t, j]

(half an ulp of bf16 is 2^-9 relative; the fp32 sum of din terms is within
din 2^-24 of the sum of their magnitudes, doubled for slack).  Masked rows
are exactly zero.  Shapes cover the RoBERTa-large linears (din 1024 and
4096, r = 256, 4096 tokens), ragged tails in every dimension (tokens, din
and r not multiples of the 64-wide tile), a strided view, masks with an
empty sample, r = 8 and a single token; fp32 inputs take the generic tiles.
Also: bitwise repeatability, and the projected call's own Y equals this one
(the projected sum with P = I on the first r features equals the dense sum
over those features).  The multi-linear projected call equals the single
calls bit for bit for every number of library streams and with the staged
fallback, and its graph replays equal its eager result.
"""
import numpy as np
import pytest

import workloads
from oracle import dp_linear
from tests.gpu_helpers import mask_dev, need_gpu, to_dev

pytestmark = pytest.mark.gpu


def _bf16_to_f64(bits):
    return workloads.bf16_bits_to_f32(np.ascontiguousarray(bits)).astype(np.float64)


def _inputs(rng, B, T, din, r, dtype):
    X = rng.standard_normal((B, T, din), dtype=np.float32)
    P = (rng.standard_normal((din, r)) / np.sqrt(r)).astype(np.float32)
    if dtype == "bf16":
        return workloads.f32_to_bf16_bits(X), workloads.f32_to_bf16_bits(P)
    return X, P


def _reference(X, P, mask, dtype):
    """Y_ref = X~ P (fp64) and the magnitude sum |X~| |P| per entry."""
    Xw = dp_linear.widen(X, dtype)
    Pw = dp_linear.widen(P, dtype)
    B, T, _ = Xw.shape
    Y = np.zeros((B, T, Pw.shape[1]))
    A = np.zeros_like(Y)
    for b in range(B):
        Xb = Xw[b].copy()
        if mask is not None:
            Xb[mask[b] == 0] = 0.0
        Y[b] = dp_linear.project_rows(Xb, Pw)
        A[b] = np.abs(Xb) @ np.abs(Pw)
    return Y, A


def _check(Yg, X, P, mask, dtype):
    Yref, A = _reference(X, P, mask, dtype)
    din = X.shape[2]
    got = _bf16_to_f64(Yg.view(np.uint16)) if dtype == "bf16" else Yg.astype(np.float64)
    if dtype == "bf16":
        tol = 2.0 ** -8 * np.abs(Yref) + din * 2.0 ** -23 * A
    else:
        tol = din * 2.0 ** -23 * A + 1e-30
    err = np.abs(got - Yref)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), (f"max excess at {worst}: |got - ref| = {err[worst]:.3e}, "
                                f"bound {tol[worst]:.3e}")
    if mask is not None:
        assert np.all(got[mask == 0] == 0.0)


def _run(torch, X, P, mask, dtype, Xview=None):
    import sample_gradient_clipping_amd as dp
    Xd = to_dev(X, dtype, torch) if Xview is None else Xview
    Pd = to_dev(P, dtype, torch)
    dp.timing_reset()
    dp.set_option("timing", 1)
    try:
        Y = dp.project(Xd, Pd, mask_dev(mask, torch))
        torch.cuda.synchronize()
        kernels = dp.timing_collect()
    finally:
        dp.set_option("timing", 0)
        dp.timing_reset()
    out = Y.cpu()
    return (out.view(torch.int16).numpy() if dtype == "bf16" else out.numpy()), kernels


@pytest.mark.parametrize("shape,lengths", [
    ((32, 128, 1024, 256), None),            # RoBERTa-large q/k/v/o/fc1 input
    ((32, 128, 4096, 256), None),            # RoBERTa-large fc2 input
    ((3, 75, 200, 72), [75, 10, 0]),         # ragged everywhere, an empty sample
    ((1, 130, 136, 40), None),               # 3 token tiles, r < one tile
    ((1, 70, 392, 136), None),               # 7 K steps (more than the ring), 3 r tiles
    ((2, 1, 8, 8), None),                    # one token per sample, r = 8
])
def test_projection_bf16_matches_oracle(shape, lengths):
    torch = need_gpu()
    B, T, din, r = shape
    rng = np.random.default_rng(sum(shape))
    X, P = _inputs(rng, B, T, din, r, "bf16")
    mask = None
    if lengths is not None:
        mask = (np.arange(T)[None, :] < np.asarray(lengths)[:, None]).astype(np.uint8)
    Y, kernels = _run(torch, X, P, mask, "bf16")
    assert "project" in kernels and "project_reduce" not in kernels, sorted(kernels)
    _check(Y, X, P, mask, "bf16")


def test_projection_random_mask_and_strided_view():
    torch = need_gpu()
    rng = np.random.default_rng(31)
    B, T, din, r = 2, 33, 72, 8
    X, P = _inputs(rng, B, T, din, r, "bf16")
    mask = (rng.random((B, T)) < 0.6).astype(np.uint8)
    wide = np.zeros((B, T, 96), np.uint16)
    wide[:, :, :din] = X
    view = to_dev(wide, "bf16", torch)[:, :, :din]
    Y, _ = _run(torch, X, P, mask, "bf16", Xview=view)
    _check(Y, X, P, mask, "bf16")


@pytest.mark.parametrize("shape", [(3, 75, 200, 72), (2, 64, 1024, 256)])
def test_projection_fp32_generic_tiles(shape):
    torch = need_gpu()
    B, T, din, r = shape
    rng = np.random.default_rng(sum(shape) + 1)
    X, P = _inputs(rng, B, T, din, r, "f32")
    mask = (np.arange(T)[None, :] < np.array([T, T // 3, 0][:B])[:, None]).astype(np.uint8)
    Y, _ = _run(torch, X, P, mask, "f32")
    _check(Y, X, P, mask, "f32")


def test_projection_is_bitwise_repeatable():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(32)
    X, P = _inputs(rng, 8, 128, 1024, 256, "bf16")
    Xd, Pd = to_dev(X, "bf16", torch), to_dev(P, "bf16", torch)
    ref = dp.project(Xd, Pd)
    for _ in range(5):
        assert torch.equal(dp.project(Xd, Pd), ref)


def test_projected_call_uses_the_same_projection():
    """With P = [I_r; 0] the projection keeps the first r features, so the
    projected call must equal the dense call on X[:, :, :r] (bitwise: the
    same kernels see the same Y), and dpfused_project returns that Y."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(33)
    B, T, din, dout, r = 4, 100, 264, 136, 64
    X, _ = _inputs(rng, B, T, din, r, "bf16")
    G = workloads.f32_to_bf16_bits(rng.standard_normal((B, T, dout), dtype=np.float32) * 1e-2)
    Pf = np.zeros((din, r), np.float32)
    Pf[np.arange(r), np.arange(r)] = 1.0
    P = workloads.f32_to_bf16_bits(Pf)
    Xd, Gd, Pd = to_dev(X, "bf16", torch), to_dev(G, "bf16", torch), to_dev(P, "bf16", torch)
    Y = dp.project(Xd, Pd)
    assert torch.equal(Y, Xd[:, :, :r].contiguous())
    o1, n1 = dp.linear_clip_accumulate_projected(Xd, Gd, Pd, None, C=0.05, sigma=0.0)
    o2, n2 = dp.linear_clip_accumulate(Xd[:, :, :r].contiguous(), Gd, None, C=0.05, sigma=0.0)
    torch.cuda.synchronize()
    assert torch.equal(n1, n2) and torch.equal(o1, o2)


def _many_case(torch, dp, seed):
    """Six RoBERTa-large linears (B = 8, r = 256), masks on every other one
    (sample 0 empty), with their consecutive noise offsets."""
    rng = np.random.default_rng(seed)
    B, T, r = 8, 128, 256
    shapes = [(1024, 1024)] * 4 + [(1024, 4096), (4096, 1024)]
    Pd = {d: to_dev(_inputs(rng, 1, 1, d, r, "bf16")[1], "bf16", torch) for d in (1024, 4096)}
    Xs, Gs, Ps, masks = [], [], [], []
    for l, (din, dout) in enumerate(shapes):
        X, _ = _inputs(rng, B, T, din, r, "bf16")
        G = workloads.f32_to_bf16_bits(rng.standard_normal((B, T, dout), dtype=np.float32) * 1e-2)
        Xs.append(to_dev(X, "bf16", torch))
        Gs.append(to_dev(G, "bf16", torch))
        Ps.append(Pd[din])
        lengths = rng.integers(1, T + 1, B)
        lengths[0] = 0
        m = (np.arange(T)[None, :] < lengths[:, None]).astype(np.uint8)
        masks.append(None if l % 2 == 0 else mask_dev(m, torch))
    offsets = dp.consecutive_offsets([(int(g.shape[2]), r) for g in Gs])
    return Xs, Gs, Ps, masks, offsets


@pytest.mark.parametrize("side,path", [(1, 0), (0, 0), (2, 0), (4, 0), (1, 3)])
def test_projected_many_equals_the_single_calls(side, path):
    """The six linears of a RoBERTa-large layer (B = 8) queued together: on the
    caller's stream alone (side 0), spread over one, two or four library
    streams, and with the staged norm path asked for (the calls then run one
    after another).  Every output and norm equals the single projected call
    bit for bit (the same kernels on the same inputs), with masks on some of
    the linears and noise from consecutive offsets; two calls in a row agree."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    Xs, Gs, Ps, masks, offsets = _many_case(torch, dp, 34)
    old_side = dp.get_option("side_streams")
    dp.set_option("side_streams", side)
    dp.set_option("norm_path", path)
    try:
        outs, norms = dp.linear_clip_accumulate_projected_many(Xs, Gs, Ps, masks, C=0.05,
                                                               sigma=0.7, seed=5, offsets=offsets)
        outs2, norms2 = dp.linear_clip_accumulate_projected_many(Xs, Gs, Ps, masks, C=0.05,
                                                                 sigma=0.7, seed=5,
                                                                 offsets=offsets)
        torch.cuda.synchronize()
        for l in range(len(Xs)):
            o1, n1 = dp.linear_clip_accumulate_projected(Xs[l], Gs[l], Ps[l], masks[l], C=0.05,
                                                         sigma=0.7, seed=5, offset=offsets[l])
            torch.cuda.synchronize()
            assert torch.equal(outs[l], o1) and torch.equal(norms[l], n1), l
            assert torch.equal(outs2[l], o1) and torch.equal(norms2[l], n1), l
    finally:
        dp.set_option("side_streams", old_side)
        dp.set_option("norm_path", 0)


def test_projected_many_graph_replays_match_eager():
    """The multi-linear call captured into a HIP graph (the calls then run one
    after another on the capturing stream, in graph-owned workspace) and
    replayed three times, with eager calls on the same data in between: every
    replay's outputs and norms equal the eager call's bit for bit."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    Xs, Gs, Ps, masks, offsets = _many_case(torch, dp, 35)
    kw = dict(C=0.05, sigma=0.7, seed=6, offsets=offsets)
    ref, ref_n = dp.linear_clip_accumulate_projected_many(Xs, Gs, Ps, masks, **kw)
    outs = [torch.empty_like(o) for o in ref]
    norms = [torch.empty_like(n) for n in ref_n]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            dp.linear_clip_accumulate_projected_many(Xs, Gs, Ps, masks, grad_outs=outs,
                                                     norms_outs=norms, **kw)
    torch.cuda.synchronize()
    for it in range(3):
        for o, n in zip(outs, norms):
            o.fill_(float(it) - 5.0)
            n.fill_(-1.0)
        graph.replay()
        torch.cuda.synchronize()
        for l in range(len(Xs)):
            assert torch.equal(outs[l], ref[l]) and torch.equal(norms[l], ref_n[l]), (it, l)
        eager, eager_n = dp.linear_clip_accumulate_projected_many(Xs, Gs, Ps, masks, **kw)
        torch.cuda.synchronize()
        for l in range(len(Xs)):
            assert torch.equal(eager[l], ref[l]) and torch.equal(eager_n[l], ref_n[l]), (it, l)
    del graph
    torch.cuda.synchronize()
