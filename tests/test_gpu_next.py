"""GPU parity for the widenings of the hot path: the projection drawn from its
seed inside the projection kernel (P never stored), group (joint) clipping
over several linears that see the same samples, and the projected Adam step
that consumes the privatised projected gradient.

Tolerances as for the dense and projected calls: norms 1e-3 relative;
aggregates 2e-2 relative Frobenius with noise; sigma = 0 companions 1e-3
(dense, bf16 inputs exact in the oracle) or 1e-2 (projected: Y rounded to
bf16 on the GPU).  The seeded projection is also checked bit for bit against
the stored-P call fed with the P that dpfused_gaussian_fill draws from the
same seed: both must run the same arithmetic on the same values.
"""
import math

import numpy as np
import pytest

import workloads
from oracle import dp_linear
from tests.gpu_helpers import (SUM_ELEM_TOL, assert_elementwise, assert_noise, mask_dev, max_rel,
                               need_gpu, random_linear, rel_fro, to_dev)

pytestmark = pytest.mark.gpu

NORM_TOL = 1e-3
AGG_TOL_BF16 = 2e-2
SUM_TOL_BF16 = 1e-3


# ---------------------------------------------------------------------------
# seeded projection
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("in_kernel", [0, 1])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 150, 1000, 136, 72), (2, 64, 136, 200, 256)])
def test_seeded_projection_equals_stored_projection(dtype, shape, in_kernel):
    """P drawn inside the projection kernel (one token tile, or p_in_kernels
    on) or once into workspace: the stored-P call's bits either way."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    dp.set_option("p_in_kernels", in_kernel)
    try:
        _seeded_vs_stored(torch, dp, dtype, shape)
    finally:
        dp.set_option("p_in_kernels", 0)


def _seeded_vs_stored(torch, dp, dtype, shape):
    B, T, din, dout, r = shape
    rng = np.random.default_rng(41)
    lin = random_linear(rng, B, T, din, dout, dtype=dtype, lengths=[T] + [T // 3] * (B - 1))
    X, G, m = to_dev(lin.X, dtype, torch), to_dev(lin.G, dtype, torch), mask_dev(lin.mask, torch)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    scale = 1.0 / math.sqrt(r)
    P = dp.gaussian_fill(9, 3, din * r, scale, dtype=tdt).view(din, r)
    o1, n1 = dp.linear_clip_accumulate_projected(X, G, P, m, C=0.05, sigma=0.7, seed=1, offset=2)
    o2, n2 = dp.linear_clip_accumulate_projected_seeded(X, G, r, m, p_seed=9, p_offset=3,
                                                        p_scale=scale, C=0.05, sigma=0.7, seed=1,
                                                        offset=2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(n1, n2)


@pytest.mark.parametrize("index", [0, 5])
def test_seeded_projection_roberta_vs_oracle(index):
    """RoBERTa-large shapes, r = 256, P from Philox seed 7 with entries
    N(0, 1/r): the GPU draws P inside the projection, the oracle with its own
    generator."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    lin = workloads.config_c5_linear(index)
    r = 256
    X, G = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch)
    P = dp_linear.projection_matrix(7, 0, lin.din, r, 1.0 / 16.0, "bf16")
    outs = {}
    for sigma, tol in ((lin.sigma, AGG_TOL_BF16), (0.0, 1e-2)):
        out, norms = dp.linear_clip_accumulate_projected_seeded(X, G, r, None, p_seed=7,
                                                                p_offset=0, C=lin.C, sigma=sigma)
        ref, rn, _ = dp_linear.oracle_projected(lin.X, lin.G, None, P, lin.C, sigma, 0, 0, "bf16")
        assert max_rel(norms.cpu().numpy(), rn) <= NORM_TOL
        assert rel_fro(out.cpu().numpy(), ref) <= tol
        outs[sigma] = out.cpu().numpy()
    # element by element (Y rounded to bf16 on the GPU: 1e-2 of the largest entry)
    assert_elementwise(outs[0.0], ref, 1e-2, "seeded projected sigma = 0")
    assert_noise(outs[lin.sigma], outs[0.0], lin.sigma, lin.C, 0, 0, lin.B, "seeded noise")


# ---------------------------------------------------------------------------
# group clipping
# ---------------------------------------------------------------------------
def _group_case(rng, B, T, dims, lengths, dtype="bf16"):
    lins = [random_linear(rng, B, T, din, dout, dtype=dtype, lengths=lengths) for din, dout in dims]
    return lins, lins[0].mask


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_group_clip_matches_oracle(dtype):
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(42)
    dims = [(512, 640), (640, 512), (256, 1024)] if dtype == "bf16" else [(64, 40), (24, 72)]
    B, T = 3, 300
    lins, mask = _group_case(rng, B, T, dims, [300, 150, 37], dtype)
    pairs = [(l.X, l.G) for l in lins]
    offsets = dp.consecutive_offsets([(dout, din) for din, dout in dims], start=1000)
    _, rn, _ = dp_linear.oracle_group(pairs, mask, 1.0, 0.0, 0, offsets, dtype)
    C = float(np.median(rn))               # some samples clip, some do not
    Xs = [to_dev(l.X, dtype, torch) for l in lins]
    Gs = [to_dev(l.G, dtype, torch) for l in lins]
    m = mask_dev(mask, torch)
    sum_tol = SUM_TOL_BF16 if dtype == "bf16" else 1e-4
    got = {}
    for sigma, tol in ((0.0, sum_tol), (1.1, AGG_TOL_BF16 if dtype == "bf16" else 1e-4)):
        outs, norms = dp.group_clip_accumulate(Xs, Gs, m, C=C, sigma=sigma, seed=3,
                                               offsets=offsets)
        refs, rn, rc = dp_linear.oracle_group(pairs, mask, C, sigma, 3, offsets, dtype)
        assert (rc == 1).any() and (rc < 1).any()
        assert max_rel(norms.cpu().numpy(), rn) <= NORM_TOL
        for o, ref in zip(outs, refs):
            assert rel_fro(o.cpu().numpy(), ref) <= tol
        got[sigma] = ([o.cpu().numpy() for o in outs], refs)
    _group_elementwise(got, 1.1, C, 3, offsets, B, dtype)


def _group_elementwise(got, sigma, C, seed, offsets, B, dtype):
    """Each linear's sigma = 0 output against the oracle, and its noise
    out(sigma) - out(0) against its own stream (seed, offsets[l])."""
    outs0, refs0 = got[0.0]
    outs1, _ = got[sigma]
    for l, (o0, r0, o1) in enumerate(zip(outs0, refs0, outs1)):
        assert_elementwise(o0, r0, SUM_ELEM_TOL[dtype], f"group linear {l}, sigma = 0")
        assert_noise(o1, o0, sigma, C, seed, offsets[l], B, f"group linear {l} noise")


def test_group_of_one_is_the_dense_call_bitwise():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(43)
    lin = random_linear(rng, 4, 257, 264, 136, masked=True)
    X, G, m = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch), mask_dev(lin.mask, torch)
    o1, n1 = dp.linear_clip_accumulate(X, G, m, C=0.01, sigma=0.9, seed=5, offset=17)
    (o2,), n2 = dp.group_clip_accumulate([X], [G], m, C=0.01, sigma=0.9, seed=5, offsets=[17])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(n1, n2)


@pytest.mark.parametrize("path", [0, 3])
def test_group_clip_unmasked_matches_oracle(path):
    """Unmasked bf16 group over the large-tile path: automatic choice, and
    every linear forced onto the staged path (per-sample tiles kept from
    each linear's norm phase until the group's clip factors exist)."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(45)
    dims = [(512, 640), (640, 512), (256, 1024)]
    lins, mask = _group_case(rng, 3, 300, dims, None)
    pairs = [(l.X, l.G) for l in lins]
    offsets = dp.consecutive_offsets([(dout, din) for din, dout in dims])
    _, rn, _ = dp_linear.oracle_group(pairs, None, 1.0, 0.0, 0, offsets, "bf16")
    C = float(np.median(rn))
    Xs = [to_dev(l.X, "bf16", torch) for l in lins]
    Gs = [to_dev(l.G, "bf16", torch) for l in lins]
    dp.set_option("norm_path", path)
    try:
        got = {}
        for sigma, tol in ((0.0, SUM_TOL_BF16), (1.1, AGG_TOL_BF16)):
            outs, norms = dp.group_clip_accumulate(Xs, Gs, None, C=C, sigma=sigma, seed=3,
                                                   offsets=offsets)
            refs, rn, rc = dp_linear.oracle_group(pairs, None, C, sigma, 3, offsets, "bf16")
            assert (rc == 1).any() and (rc < 1).any()
            assert max_rel(norms.cpu().numpy(), rn) <= NORM_TOL
            for o, ref in zip(outs, refs):
                assert rel_fro(o.cpu().numpy(), ref) <= tol
            got[sigma] = ([o.cpu().numpy() for o in outs], refs)
        _group_elementwise(got, 1.1, C, 3, offsets, 3, "bf16")
    finally:
        dp.set_option("norm_path", 0)


def test_group_of_one_is_the_staged_dense_call_bitwise():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(46)
    lin = random_linear(rng, 4, 257, 264, 136)
    X, G = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch)
    dp.set_option("norm_path", 3)
    try:
        o1, n1 = dp.linear_clip_accumulate(X, G, None, C=0.01, sigma=0.9, seed=5, offset=17)
        (o2,), n2 = dp.group_clip_accumulate([X], [G], None, C=0.01, sigma=0.9, seed=5,
                                             offsets=[17])
        torch.cuda.synchronize()
    finally:
        dp.set_option("norm_path", 0)
    assert torch.equal(o1, o2)
    assert torch.equal(n1, n2)


def test_group_row_split_reproduces_whole_layer():
    """Two linears that are the output-row halves of one linear: group
    clipping of the halves gives the whole linear's per-layer result."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(44)
    B, T, din, dout, d1 = 4, 200, 512, 768, 256
    lin = random_linear(rng, B, T, din, dout, lengths=[200, 90, 200, 13])
    X, G, m = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch), mask_dev(lin.mask, torch)
    whole, nw = dp.linear_clip_accumulate(X, G, m, C=0.02, sigma=0.6, seed=2, offset=8)
    G1 = G[:, :, :d1].contiguous()
    G2 = G[:, :, d1:].contiguous()
    (h1, h2), ng = dp.group_clip_accumulate([X, X], [G1, G2], m, C=0.02, sigma=0.6, seed=2,
                                            offsets=[8, 8 + d1 * din // 4])
    assert max_rel(ng.cpu().numpy(), nw.cpu().numpy()) <= 1e-4
    assert rel_fro(torch.cat([h1, h2]).cpu().numpy(), whole.cpu().numpy()) <= 1e-4


# ---------------------------------------------------------------------------
# projected Adam step
# ---------------------------------------------------------------------------
def _adam_case(rng, dout, din, r):
    h = (rng.standard_normal((dout, r)) * 0.01).astype(np.float32)
    m = (rng.standard_normal((dout, r)) * 0.005).astype(np.float32)
    v = (rng.random((dout, r)) * 1e-4).astype(np.float32)
    W = rng.standard_normal((dout, din)).astype(np.float32)
    return h, m, v, W


@pytest.mark.parametrize("pdtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(200, 136, 72), (1024, 4096, 256), (1024, 1024, 256)])
def test_projected_adam_step_matches_oracle(pdtype, shape):
    """Elementwise moments in float32 against float64: 1e-6 relative; the
    weight change lr * U P^T (float32 MFMA over r) within 1e-5 of the
    oracle's change."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    from oracle import optim
    dout, din, r = shape
    rng = np.random.default_rng(45)
    h, m, v, W = _adam_case(rng, dout, din, r)
    Pf = (rng.standard_normal((din, r)) / np.sqrt(r)).astype(np.float32)
    P = workloads.f32_to_bf16_bits(Pf) if pdtype == "bf16" else Pf
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    hd, md, vd, Wd = dev(h), dev(m), dev(v), dev(W)
    Pd = to_dev(P, pdtype, torch)
    step, lr, b1, b2, eps = 7, 1e-3, 0.9, 0.999, 1e-8
    dp.projected_adam_step(hd, md, vd, Wd, step, lr, b1, b2, eps, P=Pd)
    rm, rv, rW = optim.projected_adam_step(h, m, v, W, step, lr, b1, b2, eps,
                                           dp_linear.widen(P, pdtype))
    assert rel_fro(md.cpu().numpy(), rm) <= 1e-6
    assert rel_fro(vd.cpu().numpy(), rv) <= 1e-6
    dW_ref = rW - W.astype(np.float64)
    dW = Wd.cpu().numpy().astype(np.float64) - W.astype(np.float64)
    assert np.linalg.norm(dW - dW_ref) <= 1e-5 * np.linalg.norm(dW_ref) + 1e-7 * np.linalg.norm(W)


@pytest.mark.parametrize("in_kernel", [0, 1])
@pytest.mark.parametrize("dout", [300, 1024, 60])
def test_projected_adam_seeded_equals_stored(dout, in_kernel):
    """P drawn once into workspace (dout 300, 1024) or inside the update
    kernel (dout 60: one row of W tiles; or p_in_kernels on) gives the
    stored-P step bit for bit."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    dp.set_option("p_in_kernels", in_kernel)
    try:
        _adam_seeded_vs_stored(torch, dp, dout)
    finally:
        dp.set_option("p_in_kernels", 0)


def _adam_seeded_vs_stored(torch, dp, dout):
    din, r = 520, 64
    rng = np.random.default_rng(46)
    h, m, v, W = _adam_case(rng, dout, din, r)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    P = dp.gaussian_fill(5, 11, din * r, 0.125, dtype=torch.bfloat16).view(din, r)
    outs = []
    for seeded in (False, True):
        md, vd, Wd = dev(m), dev(v), dev(W)
        if seeded:
            dp.projected_adam_step(dev(h), md, vd, Wd, 2, 1e-2, P=None, p_seed=5, p_offset=11,
                                   p_scale=0.125, p_dtype=torch.bfloat16)
        else:
            dp.projected_adam_step(dev(h), md, vd, Wd, 2, 1e-2, P=P)
        outs.append((md, vd, Wd))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_projected_dp_step_end_to_end_roberta():
    """The projected call (P drawn from its seed) followed by the projected
    Adam step on one RoBERTa-large linear, against the oracles chained."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    from oracle import optim
    lin = workloads.config_c5_linear(4)          # fc1: 1024 -> 4096
    r = 256
    X, G = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch)
    h, _ = dp.linear_clip_accumulate_projected_seeded(X, G, r, None, p_seed=7, p_offset=0,
                                                      C=lin.C, sigma=lin.sigma)
    rng = np.random.default_rng(47)
    W = rng.standard_normal((lin.dout, lin.din)).astype(np.float32)
    Wd = torch.from_numpy(W).cuda()
    md = torch.zeros((lin.dout, r), dtype=torch.float32, device="cuda")
    vd = torch.zeros_like(md)
    dp.projected_adam_step(h, md, vd, Wd, 1, 1e-3, P=None, p_seed=7, p_offset=0)
    P = dp_linear.projection_matrix(7, 0, lin.din, r, 1.0 / 16.0, "bf16")
    href, _, _ = dp_linear.oracle_projected(lin.X, lin.G, None, P, lin.C, lin.sigma, 0, 0, "bf16")
    assert rel_fro(h.cpu().numpy(), href) <= AGG_TOL_BF16
    # the step from the GPU's own h (the privatised gradient is the input of the step)
    _, _, rW = optim.projected_adam_step(h.cpu().numpy(), np.zeros((lin.dout, r)),
                                         np.zeros((lin.dout, r)), W, 1, 1e-3, 0.9, 0.999, 1e-8,
                                         dp_linear.widen(P, "bf16"))
    dW_ref = rW - W.astype(np.float64)
    dW = Wd.cpu().numpy().astype(np.float64) - W.astype(np.float64)
    # a few P entries may round to the neighbouring bf16 value on either side
    assert np.linalg.norm(dW - dW_ref) <= 2e-3 * np.linalg.norm(dW_ref)


# ---------------------------------------------------------------------------
# bias gradients
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
# dout 136 and 3072: 8 bf16 columns per thread, token chunks; dout 37: one
# column per thread
@pytest.mark.parametrize("shape", [(3, 300, 264, 136), (4, 16, 64, 32), (3, 300, 40, 37),
                                   (2, 70, 64, 3072)])
def test_bias_matches_oracle(dtype, shape):
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    B, T, din, dout = shape
    rng = np.random.default_rng(48)
    lin = random_linear(rng, B, T, din, dout, dtype=dtype, lengths=[T] + [T // 2] * (B - 1))
    X, G, m = to_dev(lin.X, dtype, torch), to_dev(lin.G, dtype, torch), mask_dev(lin.mask, torch)
    _, _, rn, _ = dp_linear.oracle_linear_bias(lin.X, lin.G, lin.mask, 1.0, 0.0, 0, 0, dtype)
    C = float(np.median(rn))
    sum_tol = SUM_TOL_BF16 if dtype == "bf16" else 1e-4
    got = {}
    for sigma, tol in ((0.0, sum_tol), (0.9, AGG_TOL_BF16 if dtype == "bf16" else 1e-4)):
        ow, ob, norms = dp.linear_clip_accumulate_bias(X, G, m, C=C, sigma=sigma, seed=4, offset=6)
        rw, rb, rn, rc = dp_linear.oracle_linear_bias(lin.X, lin.G, lin.mask, C, sigma, 4, 6, dtype)
        assert (rc == 1).any() and (rc < 1).any()
        assert max_rel(norms.cpu().numpy(), rn) <= NORM_TOL
        assert rel_fro(ow.cpu().numpy(), rw) <= tol
        assert rel_fro(ob.cpu().numpy(), rb) <= tol
        got[sigma] = (ow.cpu().numpy(), ob.cpu().numpy(), rw, rb)
    _bias_elementwise(got, 0.9, C, 4, 6, B, din, dout, dtype)


def _bias_elementwise(got, sigma, C, seed, offset, B, din, dout, dtype):
    """Weight and bias outputs at sigma = 0 against the oracle; the noise of
    each: the weight's from `offset`, the bias's continuing the stream."""
    w0, b0, rw0, rb0 = got[0.0]
    w1, b1, _, _ = got[sigma]
    assert_elementwise(w0, rw0, SUM_ELEM_TOL[dtype], "bias call weight, sigma = 0")
    assert_elementwise(b0, rb0, SUM_ELEM_TOL[dtype], "bias call bias, sigma = 0")
    assert_noise(w1, w0, sigma, C, seed, offset, B, "bias call weight noise")
    assert_noise(b1, b0, sigma, C, seed, offset + (din * dout + 3) // 4, B, "bias noise")


@pytest.mark.parametrize("path", [0, 1, 3])
def test_bias_unmasked_matches_oracle(path):
    """Unmasked bf16 over the large-tile kernels: the automatic choice (the
    staged path at this shape), Gram, and staged forced."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(50)
    lin = random_linear(rng, 4, 300, 520, 264)
    X, G = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch)
    _, _, rn, _ = dp_linear.oracle_linear_bias(lin.X, lin.G, None, 1.0, 0.0, 0, 0, "bf16")
    C = float(np.median(rn))
    dp.set_option("norm_path", path)
    try:
        got = {}
        for sigma, tol in ((0.0, SUM_TOL_BF16), (0.9, AGG_TOL_BF16)):
            ow, ob, norms = dp.linear_clip_accumulate_bias(X, G, None, C=C, sigma=sigma, seed=4,
                                                           offset=6)
            rw, rb, rn, rc = dp_linear.oracle_linear_bias(lin.X, lin.G, None, C, sigma, 4, 6,
                                                          "bf16")
            assert (rc == 1).any() and (rc < 1).any()
            assert max_rel(norms.cpu().numpy(), rn) <= NORM_TOL
            assert rel_fro(ow.cpu().numpy(), rw) <= tol
            assert rel_fro(ob.cpu().numpy(), rb) <= tol
            got[sigma] = (ow.cpu().numpy(), ob.cpu().numpy(), rw, rb)
        _bias_elementwise(got, 0.9, C, 4, 6, 4, 520, 264, "bf16")
    finally:
        dp.set_option("norm_path", 0)


def test_bias_is_the_weight_of_a_constant_input_on_gpu():
    """The bias call against the dense call on [X, 1] (sigma = 0)."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(49)
    B, T, din, dout = 4, 257, 263, 136
    lin = random_linear(rng, B, T, din, dout, lengths=[257, 100, 3, 257])
    X, G, m = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch), mask_dev(lin.mask, torch)
    Xa = torch.cat([X, torch.ones((B, T, 1), dtype=X.dtype, device=X.device)], dim=2).contiguous()
    ow, ob, nb = dp.linear_clip_accumulate_bias(X, G, m, C=0.05, sigma=0.0)
    oa, na = dp.linear_clip_accumulate(Xa, G, m, C=0.05, sigma=0.0)
    assert max_rel(nb.cpu().numpy(), na.cpu().numpy()) <= 1e-4
    assert rel_fro(ow.cpu().numpy(), oa[:, :din].cpu().numpy()) <= 1e-4
    assert rel_fro(ob.cpu().numpy(), oa[:, din].cpu().numpy()) <= 1e-4


# ---------------------------------------------------------------------------
# f4: explicit denominator, accumulation into grad_out
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,path", [("bf16", 1), ("bf16", 2), ("bf16", 3), ("f32", 2)])
def test_ex_accumulates_into_grad_out_against_oracle(dtype, path):
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(47)
    lin = random_linear(rng, 3, 300, 520, 264, dtype=dtype) if dtype == "bf16" else \
        random_linear(rng, 3, 40, 72, 56, dtype=dtype)
    _, rn, _ = dp_linear.oracle_linear(lin.X, lin.G, None, 1.0, 0.0, 0, 0, dtype)
    C = float(np.median(rn))
    s0, _, _ = dp_linear.oracle_linear(lin.X, lin.G, None, C, 0.0, 0, 0, dtype, denom=10.0)
    out0 = (rng.standard_normal(s0.shape) * np.abs(s0).mean()).astype(np.float32)
    X, G = to_dev(lin.X, dtype, torch), to_dev(lin.G, dtype, torch)
    dp.set_option("norm_path", path)
    try:
        grads = {}
        for sigma in (0.0, 0.9):
            ref, rnorms, _ = dp_linear.oracle_linear(lin.X, lin.G, None, C, sigma, 5, 17, dtype,
                                                     denom=10.0, out0=out0)
            grad = torch.from_numpy(out0.copy()).cuda()
            _, norms = dp.linear_clip_accumulate(X, G, None, C=C, sigma=sigma, seed=5, offset=17,
                                                 grad_out=grad, denom=10.0, accumulate=True)
            assert max_rel(norms.cpu().numpy(), rnorms) <= NORM_TOL
            # the part this call adds, free of out0
            got = grad.cpu().numpy().astype(np.float64) - out0
            tol = (SUM_TOL_BF16 if sigma == 0.0 else AGG_TOL_BF16) if dtype == "bf16" else 1e-4
            assert rel_fro(got, ref - out0) <= tol
            grads[sigma] = (grad.cpu().numpy(), ref)
        # element by element: grad_out after the sigma = 0 call against the
        # oracle, and the noise the sigma = 0.9 call added on top of the same
        # prior contents, divided by the explicit denominator
        assert_elementwise(grads[0.0][0].astype(np.float64) - out0, grads[0.0][1] - out0,
                           SUM_ELEM_TOL[dtype], "accumulated sigma = 0")
        assert_noise(grads[0.9][0], grads[0.0][0], 0.9, C, 5, 17, 10.0, "accumulated noise")
    finally:
        dp.set_option("norm_path", 0)


@pytest.mark.parametrize("path", [1, 2, 3])
def test_micro_batches_add_up_to_the_whole_batch(path):
    """Three micro-batches of a batch of 6, each divided by 6, the noise in
    the first, accumulated into one buffer: the whole batch's result."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(48)
    lin = random_linear(rng, 6, 300, 520, 264)
    X, G = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch)
    C = 0.02
    dp.set_option("norm_path", path)
    try:
        whole, wn = dp.linear_clip_accumulate(X, G, None, C=C, sigma=0.8, seed=3, offset=4)
        acc = torch.empty_like(whole)
        parts = [(0, 2, 0.8, False), (2, 5, 0.0, True), (5, 6, 0.0, True)]
        norms = []
        for a, b, sigma, add in parts:
            _, n = dp.linear_clip_accumulate(X[a:b].contiguous(), G[a:b].contiguous(), None, C=C,
                                             sigma=sigma, seed=3, offset=4, grad_out=acc,
                                             denom=6.0, accumulate=add)
            norms.append(n)
        torch.cuda.synchronize()
    finally:
        dp.set_option("norm_path", 0)
    assert max_rel(torch.cat(norms).cpu().numpy(), wn.cpu().numpy()) <= 1e-6
    assert rel_fro(acc.cpu().numpy(), whole.cpu().numpy()) <= 1e-5
