"""Full-size parity: every linear of the Llama-13B-shaped decoder layer (B = 8,
T = 2048) and of the ragged batch (B = 16, T_i ~ U[128, 2048], masked), run
through the C ABI in the launch configuration the benchmark times, against
the full fp64 oracle (every output element, every per-sample norm).

Tolerances: norms 1e-3 relative; aggregate with noise 2e-2 relative
Frobenius; the sigma = 0 companion (clipped sum alone) 1e-3 (bf16 inputs are
exact in the oracle; only fp32 accumulation order differs).
"""
import numpy as np
import pytest

import workloads
from oracle import dp_linear
from tests.gpu_helpers import (assert_elementwise, assert_noise, max_rel, need_gpu, rel_fro,
                               run_dense)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

NORM_TOL = 1e-3
AGG_TOL = 2e-2
SUM_TOL = 1e-3


def _compare(lin, torch, path=None):
    out, norms = run_dense(lin, torch, path=path)
    ref, rnorms, rc = dp_linear.oracle_linear(lin.X, lin.G, lin.mask, lin.C, lin.sigma, lin.seed,
                                              lin.offset, lin.dtype)
    assert max_rel(norms, rnorms) <= NORM_TOL
    assert rel_fro(out, ref) <= AGG_TOL
    out0, _ = run_dense(lin, torch, sigma=0.0, path=path)
    xi = dp_linear.noise_matrix(lin.seed, lin.offset, ref.shape)
    ref0 = ref - lin.sigma * lin.C * xi / lin.B
    err0 = rel_fro(out0, ref0)
    assert err0 <= SUM_TOL, err0
    # element by element: the clipped sum, and the noise out(sigma) - out(0)
    assert_elementwise(out0, ref0, SUM_TOL, "sigma = 0 companion")
    assert_noise(out, out0, lin.sigma, lin.C, lin.seed, lin.offset, lin.B, "noise", xi=xi)
    return rnorms, rc


@pytest.mark.parametrize("index", range(7))
def test_llama13b_layer_linear(index):
    torch = need_gpu()
    lin = workloads.config_c3_linear(index)
    _compare(lin, torch)


# Each norm path forced on one linear of each shape (q: 5120 -> 5120, gate:
# 5120 -> 13824, down: 13824 -> 5120), whichever the automatic choice is:
# 1 Gram, 3 staged per-sample tiles.
@pytest.mark.parametrize("path", [1, 3])
@pytest.mark.parametrize("index", [0, 4, 6])
def test_llama13b_layer_linear_forced_path(index, path):
    torch = need_gpu()
    lin = workloads.config_c3_linear(index)
    _compare(lin, torch, path=path)


def test_llama13b_ragged_q_staged():
    torch = need_gpu()
    lin = workloads.config_c4_linear(0)
    _compare(lin, torch, path=3)


@pytest.mark.parametrize("index", range(7))
def test_llama13b_ragged_linear(index):
    torch = need_gpu()
    lin = workloads.config_c4_linear(index)
    _compare(lin, torch)


def test_llama13b_q_mixed_clip():
    """C at the median oracle norm, so half the samples take c_i = 1."""
    torch = need_gpu()
    lin = workloads.config_c3_linear(0)
    rn = dp_linear.oracle_norms(lin.X, lin.G, None, "bf16")
    C = float(np.median(rn))
    out, norms = run_dense(lin, torch, C=C, sigma=0.0)
    ref, rnorms, rc = dp_linear.oracle_linear(lin.X, lin.G, None, C, 0.0, 0, 0, "bf16")
    assert (rc == 1).any() and (rc < 1).any()
    assert max_rel(norms, rnorms) <= NORM_TOL
    assert rel_fro(out, ref) <= SUM_TOL
    assert_elementwise(out, ref, SUM_TOL, "mixed clip, sigma = 0")


# ---------------------------------------------------------------------------
# the staged path's 16 GiB limit (inputs drawn on the GPU: no oracle at these
# sizes; the paths are compared with each other)
# ---------------------------------------------------------------------------
def _kernels_of(dp, call):
    dp.timing_reset()
    dp.set_option("timing", 1)
    try:
        call()
        return dp.timing_collect()
    finally:
        dp.set_option("timing", 0)
        dp.timing_reset()


def _bf16_normal(torch, shape, scale, gen):
    return (torch.randn(shape, device="cuda", generator=gen) * scale).to(torch.bfloat16)


def test_staged_limit_falls_back_to_direct():
    """B = 168 at 5120 x 5120: the staged tiles would take 17.6 GB > 16 GiB, so
    even a forced staged call runs the direct path; its result matches the
    Gram path's."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    g = torch.Generator(device="cuda").manual_seed(5)
    B, T, D = 168, 256, 5120
    X = _bf16_normal(torch, (B, T, D), 1.0, g)
    G = _bf16_normal(torch, (B, T, D), 1e-3, g)
    res = {}
    for path in (3, 1):
        dp.set_option("norm_path", path)
        try:
            t = _kernels_of(dp, lambda: res.__setitem__(
                path, dp.linear_clip_accumulate(X, G, None, C=0.5, sigma=0.0)))
        finally:
            dp.set_option("norm_path", 0)
        if path == 3:
            assert "direct_norm" in t and "staged_norm" not in t, sorted(t)
    assert max_rel(res[3][1].cpu().numpy(), res[1][1].cpu().numpy()) <= 1e-4
    assert rel_fro(res[3][0].cpu().numpy(), res[1][0].cpu().numpy()) <= 1e-4


def test_group_past_staged_limit_mixes_paths():
    """Three linears whose staged tiles take 6.7 GB each: the first two are
    staged and the third, past the 16 GiB limit, takes its two-pass path;
    the group result matches the all-Gram group."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    g = torch.Generator(device="cuda").manual_seed(6)
    B, T, D = 64, 256, 5120
    Xs = [_bf16_normal(torch, (B, T, D), 1.0, g) for _ in range(3)]
    Gs = [_bf16_normal(torch, (B, T, D), 1e-3, g) for _ in range(3)]
    res = {}
    for path in (3, 1):
        dp.set_option("norm_path", path)
        try:
            t = _kernels_of(dp, lambda: res.__setitem__(path, dp.group_clip_accumulate(
                Xs, Gs, None, C=0.5, sigma=0.0, offsets=[0, 0, 0])))
        finally:
            dp.set_option("norm_path", 0)
        if path == 3:
            assert t["staged_norm"][1] == 2 and t["direct_norm"][1] == 1, t
    (o3, n3), (o1, n1) = res[3], res[1]
    assert max_rel(n3.cpu().numpy(), n1.cpu().numpy()) <= 1e-4
    for a, b in zip(o3, o1):
        assert rel_fro(a.cpu().numpy(), b.cpu().numpy()) <= 1e-4


def test_offsets_past_two_gib_take_the_generic_kernels():
    """X rows 8192 elements apart (a view into a 4 GiB buffer), T = 131072:
    a sample spans 2^30 elements, past what the large-tile kernels address
    with 32-bit offsets, so the call runs the generic kernels (64-bit
    addressing).  Against the oracle on the 64 columns in use; the other
    columns hold NaN, which must never be read."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    from tests.gpu_helpers import random_linear, to_dev
    B, T, din, dout, pitch = 2, 131072, 64, 64, 8192
    lin = random_linear(np.random.default_rng(33), B, T, din, dout)
    _, rn, _ = dp_linear.oracle_linear(lin.X, lin.G, None, 1.0, 0.0, 0, 0, "bf16")
    C = float(np.mean(rn))
    big = torch.full((B, T, pitch), float("nan"), dtype=torch.bfloat16, device="cuda")
    big[:, :, :din].copy_(to_dev(lin.X, "bf16", torch))
    X = big[:, :, :din]
    assert X.stride(1) * 131072 >= 1 << 30
    G = to_dev(lin.G, "bf16", torch)
    out, norms = dp.linear_clip_accumulate(X, G, None, C=C, sigma=0.8, seed=4, offset=9)
    out0, _ = dp.linear_clip_accumulate(X, G, None, C=C, sigma=0.0)
    torch.cuda.synchronize()
    ref, rnorms, _ = dp_linear.oracle_linear(lin.X, lin.G, None, C, 0.8, 4, 9, "bf16")
    ref0, _, _ = dp_linear.oracle_linear(lin.X, lin.G, None, C, 0.0, 0, 0, "bf16")
    assert max_rel(norms.cpu().numpy(), rnorms) <= NORM_TOL
    assert rel_fro(out.cpu().numpy(), ref) <= AGG_TOL
    assert rel_fro(out0.cpu().numpy(), ref0) <= SUM_TOL
    assert_elementwise(out0.cpu().numpy(), ref0, SUM_TOL, "generic kernels, sigma = 0")
    assert_noise(out.cpu().numpy(), out0.cpu().numpy(), 0.8, C, 4, 9, B, "generic kernels noise")
