"""GPU parity of the single-pass fused kernel (the "norm_path" option 4): each
per-sample gradient tile computed once, the per-sample norms reduced across
workgroups while the next sample is contracted, and c_i g_i added to a
running sum in registers -- against the fp64 oracle, element by element.

Bar: norms within 1e-3 relative; the sigma = 0 output within 1e-3 of the
largest entry (bf16 inputs are exact in the oracle; only the fp32 summation
order differs); the noise out(sigma) - out(0) within 1e-5 sigma C / denom of
the oracle's normals.  Also: bitwise repeatability, the explicit denominator
and accumulation, and the bounded wait's failure path forced from the host
(every fetch of partials treated as incomplete: the kernel gives up, exits
normally and poisons its outputs with NaN).
"""
import numpy as np
import pytest

import workloads
from oracle import dp_linear
from tests.gpu_helpers import (SUM_ELEM_TOL, assert_elementwise, assert_noise, mask_dev, max_rel,
                               need_gpu, random_linear, to_dev)

pytestmark = pytest.mark.gpu

NORM_TOL = 1e-3


class _Path:
    """The single-pass path (and other options) for one block."""

    def __init__(self, **kw):
        self.kw = {"norm_path": 4, **kw}

    def __enter__(self):
        import sample_gradient_clipping_amd as dp
        self.old = {k: dp.get_option(k) for k in self.kw}
        for k, v in self.kw.items():
            dp.set_option(k, v)

    def __exit__(self, *exc):
        import sample_gradient_clipping_amd as dp
        for k, v in self.old.items():
            dp.set_option(k, v)


def _kernels(dp, call):
    dp.timing_reset()
    dp.set_option("timing", 1)
    try:
        res = call()
        return res, dp.timing_collect()
    finally:
        dp.set_option("timing", 0)
        dp.timing_reset()


def _check(lin, C, sigma, seed=3, offset=5):
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    X, G, m = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch), mask_dev(lin.mask, torch)
    outs = {}
    with _Path():
        for sg in (0.0, sigma):
            (o, n), k = _kernels(dp, lambda: dp.linear_clip_accumulate(
                X, G, m, C=C, sigma=sg, seed=seed, offset=offset))
            torch.cuda.synchronize()
            assert "onepass" in k and "accumulate" not in k, sorted(k)
            outs[sg] = (o.cpu().numpy(), n.cpu().numpy())
    ref0, rn, rc = dp_linear.oracle_linear(lin.X, lin.G, lin.mask, C, 0.0, 0, 0, "bf16")
    for sg in (0.0, sigma):
        ok = rn > 0
        assert max_rel(outs[sg][1][ok], rn[ok]) <= NORM_TOL
        assert np.all(outs[sg][1][~ok] == 0.0)
    assert_elementwise(outs[0.0][0], ref0, SUM_ELEM_TOL["bf16"], "single pass, sigma = 0")
    assert_noise(outs[sigma][0], outs[0.0][0], sigma, C, seed, offset, lin.B, "single-pass noise")
    return rc


@pytest.mark.parametrize("shape,lengths", [
    ((3, 200, 264, 136), None),                   # 3 x 2 tiles with tails, 7 steps, ragged tail
    ((4, 300, 520, 776), [300, 0, 77, 300]),       # 5 x 7 tiles, a sample with no token
    ((1, 64, 128, 128), None),                     # one sample, one tile, two steps
    ((6, 97, 256, 512), [97, 1, 33, 64, 96, 0]),   # several short samples, an empty last one
    ((9, 40, 384, 1024), None),                    # more samples than pending places, T < step
])
def test_single_pass_small_against_oracle(shape, lengths):
    B, T, din, dout = shape
    rng = np.random.default_rng(sum(shape))
    lin = random_linear(rng, B, T, din, dout, lengths=lengths)
    _, rn, _ = dp_linear.oracle_linear(lin.X, lin.G, lin.mask, 1.0, 0.0, 0, 0, "bf16")
    pos = rn[rn > 0]
    C = float(np.median(pos)) if len(pos) > 1 else float(pos.max()) * 0.5
    rc = _check(lin, C, 0.9)
    assert (rc < 1).any()


def test_single_pass_random_mask():
    rng = np.random.default_rng(71)
    lin = random_linear(rng, 5, 257, 520, 264, masked=True)
    _, rn, _ = dp_linear.oracle_linear(lin.X, lin.G, lin.mask, 1.0, 0.0, 0, 0, "bf16")
    _check(lin, float(np.median(rn)), 1.2)


def test_single_pass_gpt2_up_projection():
    """The GPT-2-small MLP up-projection workload (B = 32, T = 512,
    768 -> 3072): 144 tiles, every one resident; sigma 0.8 and its sigma = 0
    companion, plus the mixed-clip supplement (C at the median norm)."""
    lin = workloads.config_c2().linears[0]
    _check(lin, lin.C, lin.sigma, seed=lin.seed, offset=lin.offset)
    _, rn, _ = dp_linear.oracle_linear(lin.X, lin.G, None, 1.0, 0.0, 0, 0, "bf16")
    rc = _check(lin, float(np.median(rn)), lin.sigma)
    assert (rc == 1).any() and (rc < 1).any()


def test_single_pass_is_bitwise_repeatable():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(72)
    lin = random_linear(rng, 8, 300, 768, 1024, lengths=[300, 150, 0, 299, 1, 300, 64, 200])
    X, G, m = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch), mask_dev(lin.mask, torch)
    with _Path():
        ref = dp.linear_clip_accumulate(X, G, m, C=0.05, sigma=0.7, seed=2, offset=9)
        for _ in range(10):
            got = dp.linear_clip_accumulate(X, G, m, C=0.05, sigma=0.7, seed=2, offset=9)
            torch.cuda.synchronize()
            assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_single_pass_explicit_denominator_and_accumulation():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(73)
    lin = random_linear(rng, 3, 300, 520, 264)
    _, rn, _ = dp_linear.oracle_linear(lin.X, lin.G, None, 1.0, 0.0, 0, 0, "bf16")
    C = float(np.median(rn))
    s0, _, _ = dp_linear.oracle_linear(lin.X, lin.G, None, C, 0.0, 0, 0, "bf16", denom=10.0)
    out0 = (rng.standard_normal(s0.shape) * np.abs(s0).mean()).astype(np.float32)
    X, G = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch)
    grads = {}
    with _Path():
        for sigma in (0.0, 0.9):
            grad = torch.from_numpy(out0.copy()).cuda()
            dp.linear_clip_accumulate(X, G, None, C=C, sigma=sigma, seed=5, offset=17,
                                      grad_out=grad, denom=10.0, accumulate=True)
            torch.cuda.synchronize()
            grads[sigma] = grad.cpu().numpy()
    ref, _, _ = dp_linear.oracle_linear(lin.X, lin.G, None, C, 0.0, 0, 0, "bf16", denom=10.0,
                                        out0=out0)
    assert_elementwise(grads[0.0].astype(np.float64) - out0, ref - out0, SUM_ELEM_TOL["bf16"],
                       "accumulated, sigma = 0")
    assert_noise(grads[0.9], grads[0.0], 0.9, C, 5, 17, 10.0, "accumulated noise")


def test_single_pass_matches_the_two_phase_paths():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(74)
    lin = random_linear(rng, 4, 512, 768, 768, lengths=[512, 300, 17, 511])
    X, G, m = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch), mask_dev(lin.mask, torch)
    with _Path():
        o1, n1 = dp.linear_clip_accumulate(X, G, m, C=0.1, sigma=0.0)
    for path in (1, 2):
        with _Path(norm_path=path):
            o2, n2 = dp.linear_clip_accumulate(X, G, m, C=0.1, sigma=0.0)
        torch.cuda.synchronize()
        assert max_rel(n1.cpu().numpy(), n2.cpu().numpy()) <= 1e-5
        assert_elementwise(o1.cpu().numpy(), o2.cpu().numpy(), 1e-5, f"single pass vs path {path}")


def test_single_pass_gives_up_cleanly_when_partials_never_arrive():
    """Forced from the host: every fetch of partials counts as incomplete,
    so every bounded wait gives up.  The kernel still exits, and its outputs
    are NaN (never a silent wrong value); the next call is normal."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(75)
    lin = random_linear(rng, 4, 128, 256, 384)
    X, G = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch)
    with _Path(onepass_never_ready=1, onepass_spin_limit=3):
        out, norms = dp.linear_clip_accumulate(X, G, None, C=0.05, sigma=0.5)
        torch.cuda.synchronize()
    assert torch.all(torch.isnan(out)) and torch.all(torch.isnan(norms))
    with _Path():
        out, norms = dp.linear_clip_accumulate(X, G, None, C=0.05, sigma=0.0)
        torch.cuda.synchronize()
    ref, rn, _ = dp_linear.oracle_linear(lin.X, lin.G, None, 0.05, 0.0, 0, 0, "bf16")
    assert max_rel(norms.cpu().numpy(), rn) <= NORM_TOL
    assert_elementwise(out.cpu().numpy(), ref, SUM_ELEM_TOL["bf16"], "after the forced give-up")
