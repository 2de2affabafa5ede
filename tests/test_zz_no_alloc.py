"""The entry point that allocates nothing (dpfused_linear_clip_accumulate_noalloc),
called through the C ABI, against the allocating entry point
(dpfused_linear_clip_accumulate) on the same inputs: two calls in a row, the
second with a smaller input, and a call whose workspace cannot fit the static
scratch, which must fail before writing anything.

Bar: norms within 1e-3 relative; the sigma = 0 clipped sum element by element
within 1e-3 of the largest entry (bf16 inputs: only the fp32 summation order
may differ, e.g. when the no-allocation call runs without split tiles); the
noise out(sigma) - out(0) within 1e-5 * sigma * C / B of the oracle's normals.
Where both calls take the same plan the results are identical bit for bit.
"""
import ctypes

import numpy as np
import pytest

from oracle import dp_linear
from sample_gradient_clipping_amd._lib import DPF_ERR_UNSUPPORTED, DPF_OK
from tests.gpu_helpers import (SUM_ELEM_TOL, assert_elementwise, assert_noise, mask_dev, max_rel,
                               need_gpu, random_linear, to_dev)

pytestmark = pytest.mark.gpu


def _noalloc(dp, X, G, m, C, sigma, seed, offset, out, norms):
    """One call of the no-allocation entry point through the C ABI."""
    from sample_gradient_clipping_amd import _lib
    import torch
    xa, ga = dp._act(X), dp._act(G)
    st = _lib.lib().dpfused_linear_clip_accumulate_noalloc(
        ctypes.byref(xa), ctypes.byref(ga), None if m is None else m.data_ptr(), float(C),
        float(sigma), int(seed), int(offset), out.data_ptr(),
        None if norms is None else norms.data_ptr(),
        int(torch.cuda.current_stream().cuda_stream))
    return st


def _compare(torch, dp, lin, C, sigma, seed, offset, bitwise):
    X, G, m = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch), mask_dev(lin.mask, torch)
    B, dout, din = lin.B, lin.dout, lin.din
    got = {}
    for sg in (0.0, sigma):
        out = torch.full((dout, din), 3.0, device="cuda")
        norms = torch.full((B,), -1.0, device="cuda")
        assert _noalloc(dp, X, G, m, C, sg, seed, offset, out, norms) == DPF_OK, \
            dp._lib.lib().dpfused_last_error()
        ref, ref_n = dp.linear_clip_accumulate(X, G, m, C=C, sigma=sg, seed=seed, offset=offset)
        torch.cuda.synchronize()
        if bitwise:
            assert torch.equal(out, ref) and torch.equal(norms, ref_n)
        assert max_rel(norms.cpu().numpy(), ref_n.cpu().numpy()) <= 1e-3
        got[sg] = (out.cpu().numpy(), ref.cpu().numpy(), norms.cpu().numpy())
    assert_elementwise(got[0.0][0], got[0.0][1], SUM_ELEM_TOL["bf16"], "no-alloc vs allocating")
    assert_noise(got[sigma][0], got[0.0][0], sigma, C, seed, offset, B, "no-alloc noise")
    return got


def test_noalloc_matches_the_allocating_call_twice_second_smaller():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(61)
    # 1: a masked 5120 x 5120 layer at T = 2048 on the Gram path, whose split
    #    Gram items (parked blocks plus split pieces) exceed the scratch, so
    #    the call runs without splits (summation order may differ)
    big = random_linear(rng, 2, 2048, 5120, 5120, lengths=[2048, 1000])
    _, rn, _ = dp_linear.oracle_linear(big.X, big.G, big.mask, 1.0, 0.0, 0, 0, "bf16")
    C = float(np.median(rn))
    got = _compare(torch, dp, big, C, 0.8, 3, 11, bitwise=False)
    ref0, rn0, _ = dp_linear.oracle_linear(big.X, big.G, big.mask, C, 0.0, 0, 0, "bf16")
    assert max_rel(got[0.0][2], rn0) <= 1e-3
    assert_elementwise(got[0.0][0], ref0, SUM_ELEM_TOL["bf16"], "no-alloc vs oracle")
    # 2: smaller, right after: its plan fits the scratch, so the results are
    #    the allocating call's bit for bit (the scratch's old contents unused)
    small = random_linear(rng, 3, 300, 520, 776)
    _, rn, _ = dp_linear.oracle_linear(small.X, small.G, None, 1.0, 0.0, 0, 0, "bf16")
    _compare(torch, dp, small, float(np.median(rn)), 1.1, 5, 2, bitwise=True)


def test_noalloc_rejects_a_workspace_past_the_scratch():
    """Direct norm path forced with B * tiles partials of 88 MB (> 80 MiB):
    DPF_ERR_UNSUPPORTED, nothing written."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    B, D = 1100, 25600
    X = torch.zeros((B, 1, D), dtype=torch.bfloat16, device="cuda")
    G = torch.zeros((B, 1, D), dtype=torch.bfloat16, device="cuda")
    out = torch.full((D, D), 7.0, device="cuda")   # [dout, din]: the call fails before writing
    norms = torch.full((B,), -2.0, device="cuda")
    dp.set_option("norm_path", 2)
    try:
        st = _noalloc(dp, X, G, None, 1.0, 0.0, 0, 0, out, norms)
        msg = dp._lib.lib().dpfused_last_error()   # per thread; the next call clears it
    finally:
        dp.set_option("norm_path", 0)
    assert st == DPF_ERR_UNSUPPORTED
    assert b"static scratch" in msg
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(norms == -2.0)
