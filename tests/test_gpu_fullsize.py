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
from tests.gpu_helpers import max_rel, need_gpu, rel_fro, run_dense

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
    ref0 = ref - lin.sigma * lin.C * dp_linear.noise_matrix(lin.seed, lin.offset, ref.shape) / lin.B
    err0 = rel_fro(out0, ref0)
    assert err0 <= SUM_TOL, err0
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
