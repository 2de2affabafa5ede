"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element.

Tolerances (stated for the method: per-sample norms within 1e-3 relative;
the aggregated noisy gradient within 2e-2 relative Frobenius error for bf16
inputs with fp32 accumulation).  Derived, tighter bounds used in addition:
  * fp32 inputs: aggregate within 1e-4 relative Frobenius (fp32 MFMA, K small);
  * sigma = 0 companions (the clipped sum alone, which the noise would
    otherwise swamp): 1e-3 for bf16 -- the bf16 inputs are exact in the
    oracle, so only fp32 accumulation order differs (error ~1e-6);
  * projected variant: the GPU rounds Y = X P to bf16, adding ~2^-9 relative
    error per Y entry, so its sigma = 0 companion is held to 1e-2.
Shapes here are small enough for the oracle to finish in seconds but span
several 128-wide tiles in every dimension and end in ragged tails.
"""
import numpy as np
import pytest

import workloads
from oracle import dp_linear
from tests.gpu_helpers import (SUM_ELEM_TOL, assert_elementwise, assert_noise, mask_dev, max_rel,
                               need_gpu, random_linear, rel_fro, run_dense, to_dev)

pytestmark = pytest.mark.gpu

NORM_TOL = 1e-3
AGG_TOL_BF16 = 2e-2
AGG_TOL_F32 = 1e-4
SUM_TOL_BF16 = 1e-3
# projected sigma = 0, element-wise against max|ref|: Y = X P is stored in the
# inputs' dtype on the GPU and kept in fp64 by the oracle (bf16: 2^-9 relative
# per Y entry; fp32: two chained fp32 contractions)
PROJ_ELEM_TOL = {"bf16": 1e-2, "f32": 1e-4}


def _oracle(lin, C=None, sigma=None, offset=None):
    return dp_linear.oracle_linear(lin.X, lin.G, lin.mask, lin.C if C is None else C,
                                   lin.sigma if sigma is None else sigma, lin.seed,
                                   lin.offset if offset is None else offset, lin.dtype)


def _check(lin, path, sigma, C=None, agg_tol=None):
    """The call against the oracle: norms, the aggregate (relative Frobenius),
    and element by element the clipped sum (sigma = 0) and, for sigma > 0,
    the noise out(sigma) - out(0)."""
    torch = need_gpu()
    Cv = lin.C if C is None else C
    out, norms = run_dense(lin, torch, C=C, sigma=sigma, path=path)
    ref, rnorms, _ = _oracle(lin, C=C, sigma=sigma)
    assert max_rel(norms, rnorms) <= NORM_TOL, (max_rel(norms, rnorms), norms, rnorms)
    tol = agg_tol if agg_tol is not None else (AGG_TOL_F32 if lin.dtype == "f32" else AGG_TOL_BF16)
    err = rel_fro(out, ref)
    assert err <= tol, err
    if sigma == 0.0:
        assert_elementwise(out, ref, SUM_ELEM_TOL[lin.dtype], "sigma = 0")
    else:
        out0, _ = run_dense(lin, torch, C=C, sigma=0.0, path=path)
        xi = dp_linear.noise_matrix(lin.seed, lin.offset, ref.shape)
        ref0 = ref - sigma * Cv * xi / lin.B
        assert_elementwise(out0, ref0, SUM_ELEM_TOL[lin.dtype], "sigma = 0 companion")
        assert_noise(out, out0, sigma, Cv, lin.seed, lin.offset, lin.B, "noise", xi=xi)
    return out, norms, ref, rnorms


# ---------------------------------------------------------------------------
# small multi-tile shapes with ragged tails, both norm paths, both dtypes
# ---------------------------------------------------------------------------
SHAPES = [
    (3, 200, 264, 136),     # 2 token tiles (128 + 72), 3 x 2 output tiles with tails
    (2, 130, 128, 256),     # exact tile widths, a 2-token tail
    (1, 1, 8, 8),           # T = 1 outer product
    (4, 16, 64, 32),        # the single-linear fp32 configuration's shape
]


# norm paths: 1 Gram, 2 direct (tiles dropped, second contraction), 3 staged
# (bf16 large-tile calls: tiles stored once, then combined; elsewhere direct)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("path", [1, 2, 3])
@pytest.mark.parametrize("shape", SHAPES)
def test_dense_small_mixed_clip(dtype, path, shape):
    B, T, din, dout = shape
    rng = np.random.default_rng(hash((B, T, din, dout)) % 2**32)
    lin = random_linear(rng, B, T, din, dout, dtype=dtype)
    # clip norm at the median norm: some samples clip, some do not
    _, rnorms, _ = _oracle(lin, C=1.0, sigma=0.0)
    C = float(np.median(rnorms)) * 1.0001 if B > 1 else float(rnorms[0]) * 0.5
    tol = AGG_TOL_F32 if dtype == "f32" else SUM_TOL_BF16
    _check(lin, path, sigma=0.0, C=C, agg_tol=tol)
    _check(lin, path, sigma=0.9, C=C)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("path", [1, 2])
def test_dense_odd_dims_scalar_loads(dtype, path):
    rng = np.random.default_rng(5)
    lin = random_linear(rng, 3, 45, 37, 19, dtype=dtype, masked=True)
    _, rn, _ = _oracle(lin, C=1.0, sigma=0.0)
    C = float(np.median(rn))
    _check(lin, path, sigma=0.0, C=C, agg_tol=AGG_TOL_F32 if dtype == "f32" else SUM_TOL_BF16)
    _check(lin, path, sigma=1.3, C=C)


@pytest.mark.parametrize("path", [1, 2, 3])
def test_dense_ragged_prefix_masks(path):
    rng = np.random.default_rng(6)
    lengths = [300, 0, 1, 129, 64, 65]
    lin = random_linear(rng, 6, 300, 192, 320, lengths=lengths)
    _, rn, _ = _oracle(lin, C=1.0, sigma=0.0)
    assert rn[1] == 0.0
    C = float(np.median(rn[rn > 0]))
    out, norms, _, _ = _check(lin, path, sigma=0.0, C=C, agg_tol=SUM_TOL_BF16)
    assert norms[1] == 0.0
    _check(lin, path, sigma=1.2, C=C)


@pytest.mark.parametrize("path", [1, 2, 3])
def test_dense_random_mask(path):
    rng = np.random.default_rng(7)
    lin = random_linear(rng, 4, 257, 136, 72, masked=True)
    _, rn, _ = _oracle(lin, C=1.0, sigma=0.0)
    _check(lin, path, sigma=0.0, C=float(np.median(rn)), agg_tol=SUM_TOL_BF16)


@pytest.mark.parametrize("masked", [False, True])
def test_staged_multi_tile_ragged_edges(masked):
    """Staged path over 3 x 4 output tiles whose last row and column are
    partial, 10 token steps with a ragged tail, and (masked) a sample with
    no active token, whose staged tiles are all zero."""
    rng = np.random.default_rng(31)
    lengths = [300, 0, 77, 300] if masked else None
    lin = random_linear(rng, 4, 300, 520, 776, lengths=lengths)
    _, rn, _ = _oracle(lin, C=1.0, sigma=0.0)
    C = float(np.median(rn[rn > 0]))
    out, norms, _, _ = _check(lin, 3, sigma=0.0, C=C, agg_tol=SUM_TOL_BF16)
    if masked:
        assert norms[1] == 0.0
    _check(lin, 3, sigma=1.1, C=C)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(4, 16, 64, 32), (5, 33, 24, 40), (1, 1, 8, 8), (3, 30, 96, 64),
                                   (8, 9, 37, 19)])
def test_tiny_layer_kernel(dtype, shape):
    """The one-workgroup kernel (taken automatically for these shapes): masks
    with a fully masked sample, mixed clipping, noise, against the oracle."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    B, T, din, dout = shape
    X = torch.zeros((B, T, din), device="cuda")
    dp.timing_reset()
    dp.set_option("timing", 1)
    try:
        dp.linear_clip_accumulate(X, torch.zeros((B, T, dout), device="cuda"), None, C=1.0)
        assert "tiny_layer" in dp.timing_collect()
    finally:
        dp.set_option("timing", 0)
        dp.timing_reset()
    rng = np.random.default_rng(sum(shape))
    lengths = [T] + [0] + [max(1, T // 2)] * (B - 2) if B > 2 else None
    lin = random_linear(rng, B, T, din, dout, dtype=dtype, lengths=lengths)
    _, rn, _ = _oracle(lin, C=1.0, sigma=0.0)
    C = float(np.median(rn[rn > 0])) * 1.0001 if (rn > 0).sum() > 1 else float(rn.max()) * 0.5
    tol = AGG_TOL_F32 if dtype == "f32" else SUM_TOL_BF16
    _, norms, _, _ = _check(lin, 0, sigma=0.0, C=C, agg_tol=tol)
    if lengths is not None:
        assert norms[1] == 0.0
    _check(lin, 0, sigma=0.7, C=C)


def test_strided_views():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(8)
    lin = random_linear(rng, 3, 70, 96, 40, dtype="bf16")
    Xb = np.zeros((3, 70, 96 + 24), np.uint16)
    Xb[:, :, :96] = lin.X
    Gb = np.zeros((3, 70 + 5, 40 + 8), np.uint16)
    Gb[:, :70, :40] = lin.G
    X = to_dev(Xb, "bf16", torch)[:, :, :96]
    G = to_dev(Gb, "bf16", torch)[:, :70, :40]
    out, norms = dp.linear_clip_accumulate(X, G, None, C=0.05, sigma=0.0)
    ref, rn, _ = _oracle(lin, C=0.05, sigma=0.0)
    assert max_rel(norms.cpu().numpy(), rn) <= NORM_TOL
    assert rel_fro(out.cpu().numpy(), ref) <= SUM_TOL_BF16


# ---------------------------------------------------------------------------
# the five workload configurations
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("sigma", [0.0, 1.0])
@pytest.mark.parametrize("path", [0, 1, 2])   # 0: the automatic choice, the one-workgroup kernel
def test_config_single_fp32_linear(sigma, path):
    lin = workloads.config_c1(sigma).linears[0]
    _check(lin, path, sigma=sigma)


def test_config_gpt2_up_projection():
    lin = workloads.config_c2().linears[0]
    _, norms, ref, rn = _check(lin, 0, sigma=lin.sigma)
    _check(lin, 0, sigma=0.0, agg_tol=SUM_TOL_BF16)
    # mixed-clip supplement: C at the median oracle norm exercises c_i = 1
    _check(lin, 0, sigma=0.0, C=float(np.median(rn)), agg_tol=SUM_TOL_BF16)


@pytest.mark.parametrize("path", [1, 2, 3])
def test_config_gpt2_up_projection_forced_paths(path):
    lin = workloads.config_c2().linears[0]
    _check(lin, path, sigma=0.0, agg_tol=SUM_TOL_BF16)


@pytest.mark.parametrize("index", [0, 4, 5])
def test_config_roberta_projected(index):
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    from oracle import philox
    lin = workloads.config_c5_linear(index)
    r = 256
    # P from the oracle's own Philox (seed 7), fed to both sides
    P = workloads.f32_to_bf16_bits((philox.gaussian(7, 0, lin.din * r) / 16.0)
                                   .astype(np.float32)).reshape(lin.din, r)
    X, G = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch)
    Pd = to_dev(P, "bf16", torch)
    outs = {}
    for sigma, tol in ((lin.sigma, AGG_TOL_BF16), (0.0, 1e-2)):
        out, norms = dp.linear_clip_accumulate_projected(X, G, Pd, None, C=lin.C, sigma=sigma)
        ref, rn, _ = dp_linear.oracle_projected(lin.X, lin.G, None, P, lin.C, sigma, 0, 0, "bf16")
        assert max_rel(norms.cpu().numpy(), rn) <= NORM_TOL
        assert rel_fro(out.cpu().numpy(), ref) <= tol
        outs[sigma] = out.cpu().numpy()
    # element by element: the clipped sum (Y is rounded to bf16 on the GPU,
    # 2^-9 relative per entry, hence 1e-2 of the largest entry) and the noise
    assert_elementwise(outs[0.0], ref, PROJ_ELEM_TOL["bf16"], "projected sigma = 0")
    assert_noise(outs[lin.sigma], outs[0.0], lin.sigma, lin.C, 0, 0, lin.B, "projected noise")
    # end to end: P drawn on the GPU from Philox seed 7 (each side its own generator)
    Pg = dp.gaussian_fill(7, 0, lin.din * r, 1.0 / 16, dtype=torch.bfloat16).view(lin.din, r)
    out, norms = dp.linear_clip_accumulate_projected(X, G, Pg, None, C=lin.C, sigma=lin.sigma)
    ref, rn, _ = dp_linear.oracle_projected(lin.X, lin.G, None, P, lin.C, lin.sigma, 0, 0, "bf16")
    assert max_rel(norms.cpu().numpy(), rn) <= NORM_TOL
    assert rel_fro(out.cpu().numpy(), ref) <= AGG_TOL_BF16


def test_projected_small_masked_fp32_and_bf16():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(9)
    for dtype in ("f32", "bf16"):
        lin = random_linear(rng, 3, 150, 136, 72, dtype=dtype, lengths=[150, 20, 0])
        Pf = (rng.standard_normal((136, 40)) / np.sqrt(40)).astype(np.float32)
        P = workloads.f32_to_bf16_bits(Pf) if dtype == "bf16" else Pf
        X, G = to_dev(lin.X, dtype, torch), to_dev(lin.G, dtype, torch)
        out, norms = dp.linear_clip_accumulate_projected(X, G, to_dev(P, dtype, torch),
                                                         mask_dev(lin.mask, torch), C=0.02, sigma=0.0)
        ref, rn, _ = dp_linear.oracle_projected(lin.X, lin.G, lin.mask, P, 0.02, 0.0, 0, 0, dtype)
        tol_n = NORM_TOL if dtype == "f32" else 5e-3
        assert max_rel(norms.cpu().numpy()[rn > 0], rn[rn > 0]) <= tol_n
        assert norms.cpu().numpy()[2] == 0.0
        assert rel_fro(out.cpu().numpy(), ref) <= (AGG_TOL_F32 * 10 if dtype == "f32" else 1e-2)
        assert_elementwise(out.cpu().numpy(), ref, PROJ_ELEM_TOL[dtype], f"projected {dtype}")


@pytest.mark.parametrize("path", [0, 1])
def test_masked_gram_dead_row_blocks(path):
    """Masks that leave whole 256- and 128-token row blocks empty.

    The Gram kernel works on (256-token block, 128-token block) items of a
    sample and skips those with an empty block.  Sample 0 has tokens only
    in [300, 512) (its first 256-token block is empty), sample 1 one token at
    129, sample 2 none (norm 0), sample 3 every other token.  With
    din + dout = 5120 features and few live items, the items also split over
    several workgroups.
    """
    rng = np.random.default_rng(11)
    lin = random_linear(rng, 4, 512, 2048, 3072)
    mask = np.zeros((4, 512), np.uint8)
    mask[0, 300:] = 1
    mask[1, 129] = 1
    mask[3, ::2] = 1
    lin.mask = mask
    _, rn, _ = _oracle(lin, C=1.0, sigma=0.0)
    assert rn[2] == 0.0 and (rn[[0, 1, 3]] > 0).all()
    C = float(np.median(rn[[0, 1, 3]]))
    out, norms, _, _ = _check(lin, path, sigma=0.0, C=C, agg_tol=SUM_TOL_BF16)
    assert norms[2] == 0.0
    _check(lin, path, sigma=0.7, C=C)


@pytest.mark.parametrize("B", [8, 16])
def test_gram_items_split_over_all_workgroups(B):
    """Unmasked Gram calls whose items all fall in a split last round: T = 300
    gives 3 items per sample (2 of them diagonal), 1024 + 1024 features a
    64-step item, so 24 (48) items split into 5 pieces each over the
    workgroups, with the fixup summing them.  The norms, the clipped sum and
    the noise against the oracle, with mixed clipping (C at the median
    norm)."""
    rng = np.random.default_rng(40 + B)
    lin = random_linear(rng, B, 300, 1024, 1024)
    _, rn, _ = _oracle(lin, C=1.0, sigma=0.0)
    C = float(np.median(rn))
    _check(lin, 1, sigma=0.0, C=C, agg_tol=SUM_TOL_BF16)
    _check(lin, 1, sigma=0.6, C=C)


def test_gram_split_pieces_on_odd_steps_and_tail_chunks():
    """The Gram kernel loads 64-feature chunks but computes and splits in
    32-feature steps.  300 samples of T = 40 give 300 one-block items: 256 in
    the full round, 44 split.  din = 1096 (35 steps; its last chunk holds 8
    features) and dout = 520 (17 steps) make 52 steps, which the plan cuts
    into 3 pieces: X steps [0, 17) (ends half way into a chunk), [17, 34)
    (starts half way into one), and the single step [34, 35) (the 8-feature
    tail chunk) followed by all of G.  Norms and the clipped sum against the
    oracle, with mixed clipping."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(47)
    lin = random_linear(rng, 300, 40, 1096, 520)
    _, rn, _ = _oracle(lin, C=1.0, sigma=0.0)
    C = float(np.median(rn))
    dp.timing_reset()
    dp.set_option("timing", 1)
    try:
        _check(lin, 1, sigma=0.0, C=C, agg_tol=SUM_TOL_BF16)
        kernels = dp.timing_collect()
    finally:
        dp.set_option("timing", 0)
        dp.timing_reset()
    assert "gram_norm" in kernels and "gram_fixup" in kernels, sorted(kernels)


@pytest.mark.parametrize("hole", [False, True])
def test_prefix_mask_pieces_across_samples(hole):
    """Prefix masks (padding at the end) are walked by each sample's step
    range, other masks by the active-step list.  One 256 x 256 output tile
    over 54 active steps is split into 13 pieces of about 4 steps, so
    pieces start inside samples, right after samples with no token, and
    cross sample boundaries.  Lengths include multiples of 32 (a full last
    step), single tokens and empty samples; with `hole` one token inside a
    sample is masked as well, which makes the mask no prefix.  Norms and the
    clipped sum (mixed clipping) and the noise against the oracle."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    lengths = [512, 0, 64, 1, 33, 0, 0, 480, 32, 511, 2, 0]
    rng = np.random.default_rng(48)
    lin = random_linear(rng, len(lengths), 512, 256, 256, lengths=lengths)
    if hole:
        lin.mask[7, 100] = 0
    _, rn, _ = _oracle(lin, C=1.0, sigma=0.0)
    C = float(np.median(rn[rn > 0]))
    dp.timing_reset()
    dp.set_option("timing", 1)
    try:
        _check(lin, 0, sigma=0.0, C=C, agg_tol=SUM_TOL_BF16)
        _check(lin, 0, sigma=0.7, C=C)
        kernels = dp.timing_collect()
    finally:
        dp.set_option("timing", 0)
        dp.timing_reset()
    assert "accumulate_fixup" in kernels, sorted(kernels)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(2, 100, 1000, 72), (3, 33, 1000, 70)])
def test_projected_split_along_din(dtype, shape):
    """din = 1000 is long enough for the projection to split along din into
    fp32 chunks summed in order; din, r and B*T*r all end in ragged tails."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    B, T, din, r = shape
    rng = np.random.default_rng(12)
    lin = random_linear(rng, B, T, din, 96, dtype=dtype, lengths=[T - 7] + [T] * (B - 1))
    Pf = (rng.standard_normal((din, r)) / np.sqrt(r)).astype(np.float32)
    P = workloads.f32_to_bf16_bits(Pf) if dtype == "bf16" else Pf
    X, G = to_dev(lin.X, dtype, torch), to_dev(lin.G, dtype, torch)
    out, norms = dp.linear_clip_accumulate_projected(X, G, to_dev(P, dtype, torch),
                                                     mask_dev(lin.mask, torch), C=0.05, sigma=0.0)
    ref, rn, _ = dp_linear.oracle_projected(lin.X, lin.G, lin.mask, P, 0.05, 0.0, 0, 0, dtype)
    assert max_rel(norms.cpu().numpy(), rn) <= (NORM_TOL if dtype == "f32" else 5e-3)
    assert rel_fro(out.cpu().numpy(), ref) <= (AGG_TOL_F32 * 10 if dtype == "f32" else 1e-2)
    assert_elementwise(out.cpu().numpy(), ref, PROJ_ELEM_TOL[dtype], f"projected split {dtype}")


def _projected_case(rng, dtype, B, T, din, dout, r, lengths):
    lin = random_linear(rng, B, T, din, dout, dtype=dtype, lengths=lengths)
    Pf = (rng.standard_normal((din, r)) / np.sqrt(r)).astype(np.float32)
    P = workloads.f32_to_bf16_bits(Pf) if dtype == "bf16" else Pf
    return lin, P


_LEN32 = [50, 0, 1, 49, 50, 7, 50, 33] * 4


@pytest.mark.parametrize("tiles", [0, 1, 2])
@pytest.mark.parametrize("dtype,B,T,din,dout,r,lengths", [
    # 4 tiles of 128 x 128 in r space (a tail in r), 32 pieces of one
    # sample; empty and one-token samples
    ("bf16", 32, 50, 72, 256, 136, _LEN32),
    # 15 tiles with ragged tails in r and dout, 20 samples over 17 pieces
    # (pieces of one and two samples), three 64-token steps per sample
    ("bf16", 20, 150, 64, 520, 264, None),
    # fp32, 2 tiles, 6 pieces, samples of 1 and 0 tokens
    ("f32", 6, 70, 40, 200, 40, [70, 1, 35, 0, 70, 12]),
])
def test_projected_rspace_tiles(tiles, dtype, B, T, din, dout, r, lengths):
    """The r-space sum of the projected call on each "rspace_tiles" setting
    (0: 256 x 256 tiles; 1: 128 x 128 tiles whose samples are cut into
    pieces, their parts added in order by a second kernel; 2: that and the
    direct norm on 128 x 128 tiles) against the oracle: the norms, the
    clipped sum element by element (mixed clipping, C at the median norm) and
    the noise; each setting bitwise repeatable.  The shapes are ones the
    pieces take (enough pieces to fill half the compute units)."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    rng = np.random.default_rng(70 + B)
    lin, P = _projected_case(rng, dtype, B, T, din, dout, r, lengths)
    _, rn, _ = dp_linear.oracle_projected(lin.X, lin.G, lin.mask, P, 1.0, 0.0, 0, 0, dtype)
    C = float(np.median(rn[rn > 0]))
    X, G = to_dev(lin.X, dtype, torch), to_dev(lin.G, dtype, torch)
    Pd, m = to_dev(P, dtype, torch), mask_dev(lin.mask, torch)
    old = dp.get_option("rspace_tiles")
    dp.set_option("rspace_tiles", tiles)
    try:
        outs = {}
        for sigma in (0.0, 0.9):
            out, norms = dp.linear_clip_accumulate_projected(X, G, Pd, m, C=C, sigma=sigma,
                                                             seed=3, offset=5)
            again, _ = dp.linear_clip_accumulate_projected(X, G, Pd, m, C=C, sigma=sigma,
                                                           seed=3, offset=5)
            torch.cuda.synchronize()
            assert torch.equal(out, again), "not bitwise repeatable"
            outs[sigma] = out.cpu().numpy()
            nrm = norms.cpu().numpy()
        ref, rn, _ = dp_linear.oracle_projected(lin.X, lin.G, lin.mask, P, C, 0.0, 3, 5, dtype)
        tol_n = NORM_TOL if dtype == "f32" else 5e-3
        live = rn > 0
        assert max_rel(nrm[live], rn[live]) <= tol_n
        assert (nrm[~live] == 0.0).all()
        assert_elementwise(outs[0.0], ref, PROJ_ELEM_TOL[dtype], f"rspace_tiles {tiles} sigma = 0")
        assert_noise(outs[0.9], outs[0.0], 0.9, C, 3, 5, B, f"rspace_tiles {tiles} noise")
    finally:
        dp.set_option("rspace_tiles", old)


@pytest.mark.parametrize("tiles", [0, 2])
@pytest.mark.parametrize("index", [0, 4])
def test_config_roberta_projected_rspace_tiles(index, tiles):
    """The RoBERTa-large projected linears q (1024 -> 1024) and fc1 (1024 ->
    4096) on the other "rspace_tiles" settings (the default, 1, is the
    projected configuration test above) against the oracle."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    from oracle import philox
    lin = workloads.config_c5_linear(index)
    r = 256
    P = workloads.f32_to_bf16_bits((philox.gaussian(7, 0, lin.din * r) / 16.0)
                                   .astype(np.float32)).reshape(lin.din, r)
    X, G = to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch)
    Pd = to_dev(P, "bf16", torch)
    old = dp.get_option("rspace_tiles")
    dp.set_option("rspace_tiles", tiles)
    try:
        outs = {}
        for sigma in (lin.sigma, 0.0):
            out, norms = dp.linear_clip_accumulate_projected(X, G, Pd, None, C=lin.C, sigma=sigma)
            torch.cuda.synchronize()
            outs[sigma] = out.cpu().numpy()
            nrm = norms.cpu().numpy()
    finally:
        dp.set_option("rspace_tiles", old)
    ref, rn, _ = dp_linear.oracle_projected(lin.X, lin.G, None, P, lin.C, 0.0, 0, 0, "bf16")
    assert max_rel(nrm, rn) <= NORM_TOL
    assert_elementwise(outs[0.0], ref, PROJ_ELEM_TOL["bf16"], f"rspace_tiles {tiles} sigma = 0")
    assert_noise(outs[lin.sigma], outs[0.0], lin.sigma, lin.C, 0, 0, lin.B,
                 f"rspace_tiles {tiles} noise")
