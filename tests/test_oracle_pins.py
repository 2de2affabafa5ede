"""Pins for the CPU oracle: checks against things other than the oracle itself.

The FlashDP and DP-GRAPE pages print no worked example, so every pin here is
a closed form, an invariant, a textbook identity, brute force on tiny inputs,
or agreement with an independent library (rocRAND's Philox4x32-10 engine).
The last group plants mistakes in the oracle (on the CPU) and checks that at
least one pin catches each of them.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import dp_linear, optim, philox
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def _rand_case(rng, B, T, din, dout, masked=False, dtype="f32"):
    X = rng.standard_normal((B, T, din)).astype(np.float32)
    G = (0.3 * rng.standard_normal((B, T, dout))).astype(np.float32)
    mask = None
    if masked:
        mask = (rng.random((B, T)) < 0.6).astype(np.uint8)
    if dtype == "bf16":
        return f32_to_bf16_bits(X), f32_to_bf16_bits(G), mask
    return X, G, mask


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------
# Philox4x32-10 against rocRAND (independent library implementation)
# --------------------------------------------------------------------------
@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference helper")
    out = tmp_path_factory.mktemp("rr") / "rocrand_philox_ref"
    src = os.path.join(HERE, "golden", "rocrand_philox_ref.cpp")
    subprocess.run([hipcc, "-x", "c++", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                    "-O1", src, "-o", str(out)], check=True, capture_output=True)

    def run(pairs):
        text = "".join(f"{s} {b}\n" for s, b in pairs)
        res = subprocess.run([str(out)], input=text, capture_output=True, text=True, check=True)
        return [list(map(int, line.split())) for line in res.stdout.strip().splitlines()]
    return run


def _philox_cases():
    rng = np.random.default_rng(123)
    pairs = [(0, 0), (0, 1), (7, 0), (1, 2**32 - 1), (1, 2**32), (3, 2**32 + 5),
             (2**64 - 1, 2**64 - 1), (0xDEADBEEFCAFEF00D, 2**63 + 17)]
    pairs += [(int(s), int(b)) for s, b in zip(rng.integers(0, 2**63, 40, dtype=np.int64),
                                               rng.integers(0, 2**40, 40, dtype=np.int64))]
    return pairs


def test_philox_scalar_matches_rocrand(rocrand_ref):
    pairs = _philox_cases()
    ref = rocrand_ref(pairs)
    for (s, b), r in zip(pairs, ref):
        assert philox.philox4x32_10(philox.block_counter(b), philox.seed_key(s)) == r, (s, b)


def test_philox_vector_matches_rocrand(rocrand_ref):
    pairs = [(5, b) for b in range(2**32 - 6, 2**32 + 6)]   # carry into hi32(block)
    ref = np.array(rocrand_ref(pairs), dtype=np.uint32)
    got = philox.philox_words(5, [b for _, b in pairs])
    np.testing.assert_array_equal(got, ref)


def test_philox_vector_matches_scalar():
    got = philox.philox_words(99, np.arange(1000, 1064, dtype=np.uint64))
    ref = np.array(philox.philox_words_scalar(99, 1000, 64), dtype=np.uint32)
    np.testing.assert_array_equal(got, ref)


# --------------------------------------------------------------------------
# uniform map and Box-Muller
# --------------------------------------------------------------------------
def test_uniform_map_endpoints():
    u = philox.words_to_uniform(np.array([0, 511, 512, 2**32 - 1], dtype=np.uint64))
    assert u[0] == 0.5 * 2.0 ** -23
    assert u[1] == u[0]                       # the low 9 bits are dropped
    assert u[2] == 1.5 * 2.0 ** -23
    assert u[3] == 1.0 - 2.0 ** -24
    assert np.all((u > 0) & (u < 1))
    assert np.all(u.astype(np.float32).astype(np.float64) == u)   # exact in fp32


def test_box_muller_closed_forms():
    z0, z1 = philox.box_muller(np.array([math.exp(-0.5)]), np.array([0.0]))
    assert abs(z0[0] - 1.0) < 1e-15 and abs(z1[0]) < 1e-15
    z0, z1 = philox.box_muller(np.array([math.exp(-2.0)]), np.array([0.25]))
    assert abs(z0[0]) < 1e-15 and abs(z1[0] - 2.0) < 1e-15
    z0, z1 = philox.box_muller(np.array([math.exp(-4.5)]), np.array([0.5]))
    assert abs(z0[0] + 3.0) < 1e-14 and abs(z1[0]) < 1e-14


def test_box_muller_lane_pairing():
    """z0, z1 come from (u0, u1) and z2, z3 from (u2, u3)."""
    w = philox.philox_words(11, np.arange(4, dtype=np.uint64))
    u = philox.words_to_uniform(w)
    z = philox.normals_of_words(w)
    r01 = np.sqrt(-2 * np.log(u[:, 0]))
    r23 = np.sqrt(-2 * np.log(u[:, 2]))
    np.testing.assert_allclose(z[:, 0] ** 2 + z[:, 1] ** 2, r01 ** 2, rtol=1e-12)
    np.testing.assert_allclose(z[:, 2] ** 2 + z[:, 3] ** 2, r23 ** 2, rtol=1e-12)
    np.testing.assert_allclose(np.arctan2(z[:, 1], z[:, 0]) % (2 * np.pi),
                               (2 * np.pi * u[:, 1]) % (2 * np.pi), atol=1e-9)


def test_gaussian_statistics():
    from scipy import stats
    z = philox.gaussian(0, 0, 2_000_000)
    assert abs(z.mean()) < 5e-3
    assert abs(z.var() - 1.0) < 5e-3
    assert stats.kstest(z, "norm").pvalue > 1e-4
    zz = z.reshape(-1, 2)
    assert abs(np.corrcoef(zz[:, 0], zz[:, 1])[0, 1]) < 5e-3
    # 23-bit uniforms cap |z| at sqrt(-2 ln 2**-24) ~ 5.77
    assert np.abs(z).max() <= math.sqrt(-2 * math.log(0.5 * 2.0 ** -23)) + 1e-12


def test_gaussian_scalar_matches_vector():
    np.testing.assert_allclose(philox.gaussian_scalar(3, 17, 37), philox.gaussian(3, 17, 37),
                               rtol=0, atol=1e-14)


def test_gaussian_offset_concatenation():
    n = 4 * 257
    whole = philox.gaussian(42, 10, 2 * n)
    first = philox.gaussian(42, 10, n)
    second = philox.gaussian(42, 10 + philox.noise_blocks(n), n)
    np.testing.assert_array_equal(whole, np.concatenate([first, second]))


def test_gaussian_at_matches_gaussian():
    full = philox.gaussian(9, 5, 1001)
    idx = np.array([0, 1, 2, 3, 4, 999, 1000, 517])
    np.testing.assert_array_equal(philox.gaussian_at(9, 5, idx), full[idx])


# --------------------------------------------------------------------------
# the clip-and-accumulate oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("masked", [False, True])
def test_oracle_matches_brute_force(masked):
    rng = np.random.default_rng(1)
    X, G, mask = _rand_case(rng, 3, 4, 5, 4, masked)
    C = 0.9
    out, norms, c = dp_linear.oracle_linear(X, G, mask, C, 0.0, 0, 0, "f32")
    S, bn = dp_linear.brute_force_linear(X.astype(np.float64).tolist(),
                                         G.astype(np.float64).tolist(),
                                         None if mask is None else mask.tolist(), C)
    np.testing.assert_allclose(norms, bn, rtol=1e-12)
    np.testing.assert_allclose(out * 3, np.array(S), rtol=1e-12, atol=1e-14)


def test_t1_closed_form():
    """T = 1: g_i is the outer product G_i X_i^T, so ||g_i|| = ||G_i|| ||X_i||."""
    rng = np.random.default_rng(2)
    X, G, _ = _rand_case(rng, 5, 1, 7, 6)
    _, norms, _ = dp_linear.oracle_linear(X, G, None, 1.0, 0.0, 0, 0, "f32")
    ref = np.linalg.norm(G.astype(np.float64)[:, 0, :], axis=1) * \
        np.linalg.norm(X.astype(np.float64)[:, 0, :], axis=1)
    np.testing.assert_allclose(norms, ref, rtol=1e-12)


def test_gram_identity():
    """||G^T X||_F^2 = <X X^T, G G^T>_F (the Gram-norm identity)."""
    rng = np.random.default_rng(3)
    X, G, mask = _rand_case(rng, 4, 9, 11, 13, masked=True)
    _, norms, _ = dp_linear.oracle_linear(X, G, mask, 1.0, 0.0, 0, 0, "f32")
    for i in range(4):
        keep = mask[i].astype(bool)
        x = X[i].astype(np.float64)[keep]
        g = G[i].astype(np.float64)[keep]
        gram = np.sum((x @ x.T) * (g @ g.T))
        assert abs(norms[i] ** 2 - gram) <= 1e-12 * max(gram, 1e-300)


def test_no_clip_no_noise_is_plain_gradient():
    """C -> inf, sigma = 0: out = (sum over all rows of G~^T X~) / B, one big GEMM."""
    rng = np.random.default_rng(4)
    X, G, mask = _rand_case(rng, 3, 6, 8, 5, masked=True)
    out, _, c = dp_linear.oracle_linear(X, G, mask, 1e30, 0.0, 0, 0, "f32")
    assert np.all(c == 1.0)
    keep = mask.reshape(-1).astype(bool)
    Xf = X.reshape(-1, 8).astype(np.float64)[keep]
    Gf = G.reshape(-1, 5).astype(np.float64)[keep]
    np.testing.assert_allclose(out, Gf.T @ Xf / 3, rtol=1e-12, atol=1e-15)


def test_clip_invariant():
    rng = np.random.default_rng(5)
    X, G, _ = _rand_case(rng, 8, 5, 6, 7)
    G = G * (10.0 ** np.arange(-4, 4)[:, None, None]).astype(np.float32)
    C = 0.7
    _, norms, c = dp_linear.oracle_linear(X, G, None, C, 0.0, 0, 0, "f32")
    assert np.all(c * norms <= C * (1 + 1e-12))
    assert np.all((c == 1.0) == (norms <= C))
    assert (c < 1).any() and (c == 1).any()


def test_single_sample_clipped_norm():
    """B = 1, sigma = 0: ||B out|| = min(n_1, C)."""
    rng = np.random.default_rng(6)
    X, G, _ = _rand_case(rng, 1, 7, 9, 4)
    for C in (1e-3, 1e3):
        out, norms, _ = dp_linear.oracle_linear(X, G, None, C, 0.0, 0, 0, "f32")
        assert abs(np.linalg.norm(out) - min(norms[0], C)) <= 1e-12 * min(norms[0], C)


def test_scale_invariance_of_clipped_sample():
    rng = np.random.default_rng(7)
    X, G, _ = _rand_case(rng, 3, 5, 6, 4)
    C = 1e-2
    out1, n1, c1 = dp_linear.oracle_linear(X, G, None, C, 0.0, 0, 0, "f32")
    assert np.all(c1 < 1)
    G2 = G.astype(np.float64)
    G2[1] *= 8.0                               # exact in fp32
    out2, _, _ = dp_linear.oracle_linear(X, G2.astype(np.float32), None, C, 0.0, 0, 0, "f32")
    np.testing.assert_allclose(out2, out1, rtol=1e-12, atol=1e-16)


def test_permutation_invariance():
    rng = np.random.default_rng(8)
    X, G, mask = _rand_case(rng, 5, 4, 6, 3, masked=True)
    p = np.array([3, 0, 4, 1, 2])
    o1, n1, _ = dp_linear.oracle_linear(X, G, mask, 0.5, 0.0, 0, 0, "f32")
    o2, n2, _ = dp_linear.oracle_linear(X[p], G[p], mask[p], 0.5, 0.0, 0, 0, "f32")
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(n2, n1[p], rtol=1e-14)


def test_batch_split_linearity():
    rng = np.random.default_rng(9)
    X, G, _ = _rand_case(rng, 6, 4, 5, 3)
    C = 0.3
    o_all, _, _ = dp_linear.oracle_linear(X, G, None, C, 0.0, 0, 0, "f32")
    o_a, _, _ = dp_linear.oracle_linear(X[:2], G[:2], None, C, 0.0, 0, 0, "f32")
    o_b, _, _ = dp_linear.oracle_linear(X[2:], G[2:], None, C, 0.0, 0, 0, "f32")
    np.testing.assert_allclose(6 * o_all, 2 * o_a + 4 * o_b, rtol=1e-12, atol=1e-15)


def test_parts_with_the_whole_batch_denominator_add_up():
    """Micro-batches (or per-device shares) called with the whole batch's
    size as the denominator, the noise in one of them and the results added
    into one buffer, give the call on the whole batch: clipping stays per
    sample, so the split changes nothing."""
    rng = np.random.default_rng(11)
    X, G, _ = _rand_case(rng, 6, 4, 5, 3)
    C, sigma = 0.3, 0.7
    whole, _, _ = dp_linear.oracle_linear(X, G, None, C, sigma, 4, 9, "f32")
    acc, _, _ = dp_linear.oracle_linear(X[:2], G[:2], None, C, sigma, 4, 9, "f32", denom=6)
    acc, _, _ = dp_linear.oracle_linear(X[2:5], G[2:5], None, C, 0.0, 4, 9, "f32", denom=6,
                                        out0=acc)
    acc, _, _ = dp_linear.oracle_linear(X[5:], G[5:], None, C, 0.0, 4, 9, "f32", denom=6,
                                        out0=acc)
    np.testing.assert_allclose(acc, whole, rtol=1e-12, atol=1e-15)


def test_denominator_defaults_to_the_batch_size():
    rng = np.random.default_rng(12)
    X, G, _ = _rand_case(rng, 3, 4, 5, 3)
    o1, _, _ = dp_linear.oracle_linear(X, G, None, 0.3, 0.5, 1, 2, "f32")
    o2, _, _ = dp_linear.oracle_linear(X, G, None, 0.3, 0.5, 1, 2, "f32", denom=3)
    o3, _, _ = dp_linear.oracle_linear(X, G, None, 0.3, 0.5, 1, 2, "f32", denom=6)
    assert np.array_equal(o1, o2)
    assert np.array_equal(o3, o1 / 2)


def test_mask_equals_unpadded_calls_and_ignores_padding():
    rng = np.random.default_rng(10)
    B, T, din, dout = 4, 9, 5, 6
    X, G, _ = _rand_case(rng, B, T, din, dout)
    lengths = np.array([9, 1, 4, 0])
    mask = (np.arange(T)[None, :] < lengths[:, None]).astype(np.uint8)
    C = 0.8
    out, norms, _ = dp_linear.oracle_linear(X, G, mask, C, 0.0, 0, 0, "f32")
    S = np.zeros((dout, din))
    for i in range(B):
        if lengths[i] == 0:
            assert norms[i] == 0.0
            continue
        o_i, n_i, _ = dp_linear.oracle_linear(X[i:i + 1, :lengths[i]], G[i:i + 1, :lengths[i]],
                                              None, C, 0.0, 0, 0, "f32")
        S += o_i
        assert abs(n_i[0] - norms[i]) <= 1e-13 * n_i[0]
    np.testing.assert_allclose(out * B, S, rtol=1e-12, atol=1e-15)
    Xn, Gn = X.copy(), G.copy()
    Xn[mask == 0] = np.nan
    Gn[mask == 0] = np.inf
    out2, norms2, _ = dp_linear.oracle_linear(Xn, Gn, mask, C, 0.0, 0, 0, "f32")
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(norms2, norms)


def test_bias_is_the_weight_of_a_constant_input():
    """Appending a constant-one column to X turns the bias into one more weight
    column: without noise the bias variant equals the dense oracle on [X, 1]
    (the masked rows of the extra column are selected away like the rest)."""
    rng = np.random.default_rng(35)
    B, T, din, dout = 4, 6, 5, 3
    X, G, mask = _rand_case(rng, B, T, din, dout, masked=True)
    Xa = np.concatenate([X, np.ones((B, T, 1), np.float32)], axis=2)
    C = 0.4
    ow, ob, n, c = dp_linear.oracle_linear_bias(X, G, mask, C, 0.0, 0, 0, "f32")
    oa, na, ca = dp_linear.oracle_linear(Xa, G, mask, C, 0.0, 0, 0, "f32")
    assert (c < 1).any()
    np.testing.assert_allclose(ow, oa[:, :din], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(ob, oa[:, din], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(n, na, rtol=1e-13)


def test_bias_noise_continues_the_weight_stream():
    """X = 0 and G = 0: both outputs are pure noise, the bias's drawn from the
    blocks right after the weight's."""
    B, T, din, dout = 2, 3, 6, 5          # 30 weight elements: 8 blocks (the last one partly used)
    X = np.zeros((B, T, din), np.float32)
    G = np.zeros((B, T, dout), np.float32)
    ow, ob, n, c = dp_linear.oracle_linear_bias(X, G, None, 0.5, 2.0, 9, 4, "f32")
    assert (n == 0).all() and (c == 1).all()
    z = philox.gaussian_scalar(9, 4, 30)
    zb = philox.gaussian_scalar(9, 4 + 8, dout)
    np.testing.assert_allclose(ow.ravel(), 2.0 * 0.5 * np.array(z) / B, rtol=1e-12)
    np.testing.assert_allclose(ob, 2.0 * 0.5 * np.array(zb) / B, rtol=1e-12)


def test_group_of_one_is_per_layer():
    rng = np.random.default_rng(30)
    X, G, mask = _rand_case(rng, 4, 5, 6, 3, masked=True)
    outs, n_g, c_g = dp_linear.oracle_group([(X, G)], mask, 0.4, 0.9, 5, [7], "f32")
    o, n, c = dp_linear.oracle_linear(X, G, mask, 0.4, 0.9, 5, 7, "f32")
    np.testing.assert_allclose(outs[0], o, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(n_g, n, rtol=1e-14)
    np.testing.assert_array_equal(c_g == 1.0, c == 1.0)


def test_group_row_split_reproduces_whole_layer():
    """Cutting one linear's output rows into two linears with the same input:
    the group norm of the two halves is the norm of the whole gradient, so
    group clipping of the halves equals per-layer clipping of the whole (the
    noise follows the row-major element index, so the second half's offset
    is the first half's element count / 4)."""
    rng = np.random.default_rng(31)
    B, T, din, dout, d1 = 4, 6, 8, 10, 4
    X, G, mask = _rand_case(rng, B, T, din, dout, masked=True)
    C, sigma, seed, off = 0.3, 0.8, 11, 5
    whole, n_w, c_w = dp_linear.oracle_linear(X, G, mask, C, sigma, seed, off, "f32")
    outs, n_g, c_g = dp_linear.oracle_group([(X, G[:, :, :d1]), (X, G[:, :, d1:])], mask, C,
                                            sigma, seed, [off, off + d1 * din // 4], "f32")
    assert (c_w < 1).any()
    np.testing.assert_allclose(np.concatenate(outs, axis=0), whole, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(n_g, n_w, rtol=1e-13)


def test_group_clip_bounds_the_group_norm():
    rng = np.random.default_rng(32)
    lin = []
    for din, dout in ((5, 3), (4, 7), (6, 2)):
        X, G, _ = _rand_case(rng, 5, 4, din, dout)
        lin.append((X, G))
    C = 0.2
    _, norms, c = dp_linear.oracle_group(lin, None, C, 0.0, 0, [0, 0, 0], "f32")
    Xw = [dp_linear.widen(x, "f32") for x, _ in lin]
    Gw = [dp_linear.widen(g, "f32") for _, g in lin]
    for i in range(5):
        sq = sum(float(np.sum((Gw[l][i].T @ Xw[l][i]) ** 2)) for l in range(3))
        assert abs(math.sqrt(sq) - norms[i]) <= 1e-12 * norms[i]
        assert c[i] * norms[i] <= C * (1 + 1e-12)
        # each layer's norm alone would have clipped less
        assert c[i] <= min(1.0, C / math.sqrt(float(np.sum((Gw[0][i].T @ Xw[0][i]) ** 2))))


def test_projected_adam_first_step_closed_form():
    """m = v = 0, t = 1: m_hat = h, v_hat = h^2, so U = h / (|h| + eps)."""
    rng = np.random.default_rng(33)
    dout, din, r = 5, 7, 3
    h = rng.standard_normal((dout, r))
    W = rng.standard_normal((dout, din))
    P = rng.standard_normal((din, r))
    eps, lr = 1e-3, 0.05
    m, v, W1 = optim.projected_adam_step(h, np.zeros_like(h), np.zeros_like(h), W, 1, lr, 0.9,
                                         0.999, eps, P)
    np.testing.assert_allclose(W1, W - lr * (h / (np.abs(h) + eps)) @ P.T, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(m, 0.1 * h, rtol=1e-15)
    np.testing.assert_allclose(v, 0.001 * h * h, rtol=1e-12)


def test_projected_adam_identity_projection_is_torch_adam():
    """With P = I (r = din) the projected step is plain Adam: compare several
    steps against torch.optim.Adam (float64, CPU)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(34)
    dout, din = 4, 6
    W0 = rng.standard_normal((dout, din))
    p = torch.nn.Parameter(torch.tensor(W0, dtype=torch.float64))
    opt = torch.optim.Adam([p], lr=0.01, betas=(0.8, 0.95), eps=1e-6, foreach=False)
    m = np.zeros((dout, din))
    v = np.zeros((dout, din))
    W = W0.copy()
    I = np.eye(din)
    for t in range(1, 6):
        g = rng.standard_normal((dout, din)) * (0.1 * t)
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        m, v, W = optim.projected_adam_step(g, m, v, W, t, 0.01, 0.8, 0.95, 1e-6, I)
        np.testing.assert_allclose(W, p.detach().numpy(), rtol=1e-12, atol=1e-14)
        st = opt.state[p]
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-15)


def test_projection_identity_reduces_to_dense():
    rng = np.random.default_rng(11)
    X, G, mask = _rand_case(rng, 3, 5, 6, 4, masked=True)
    P = np.eye(6, dtype=np.float32)
    o1, n1, _ = dp_linear.oracle_linear(X, G, mask, 0.5, 0.7, 3, 2, "f32")
    o2, n2, _ = dp_linear.oracle_projected(X, G, mask, P, 0.5, 0.7, 3, 2, "f32")
    np.testing.assert_array_equal(o2, o1)
    np.testing.assert_array_equal(n2, n1)


def test_projection_associativity():
    """h_i = G~_i^T (X~_i P) equals (G~_i^T X~_i) P, so n_i = ||g_i P||."""
    rng = np.random.default_rng(12)
    X, G, mask = _rand_case(rng, 3, 5, 8, 4, masked=True)
    P = rng.standard_normal((8, 3)).astype(np.float32)
    _, n_proj, _ = dp_linear.oracle_projected(X, G, mask, P, 1.0, 0.0, 0, 0, "f32")
    for i in range(3):
        keep = mask[i].astype(bool)
        g = G[i].astype(np.float64)[keep].T @ X[i].astype(np.float64)[keep]
        assert abs(np.linalg.norm(g @ P.astype(np.float64)) - n_proj[i]) <= 1e-12 * n_proj[i]


def test_zero_activations_give_pure_noise():
    """X = 0: every norm is 0, every c_i = 1, out = sigma C xi / B."""
    B, T, din, dout = 3, 4, 6, 5
    X = np.zeros((B, T, din), np.float32)
    G = np.ones((B, T, dout), np.float32)
    sigma, C, seed, off = 1.3, 0.4, 77, 1234
    out, norms, c = dp_linear.oracle_linear(X, G, None, C, sigma, seed, off, "f32")
    assert np.all(norms == 0) and np.all(c == 1)
    xi = philox.gaussian(seed, off, din * dout).reshape(dout, din)
    np.testing.assert_allclose(out, sigma * C * xi / B, rtol=1e-15)


def test_entries_and_norms_helpers_agree_with_oracle():
    rng = np.random.default_rng(13)
    X, G, mask = _rand_case(rng, 4, 6, 10, 7, masked=True, dtype="bf16")
    C, sigma = 0.05, 0.9
    out, norms, c = dp_linear.oracle_linear(X, G, mask, C, sigma, 5, 3, "bf16")
    rows = np.array([0, 6, 3, 2])
    cols = np.array([9, 0, 4, 5])
    ent = dp_linear.oracle_entries(X, G, mask, c, rows, cols, sigma, C, 5, 3, "bf16")
    np.testing.assert_allclose(ent, out[rows, cols], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dp_linear.oracle_norms(X, G, mask, "bf16", samples=[2, 0]),
                               norms[[2, 0]], rtol=1e-14)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(14)
    a = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.0 ** -130, 3.0e38], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(a), ref)
    b = f32_to_bf16_bits(a)
    np.testing.assert_array_equal(f32_to_bf16_bits(bf16_bits_to_f32(b)), b)


def test_widen_bf16_matches_torch_on_every_bit_pattern():
    """widen(bits, "bf16") against torch's own bfloat16 -> float64 conversion,
    over all 65536 patterns (zeros, subnormals, infinities and NaNs included)."""
    torch = pytest.importorskip("torch")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = dp_linear.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127   # exponent all ones with a non-zero fraction, both signs
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_widen_f32_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(15)
    a = np.concatenate([rng.standard_normal(4096).astype(np.float32) * 1e3,
                        np.array([0.0, -0.0, 1e-45, -3.4e38, np.inf, -np.inf], np.float32)])
    got = dp_linear.widen(a, "f32")
    ref = torch.from_numpy(a).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(ref))


def _bf16_bits_by_torch(v32: np.ndarray) -> np.ndarray:
    torch = pytest.importorskip("torch")
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_projection_matrix_entries_follow_the_row_major_stream():
    """P[d, j] is normal number d*r + j of the (seed, offset) stream, computed
    here by the pure-Python scalar generator (itself pinned against rocRAND),
    scaled in float32, and for bf16 rounded by torch's conversion.  Reading of
    the DP-GRAPE explainer, Methodology, "Random Projection over SVD": the
    projection is drawn again from its seed, row-major over [din, r]."""
    seed, off, din, r = 7, 5, 37, 24
    scale = 1.0 / math.sqrt(r)
    z = philox.gaussian_scalar(seed, off, din * r)
    P32 = dp_linear.projection_matrix(seed, off, din, r, scale, "f32")
    P16 = dp_linear.projection_matrix(seed, off, din, r, scale, "bf16")
    assert P32.shape == (din, r) and P32.dtype == np.float32
    assert P16.shape == (din, r) and P16.dtype == np.uint16
    rng = np.random.default_rng(16)
    picks = [(0, 0), (0, 1), (1, 0), (din - 1, r - 1), (din - 1, 0), (0, r - 1)]
    picks += [(int(d), int(j)) for d, j in zip(rng.integers(0, din, 40), rng.integers(0, r, 40))]
    want32 = np.array([np.float32(scale) * np.float32(z[d * r + j]) for d, j in picks], np.float32)
    got32 = np.array([P32[d, j] for d, j in picks], np.float32)
    np.testing.assert_array_equal(got32, want32)
    np.testing.assert_array_equal(np.array([P16[d, j] for d, j in picks], np.uint16),
                                  _bf16_bits_by_torch(want32))
    # the whole matrix, bf16 against torch's rounding of the float32 matrix
    np.testing.assert_array_equal(P16, _bf16_bits_by_torch(P32))


def test_projection_matrix_moments():
    """Entries N(0, scale^2): sample mean and variance over 2^17 entries."""
    din, r = 512, 256
    s = 1.0 / math.sqrt(r)
    P = dp_linear.projection_matrix(7, 0, din, r, s, "f32").astype(np.float64)
    n = P.size
    assert abs(P.mean()) < 5.0 * s / math.sqrt(n)
    assert abs(P.var() / s ** 2 - 1.0) < 5.0 * math.sqrt(2.0 / n)
    # rows are not copies of each other and columns are uncorrelated
    c = np.corrcoef(P[:, 0], P[:, 1])[0, 1]
    assert abs(c) < 5.0 / math.sqrt(din)


# --------------------------------------------------------------------------
# planted mistakes: each must trip at least one pin
# --------------------------------------------------------------------------
def _pins_fail(fns):
    for fn in fns:
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


_DENSE_PINS = [
    lambda: test_oracle_matches_brute_force(True),
    test_t1_closed_form, test_gram_identity, test_no_clip_no_noise_is_plain_gradient,
    test_clip_invariant, test_single_sample_clipped_norm, test_mask_equals_unpadded_calls_and_ignores_padding,
    test_zero_activations_give_pure_noise,
]


def test_planted_transposed_operand(monkeypatch):
    monkeypatch.setattr(dp_linear, "per_sample_grad", lambda Xi, Gi: Xi.T @ Gi)
    assert _pins_fail(_DENSE_PINS)


def test_planted_clip_rule(monkeypatch):
    monkeypatch.setattr(dp_linear, "clip_factor", lambda n, C: C / n if n > 0 else 1.0)
    assert _pins_fail(_DENSE_PINS)


def test_planted_mask_as_product(monkeypatch):
    def mult(rows, mask_row):
        return rows if mask_row is None else rows * np.asarray(mask_row)[:, None]
    monkeypatch.setattr(dp_linear, "select_active", mult)
    assert _pins_fail(_DENSE_PINS)


def test_planted_noise_lane(monkeypatch):
    orig = philox.normals_of_words
    monkeypatch.setattr(philox, "normals_of_words", lambda w: orig(w)[:, [1, 0, 2, 3]])
    assert _pins_fail([test_box_muller_lane_pairing, test_gaussian_statistics])


def test_planted_philox_multiplier(monkeypatch, rocrand_ref):
    monkeypatch.setattr(philox, "PHILOX_M1", 0xCD9E8D55)
    assert _pins_fail([lambda: test_philox_scalar_matches_rocrand(rocrand_ref)])


def test_planted_noise_offset(monkeypatch):
    orig = dp_linear.noise_matrix
    monkeypatch.setattr(dp_linear, "noise_matrix", lambda s, o, sh: orig(s, o + 1, sh))
    assert _pins_fail(_DENSE_PINS)


def test_planted_noise_without_clip_norm(monkeypatch):
    # simulates out = (S + sigma xi) / B, i.e. the factor C dropped (C = 0.4 in the pin)
    orig = dp_linear.noise_matrix
    monkeypatch.setattr(dp_linear, "noise_matrix", lambda s, o, sh: orig(s, o, sh) / 0.4)
    assert _pins_fail(_DENSE_PINS)


def test_planted_dropped_sample(monkeypatch):
    orig = dp_linear.clip_accumulate
    monkeypatch.setattr(dp_linear, "clip_accumulate",
                        lambda gs, C: orig(list(gs)[:-1] or [np.zeros((1, 1))], C))
    assert _pins_fail(_DENSE_PINS)


def test_planted_widen_shift(monkeypatch):
    def wrong(a, dtype):
        a = np.asarray(a)
        if dtype == "bf16":
            return (a.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    monkeypatch.setattr(dp_linear, "widen", wrong)
    assert _pins_fail([test_widen_bf16_matches_torch_on_every_bit_pattern])


def test_planted_transposed_projection(monkeypatch):
    def transposed(seed, offset, din, r, scale, dtype="bf16"):
        z = philox.gaussian(seed, offset, din * r).astype(np.float32)
        v = (np.float32(scale) * z).astype(np.float32).reshape(r, din).T.copy()
        return v if dtype == "f32" else _bf16_bits_by_torch(v)
    monkeypatch.setattr(dp_linear, "projection_matrix", transposed)
    assert _pins_fail([test_projection_matrix_entries_follow_the_row_major_stream])
