"""Helpers for the GPU tests: uploading seeded numpy inputs and comparing with the oracle."""
import numpy as np
import pytest


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sample_gradient_clipping_amd as dp
    dp.load()   # raises if the HIP library is missing: no fallback
    return torch


def to_dev(a: np.ndarray, dtype: str, torch):
    """numpy float32 or uint16 (bf16 bits) -> GPU tensor of that dtype (bytes unchanged)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def mask_dev(mask, torch):
    return None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()


def rel_fro(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_rel(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)))


def run_dense(lin, torch, C=None, sigma=None, path=None, offset=None):
    import sample_gradient_clipping_amd as dp
    X = to_dev(lin.X, lin.dtype, torch)
    G = to_dev(lin.G, lin.dtype, torch)
    m = mask_dev(lin.mask, torch)
    if path is not None:
        dp.set_option("norm_path", path)
    try:
        out, norms = dp.linear_clip_accumulate(
            X, G, m, C=lin.C if C is None else C, sigma=lin.sigma if sigma is None else sigma,
            seed=lin.seed, offset=lin.offset if offset is None else offset)
        torch.cuda.synchronize()
    finally:
        dp.set_option("norm_path", 0)
    return out.cpu().numpy(), norms.cpu().numpy()


def random_linear(rng, B, T, din, dout, dtype="bf16", masked=False, C=1.0, sigma=0.0,
                  g_scale=1e-2, lengths=None, seed=0, offset=0):
    """Small seeded case with per-sample lognormal scales (mix of clipped/unclipped)."""
    from workloads import Linear, f32_to_bf16_bits
    X = rng.standard_normal((B, T, din), dtype=np.float32)
    s = rng.lognormal(0.0, 1.0, B).astype(np.float32)
    G = (rng.standard_normal((B, T, dout), dtype=np.float32) * (s * g_scale)[:, None, None]).astype(np.float32)
    mask = None
    if lengths is not None:
        mask = (np.arange(T)[None, :] < np.asarray(lengths)[:, None]).astype(np.uint8)
    elif masked:
        mask = (rng.random((B, T)) < 0.7).astype(np.uint8)
    if dtype == "bf16":
        X, G = f32_to_bf16_bits(X), f32_to_bf16_bits(G)
    return Linear("rand", X, G, mask, C, sigma, seed, offset, dtype)


# Element-wise bounds (in addition to the stated relative-Frobenius ones):
# a sigma = 0 output against the oracle, max|got - ref| <= tol * max|ref|,
# with tol 1e-3 for bf16 inputs (exact in the oracle: only the fp32
# accumulation order differs) and 1e-5 for fp32 inputs; and the noise, taken
# as out(sigma) - out(0) of two GPU calls that differ only in sigma, against
# sigma * C * xi / denom with xi from the oracle's own Philox + Box-Muller,
# to 1e-5 * sigma * C / denom absolute (fp32 normals are within 7e-7 of the
# fp64 ones for |z| <= 5.8; the fp32 roundings of the epilogue add ~1e-7).
SUM_ELEM_TOL = {"bf16": 1e-3, "f32": 1e-5}
NOISE_ELEM_TOL = 1e-5


def assert_elementwise(got, ref, tol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    assert np.isfinite(err) and err <= tol * scale, (
        f"{what}: max|got - ref| = {err:.3e} > {tol:g} * max|ref| = {tol * scale:.3e}")
    return err / scale if scale > 0 else 0.0


def assert_noise(out_sigma, out_zero, sigma, C, seed, offset, denom, what="", xi=None):
    """out(sigma) - out(0) = sigma C xi / denom, element by element."""
    d = np.asarray(out_sigma, np.float64) - np.asarray(out_zero, np.float64)
    if xi is None:
        from oracle import philox
        xi = philox.gaussian(seed, offset, d.size).reshape(d.shape)
    want = sigma * C * np.asarray(xi, np.float64) / denom
    err = float(np.max(np.abs(d - want)))
    tol = NOISE_ELEM_TOL * sigma * C / denom
    assert np.isfinite(err) and err <= tol, (
        f"{what}: max|noise - sigma C xi / denom| = {err:.3e} > {tol:.3e}")
    return err
