"""GPU Philox4x32-10 and Gaussian fill against the oracle's generator.

Tolerances: Philox words bit-exact; float32 normals within 1e-5 absolute
(fp32 log/sqrt/sincospi against fp64, |z| <= 5.8); bfloat16 output within one
bf16 rounding of the oracle's value."""
import numpy as np
import pytest

from oracle import philox
from tests.gpu_helpers import need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,offset,n", [
    (0, 0, 4096), (7, 0, 1000), (12345, 2**32 - 100, 300), (2**64 - 1, 2**63 + 11, 257),
    (0xDEADBEEF, 5, 1),
])
def test_philox_words_bit_exact(seed, offset, n):
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    w = dp.philox4x32_10(seed, offset, n).cpu().numpy().view(np.uint32)
    blocks = (np.uint64(offset) + np.arange(n, dtype=np.uint64))
    np.testing.assert_array_equal(w, philox.philox_words(seed, blocks))


@pytest.mark.parametrize("seed,offset,n,scale", [
    (0, 0, 100003, 1.0), (7, 0, 4096 * 256, 1.0 / 16), (3, 2**32 - 2, 37, 2.5), (1, 9, 1, 1.0),
])
def test_gaussian_fill_f32(seed, offset, n, scale):
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    z = dp.gaussian_fill(seed, offset, n, scale).cpu().numpy().astype(np.float64)
    ref = scale * philox.gaussian(seed, offset, n)
    assert np.max(np.abs(z - ref)) <= 1e-5 * max(1.0, scale)


def test_gaussian_fill_bf16():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    n, scale = 1024 * 256, 1.0 / 16
    from workloads import f32_to_bf16_bits
    bits = dp.gaussian_fill(7, 0, n, scale, dtype=torch.bfloat16).cpu().view(torch.int16).numpy()
    ref = scale * philox.gaussian(7, 0, n)
    ref_bits = f32_to_bf16_bits(ref.astype(np.float32)).view(np.int16)
    # identical bf16 except where the fp32 and fp64 normals straddle a rounding
    # midpoint (probability ~2^-15 per element); there, one ulp apart
    diff = np.abs(bits.astype(np.int32) - ref_bits.astype(np.int32))
    assert diff.max() <= 1
    assert np.mean(diff == 0) > 0.999


def test_gaussian_fill_offset_concatenation():
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    n = 4 * 1000
    a = dp.gaussian_fill(5, 100, 2 * n).cpu()
    b = dp.gaussian_fill(5, 100, n).cpu()
    c = dp.gaussian_fill(5, 100 + dp.noise_blocks(n), n).cpu()
    assert torch.equal(a, torch.cat([b, c]))
