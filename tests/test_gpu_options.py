"""GPU checks of the library options that change how a call runs but not what
it computes: the workspace limit (allocation failure leaves every output as it
was and the next call works), and the trace and debug modes (roctx ranges,
synchronise after every launch), whose results must be bit-identical to a
plain call on every norm path."""
import numpy as np
import pytest

from sample_gradient_clipping_amd._lib import DPF_ERR_OUT_OF_MEMORY
from tests.gpu_helpers import need_gpu, random_linear, to_dev

pytestmark = pytest.mark.gpu

SHAPE = (4, 256, 768, 768)   # B, T, din, dout: staged tiles of 9.4 MB, a few KB of partials


def _inputs(torch, seed=5, shape=SHAPE):
    B, T, din, dout = shape
    lin = random_linear(np.random.default_rng(seed), B, T, din, dout, dtype="bf16")
    return to_dev(lin.X, "bf16", torch), to_dev(lin.G, "bf16", torch)


class _Options:
    """Sets library options for one block and restores the old values."""

    def __init__(self, **kw):
        self.kw = kw

    def __enter__(self):
        import sample_gradient_clipping_amd as dp
        self.old = {k: dp.get_option(k) for k in self.kw}
        for k, v in self.kw.items():
            dp.set_option(k, v)

    def __exit__(self, *exc):
        import sample_gradient_clipping_amd as dp
        for k, v in self.old.items():
            dp.set_option(k, v)


@pytest.mark.parametrize("path", [0, 1, 2, 3])
@pytest.mark.parametrize("limit", [1, 4 << 20])
def test_workspace_limit_fails_without_writing(path, limit):
    """limit 1: the first workspace request fails; 4 MiB: the partials fit and,
    on the staged path, the tile buffer does not."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    X, G = _inputs(torch)
    B, dout, din = X.shape[0], G.shape[2], X.shape[2]
    with _Options(norm_path=path):
        ref, ref_n = dp.linear_clip_accumulate(X, G, C=0.5, sigma=0.3, seed=3, offset=1)
        out = torch.full((dout, din), 7.0, device="cuda")
        norms = torch.full((B,), -2.0, device="cuda")
        with _Options(workspace_limit_bytes=limit):
            try:
                dp.linear_clip_accumulate(X, G, C=0.5, sigma=0.3, seed=3, offset=1,
                                          grad_out=out, norms_out=norms)
                failed = None
            except dp.DpfError as e:
                failed = e
        torch.cuda.synchronize()
        if failed is None:
            # only the 4 MiB limit on a path without staged tiles may pass
            assert limit > 1 and path != 3
        else:
            assert failed.status == DPF_ERR_OUT_OF_MEMORY
            assert torch.all(out == 7.0) and torch.all(norms == -2.0)
        dp.linear_clip_accumulate(X, G, C=0.5, sigma=0.3, seed=3, offset=1,
                                  grad_out=out, norms_out=norms)
        torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(norms, ref_n)


def test_workspace_limit_group_and_bias():
    """Staged path forced, so the 4 MiB limit fails at the tile buffer."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    with _Options(norm_path=3):
        _group_and_bias(torch, dp)


@pytest.mark.parametrize("path", [0, 1, 2])
def test_workspace_limit_just_below_the_call_leaves_outputs(path):
    """Masked group and bias calls on the two-pass paths: a limit one byte
    below what the call takes fails before anything is written (the call
    takes all its workspace before its first launch), and a limit equal to
    it lets the call run."""
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    X, G = _inputs(torch)
    X2, G2 = _inputs(torch, seed=6, shape=(4, 256, 768, 256))
    mask = torch.ones(X.shape[:2], dtype=torch.uint8, device="cuda")
    mask[1, 100:] = 0
    mask[3, :] = 0
    offs = dp.consecutive_offsets([(768, 768), (256, 768)])
    calls = {
        "group": lambda outs: dp.group_clip_accumulate(
            [X, X2], [G, G2], mask, C=0.5, sigma=0.3, seed=3, offsets=offs,
            grad_outs=outs[:2], norms_out=outs[2]),
        "bias": lambda outs: dp.linear_clip_accumulate_bias(
            X, G, mask, C=0.5, sigma=0.3, seed=3, grad_out=outs[0], bias_grad_out=outs[1],
            norms_out=outs[2]),
    }
    with _Options(norm_path=path):
        for name, call in calls.items():
            shapes = [(768, 768), (256, 768), (4,)] if name == "group" else \
                [(768, 768), (768,), (4,)]
            ref = [torch.empty(sh, device="cuda") for sh in shapes]
            call(ref)
            torch.cuda.synchronize()
            need = dp.get_option("workspace_call_bytes")
            assert need > 0
            outs = [torch.full(sh, 7.0, device="cuda") for sh in shapes]
            with _Options(workspace_limit_bytes=need - 1):
                with pytest.raises(dp.DpfError) as e:
                    call(outs)
                assert e.value.status == DPF_ERR_OUT_OF_MEMORY
            torch.cuda.synchronize()
            assert all(torch.all(o == 7.0) for o in outs), name
            with _Options(workspace_limit_bytes=need):
                call(outs)
            torch.cuda.synchronize()
            assert all(torch.equal(a, b) for a, b in zip(outs, ref)), name


def _group_and_bias(torch, dp):
    X, G = _inputs(torch)
    X2, G2 = _inputs(torch, seed=6, shape=(4, 256, 768, 256))
    ref = dp.group_clip_accumulate([X, X2], [G, G2], C=0.5, sigma=0.3, seed=3,
                                   offsets=[0, dp.noise_blocks(768 * 768)])
    refb = dp.linear_clip_accumulate_bias(X, G, C=0.5, sigma=0.3, seed=3)
    outs = [torch.full_like(ref[0][0], 7.0), torch.full_like(ref[0][1], 7.0)]
    ob = (torch.full_like(refb[0], 7.0), torch.full_like(refb[1], 7.0))
    for limit in (1, 4 << 20):
        with _Options(workspace_limit_bytes=limit):
            with pytest.raises(dp.DpfError) as e:
                dp.group_clip_accumulate([X, X2], [G, G2], C=0.5, sigma=0.3, seed=3,
                                         offsets=[0, dp.noise_blocks(768 * 768)], grad_outs=outs)
            assert e.value.status == DPF_ERR_OUT_OF_MEMORY
            with pytest.raises(dp.DpfError) as e:
                dp.linear_clip_accumulate_bias(X, G, C=0.5, sigma=0.3, seed=3, grad_out=ob[0],
                                               bias_grad_out=ob[1])
            assert e.value.status == DPF_ERR_OUT_OF_MEMORY
        torch.cuda.synchronize()
        assert all(torch.all(o == 7.0) for o in outs + list(ob))
    got = dp.group_clip_accumulate([X, X2], [G, G2], C=0.5, sigma=0.3, seed=3,
                                   offsets=[0, dp.noise_blocks(768 * 768)], grad_outs=outs)
    gotb = dp.linear_clip_accumulate_bias(X, G, C=0.5, sigma=0.3, seed=3, grad_out=ob[0],
                                          bias_grad_out=ob[1])
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(got[0], ref[0])) and torch.equal(got[1], ref[1])
    assert all(torch.equal(a, b) for a, b in zip(gotb, refb))


@pytest.mark.parametrize("path", [0, 1, 2, 3])
def test_trace_and_debug_modes_change_nothing(path, capfd):
    torch = need_gpu()
    import sample_gradient_clipping_amd as dp
    X, G = _inputs(torch)
    mask = torch.ones(X.shape[:2], dtype=torch.uint8, device="cuda")
    mask[1, 100:] = 0
    with _Options(norm_path=path):
        ref = dp.linear_clip_accumulate(X, G, mask, C=0.5, sigma=0.3, seed=3)
        refb = dp.linear_clip_accumulate_bias(X, G, None, C=0.5, sigma=0.3, seed=3)
        with _Options(trace=1, debug=1):
            got = dp.linear_clip_accumulate(X, G, mask, C=0.5, sigma=0.3, seed=3)
            gotb = dp.linear_clip_accumulate_bias(X, G, None, C=0.5, sigma=0.3, seed=3)
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    assert all(torch.equal(a, b) for a, b in zip(gotb, refb))
    assert "dpfused: kernel" not in capfd.readouterr().err
