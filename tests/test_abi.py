"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call is made."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from sample_gradient_clipping_amd import _lib
from sample_gradient_clipping_amd._lib import (DPF_BF16, DPF_ERR_INVALID_ARGUMENT,
                                               DPF_ERR_UNSUPPORTED, DPF_F32, DPF_OK, DpfAct)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dpfused.h")

FAKE = 0x10000   # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libdpfused.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dpfused_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("dpfused_linear_clip_accumulate", "dpfused_linear_clip_accumulate_projected",
                     "dpfused_philox4x32_10", "dpfused_gaussian_fill", "dpfused_noise_blocks",
                     "dpfused_status_string", "dpfused_last_error", "dpfused_abi_version"):
        assert required in names


def test_every_declared_symbol_is_exported(L):
    raw = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(raw, n)]
    assert not missing, missing
    assert set(declared_functions()) == set(_lib._SIGNATURES), "binding and header disagree"


def test_abi_version_and_strings(L):
    assert L.dpfused_abi_version() == 1
    assert L.dpfused_status_string(DPF_OK) == b"DPF_OK"
    assert L.dpfused_status_string(DPF_ERR_INVALID_ARGUMENT) == b"DPF_ERR_INVALID_ARGUMENT"
    assert L.dpfused_status_string(99) == b"DPF_UNKNOWN_STATUS"


def test_noise_blocks(L):
    for n, want in [(0, 0), (-5, 0), (1, 1), (4, 1), (5, 2), (70778880, 17694720)]:
        assert L.dpfused_noise_blocks(n) == want


def test_options(L):
    assert L.dpfused_set_option(b"norm_path", 2) == DPF_OK
    assert L.dpfused_get_option(b"norm_path") == 2
    assert L.dpfused_set_option(b"norm_path", 0) == DPF_OK
    assert L.dpfused_set_option(b"norm_path", 3) == DPF_OK
    assert L.dpfused_get_option(b"norm_path") == 3
    assert L.dpfused_set_option(b"norm_path", 0) == DPF_OK
    assert L.dpfused_set_option(b"norm_path", 4) == DPF_OK
    assert L.dpfused_get_option(b"norm_path") == 4
    assert L.dpfused_set_option(b"norm_path", 0) == DPF_OK
    assert L.dpfused_set_option(b"norm_path", 5) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_set_option(b"onepass_spin_limit", -1) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_set_option(b"onepass_never_ready", 2) == DPF_ERR_INVALID_ARGUMENT
    spin = L.dpfused_get_option(b"onepass_spin_limit")
    assert spin == 1 << 20 and L.dpfused_get_option(b"onepass_never_ready") == 0
    assert L.dpfused_set_option(b"onepass_spin_limit", 7) == DPF_OK
    assert L.dpfused_get_option(b"onepass_spin_limit") == 7
    assert L.dpfused_set_option(b"onepass_spin_limit", spin) == DPF_OK
    assert L.dpfused_set_option(b"norm_path", -1) == DPF_ERR_INVALID_ARGUMENT
    keep = L.dpfused_get_option(b"workspace_keep_bytes")
    assert keep == 512 << 20
    assert L.dpfused_set_option(b"workspace_keep_bytes", -1) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_set_option(b"workspace_keep_bytes", 1 << 20) == DPF_OK
    assert L.dpfused_get_option(b"workspace_keep_bytes") == 1 << 20
    assert L.dpfused_set_option(b"workspace_keep_bytes", keep) == DPF_OK
    assert L.dpfused_set_option(b"bogus", 1) == DPF_ERR_INVALID_ARGUMENT
    assert b"bogus" in L.dpfused_last_error()
    assert L.dpfused_get_option(b"bogus") == -1
    assert L.dpfused_set_option(b"timing", 0) == DPF_OK
    for name in (b"trace", b"debug", b"p_in_kernels"):
        assert L.dpfused_set_option(name, 1) == DPF_OK
        assert L.dpfused_get_option(name) == 1
        assert L.dpfused_set_option(name, 0) == DPF_OK
        assert L.dpfused_get_option(name) == 0
        assert L.dpfused_set_option(name, 2) == DPF_ERR_INVALID_ARGUMENT
    side = L.dpfused_get_option(b"side_streams")
    assert side == 1
    for v in (0, 4):
        assert L.dpfused_set_option(b"side_streams", v) == DPF_OK
        assert L.dpfused_get_option(b"side_streams") == v
    assert L.dpfused_set_option(b"side_streams", 5) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_set_option(b"side_streams", -1) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_set_option(b"side_streams", side) == DPF_OK
    tiles = L.dpfused_get_option(b"rspace_tiles")
    assert tiles == 1
    for v in (0, 2):
        assert L.dpfused_set_option(b"rspace_tiles", v) == DPF_OK
        assert L.dpfused_get_option(b"rspace_tiles") == v
    assert L.dpfused_set_option(b"rspace_tiles", 3) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_set_option(b"rspace_tiles", -1) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_set_option(b"rspace_tiles", tiles) == DPF_OK
    assert L.dpfused_get_option(b"workspace_limit_bytes") == 0
    assert L.dpfused_set_option(b"workspace_limit_bytes", -1) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_set_option(b"workspace_limit_bytes", 4096) == DPF_OK
    assert L.dpfused_get_option(b"workspace_limit_bytes") == 4096
    assert L.dpfused_set_option(b"workspace_limit_bytes", 0) == DPF_OK


@pytest.mark.parametrize("env,want", [
    ({"DPFUSED_NORM_PATH": "staged"}, {"norm_path": 3}),
    ({"DPFUSED_NORM_PATH": "gram", "DPFUSED_TRACE": "1"}, {"norm_path": 1, "trace": 1}),
    ({"DPFUSED_NORM_PATH": "2", "DPFUSED_DEBUG": "1"}, {"norm_path": 2, "debug": 1}),
    ({"DPFUSED_NORM_PATH": "bogus", "DPFUSED_WS_LIMIT": "123456"},
     {"norm_path": 0, "workspace_limit_bytes": 123456, "trace": 0, "debug": 0}),
])
def test_options_from_environment(env, want):
    # read once when the library is loaded, so each case loads it in a fresh process
    import subprocess
    import sys
    code = ("import ctypes, sys; L = ctypes.CDLL(sys.argv[1]); "
            "L.dpfused_get_option.restype = ctypes.c_int64; "
            "print(' '.join(str(L.dpfused_get_option(n.encode())) for n in sys.argv[2:]))")
    names = list(want)
    out = subprocess.run([sys.executable, "-c", code, _lib.LIB_PATH, *names],
                         env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert [int(v) for v in out.stdout.split()] == [want[n] for n in names]


def _act(B=2, T=3, D=8, dtype=DPF_BF16, data=FAKE, reserved=0, sb=None, st=None):
    st = D if st is None else st
    sb = T * st if sb is None else sb
    return DpfAct(data, dtype, reserved, B, T, D, sb, st)


def _call(L, X, G, C=1.0, sigma=0.5, out=FAKE, mask=None):
    return L.dpfused_linear_clip_accumulate(ctypes.byref(X) if X is not None else None,
                                            ctypes.byref(G) if G is not None else None,
                                            mask, C, sigma, 0, 0, out, None, None)


@pytest.mark.parametrize("case,status", [
    (dict(X=None), DPF_ERR_INVALID_ARGUMENT),
    (dict(xdata=0), DPF_ERR_INVALID_ARGUMENT),
    (dict(out=0), DPF_ERR_INVALID_ARGUMENT),
    (dict(xB=0), DPF_ERR_INVALID_ARGUMENT),
    (dict(xT=0), DPF_ERR_INVALID_ARGUMENT),
    (dict(xD=0), DPF_ERR_INVALID_ARGUMENT),
    (dict(gB=3), DPF_ERR_INVALID_ARGUMENT),
    (dict(gT=4), DPF_ERR_INVALID_ARGUMENT),
    (dict(C=0.0), DPF_ERR_INVALID_ARGUMENT),
    (dict(C=-1.0), DPF_ERR_INVALID_ARGUMENT),
    (dict(C=math.nan), DPF_ERR_INVALID_ARGUMENT),
    (dict(C=math.inf), DPF_ERR_INVALID_ARGUMENT),
    (dict(sigma=-0.1), DPF_ERR_INVALID_ARGUMENT),
    (dict(sigma=math.nan), DPF_ERR_INVALID_ARGUMENT),
    (dict(sigma=3e38, C=10.0), DPF_ERR_INVALID_ARGUMENT),
    (dict(xst=4), DPF_ERR_INVALID_ARGUMENT),
    (dict(xsb=10), DPF_ERR_INVALID_ARGUMENT),
    (dict(gdtype=DPF_F32), DPF_ERR_UNSUPPORTED),
    (dict(xdtype=7, gdtype=7), DPF_ERR_UNSUPPORTED),
    (dict(xreserved=1), DPF_ERR_UNSUPPORTED),
    (dict(xdata=FAKE + 2), DPF_ERR_UNSUPPORTED),
    (dict(out=FAKE + 4), DPF_ERR_UNSUPPORTED),
])
def test_dense_argument_checks(L, case, status):
    X = _act(B=case.get("xB", 2), T=case.get("xT", 3), D=case.get("xD", 8),
             dtype=case.get("xdtype", DPF_BF16), data=case.get("xdata", FAKE),
             reserved=case.get("xreserved", 0), sb=case.get("xsb"), st=case.get("xst"))
    G = _act(B=case.get("gB", 2), T=case.get("gT", 3), D=16, dtype=case.get("gdtype", case.get("xdtype", DPF_BF16)))
    got = _call(L, None if case.get("X", 1) is None else X, G, C=case.get("C", 1.0),
                sigma=case.get("sigma", 0.5), out=case.get("out", FAKE))
    assert got == status, L.dpfused_last_error()
    assert L.dpfused_last_error() != b""


def test_projected_argument_checks(L):
    X, G = _act(), _act(D=16)
    f = L.dpfused_linear_clip_accumulate_projected
    assert f(ctypes.byref(X), ctypes.byref(G), None, None, 4, 1.0, 1.0, 0, 0, FAKE, None, None) \
        == DPF_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(X), ctypes.byref(G), None, FAKE, 0, 1.0, 1.0, 0, 0, FAKE, None, None) \
        == DPF_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(X), ctypes.byref(G), None, FAKE + 8, 4, 1.0, 1.0, 0, 0, FAKE, None, None) \
        == DPF_ERR_UNSUPPORTED
    assert f(ctypes.byref(X), ctypes.byref(G), None, FAKE, 4, 0.0, 1.0, 0, 0, FAKE, None, None) \
        == DPF_ERR_INVALID_ARGUMENT


def test_project_argument_checks(L):
    X = _act()
    f = L.dpfused_project
    ok_args = dict(P=FAKE, r=4, Y=FAKE)

    def call(**kw):
        a = {**ok_args, **kw}
        return f(ctypes.byref(X), None, a["P"], a["r"], a["Y"], None)

    assert call(P=None) == DPF_ERR_INVALID_ARGUMENT
    assert call(Y=None) == DPF_ERR_INVALID_ARGUMENT
    assert call(r=0) == DPF_ERR_INVALID_ARGUMENT
    assert call(r=-3) == DPF_ERR_INVALID_ARGUMENT
    assert call(P=FAKE + 8) == DPF_ERR_UNSUPPORTED
    assert call(Y=FAKE + 8) == DPF_ERR_UNSUPPORTED
    assert call(r=1 << 40) == DPF_ERR_UNSUPPORTED
    bad = _act(B=0)
    assert f(ctypes.byref(bad), None, FAKE, 4, FAKE, None) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_last_error() != b""


def test_ex_argument_checks(L):
    X, G = _act(), _act(D=16)
    f = L.dpfused_linear_clip_accumulate_ex
    args = lambda denom=2.0, acc=0, C=1.0, out=FAKE: (ctypes.byref(X), ctypes.byref(G), None, C, 0.5,
                                                      0, 0, denom, acc, out, None, None)
    assert f(*args(denom=0.0)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(denom=-1.0)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(denom=math.nan)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(denom=math.inf)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(acc=2)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(acc=-1)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(C=0.0)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(out=0)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(out=FAKE + 4)) == DPF_ERR_UNSUPPORTED
    assert b"" != L.dpfused_last_error()


def test_seeded_projected_argument_checks(L):
    X, G = _act(), _act(D=16)
    f = L.dpfused_linear_clip_accumulate_projected_seeded
    args = lambda r=8, scale=0.25, C=1.0, out=FAKE: (ctypes.byref(X), ctypes.byref(G), None, r, 7, 0,
                                                      scale, C, 1.0, 0, 0, out, None, None)
    assert f(*args(r=0)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(r=12)) == DPF_ERR_UNSUPPORTED             # not a multiple of 8
    assert f(*args(scale=math.inf)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(scale=-math.inf)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(C=0.0)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(out=0)) == DPF_ERR_INVALID_ARGUMENT
    assert f(*args(out=FAKE + 4)) == DPF_ERR_UNSUPPORTED


def test_bias_argument_checks(L):
    X, G = _act(), _act(D=16)
    f = L.dpfused_linear_clip_accumulate_bias
    call = lambda out=FAKE, bout=FAKE, C=1.0: f(ctypes.byref(X), ctypes.byref(G), None, C, 1.0, 0,
                                                 0, out, bout, None, None)
    assert call(bout=None) == DPF_ERR_INVALID_ARGUMENT
    assert call(out=None) == DPF_ERR_INVALID_ARGUMENT
    assert call(bout=FAKE + 2) == DPF_ERR_UNSUPPORTED
    assert call(out=FAKE + 4) == DPF_ERR_UNSUPPORTED
    assert call(C=-1.0) == DPF_ERR_INVALID_ARGUMENT


def test_group_argument_checks(L):
    n = 2
    Xs = (DpfAct * n)(_act(), _act(D=16))
    Gs = (DpfAct * n)(_act(D=16), _act(D=8))
    offs = (ctypes.c_uint64 * n)(0, 32)
    outs = (ctypes.c_void_p * n)(FAKE, FAKE)
    f = L.dpfused_group_clip_accumulate
    assert f(0, Xs, Gs, None, 1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert f(n, None, Gs, None, 1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert f(n, Xs, Gs, None, 1.0, 1.0, 0, None, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert f(n, Xs, Gs, None, -1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    bad_t = (DpfAct * n)(_act(), _act(T=5, D=16))
    bad_tg = (DpfAct * n)(_act(D=16), _act(T=5, D=8))
    assert f(n, bad_t, bad_tg, None, 1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert b"same B and T" in L.dpfused_last_error()
    bad_out = (ctypes.c_void_p * n)(FAKE, FAKE + 4)
    assert f(n, Xs, Gs, None, 1.0, 1.0, 0, offs, bad_out, None, None) == DPF_ERR_UNSUPPORTED
    null_out = (ctypes.c_void_p * n)(FAKE, None)
    assert f(n, Xs, Gs, None, 1.0, 1.0, 0, offs, null_out, None, None) == DPF_ERR_INVALID_ARGUMENT


def test_projected_adam_argument_checks(L):
    f = L.dpfused_projected_adam_step
    ok = dict(grad=FAKE, m=FAKE, v=FAKE, W=FAKE, dout=4, din=8, r=8, step=1, lr=1e-3, b1=0.9,
              b2=0.999, eps=1e-8, P=FAKE, pdt=DPF_BF16, scale=0.25)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["grad"], a["m"], a["v"], a["W"], a["dout"], a["din"], a["r"], a["step"],
                 a["lr"], a["b1"], a["b2"], a["eps"], a["P"], a["pdt"], 0, 0, a["scale"], None)
    assert call(grad=None) == DPF_ERR_INVALID_ARGUMENT
    assert call(W=None) == DPF_ERR_INVALID_ARGUMENT
    assert call(r=0) == DPF_ERR_INVALID_ARGUMENT
    assert call(r=6) == DPF_ERR_UNSUPPORTED
    assert call(din=10) == DPF_ERR_UNSUPPORTED
    assert call(step=0) == DPF_ERR_INVALID_ARGUMENT
    assert call(b1=1.0) == DPF_ERR_INVALID_ARGUMENT
    assert call(b2=-0.1) == DPF_ERR_INVALID_ARGUMENT
    assert call(eps=0.0) == DPF_ERR_INVALID_ARGUMENT
    assert call(lr=math.inf) == DPF_ERR_INVALID_ARGUMENT
    assert call(pdt=9) == DPF_ERR_UNSUPPORTED
    assert call(P=None, scale=math.inf) == DPF_ERR_INVALID_ARGUMENT
    assert call(m=FAKE + 4) == DPF_ERR_UNSUPPORTED


def test_building_block_argument_checks(L):
    X, G = _act(), _act(D=16)
    assert L.dpfused_per_sample_sqnorms(ctypes.byref(X), ctypes.byref(G), None, None, 0, None) \
        == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_clip_factors(None, 4, 1.0, FAKE, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_clip_factors(FAKE, 0, 1.0, FAKE, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_clip_factors(FAKE, 4, -1.0, FAKE, None, None) == DPF_ERR_INVALID_ARGUMENT
    sa = L.dpfused_scaled_accumulate
    assert sa(ctypes.byref(X), ctypes.byref(G), None, None, 0.0, 0, 0, FAKE, None) == DPF_ERR_INVALID_ARGUMENT
    assert sa(ctypes.byref(X), ctypes.byref(G), None, FAKE, -1.0, 0, 0, FAKE, None) == DPF_ERR_INVALID_ARGUMENT


def test_rng_argument_checks(L):
    assert L.dpfused_philox4x32_10(0, 0, 0, None, None) == DPF_OK   # nothing to do
    assert L.dpfused_philox4x32_10(0, 0, -1, FAKE, None) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_philox4x32_10(0, 0, 5, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_philox4x32_10(0, 0, 5, FAKE + 4, None) == DPF_ERR_UNSUPPORTED
    assert L.dpfused_gaussian_fill(0, 0, 0, 1.0, DPF_F32, None, None) == DPF_OK
    assert L.dpfused_gaussian_fill(0, 0, -1, 1.0, DPF_F32, FAKE, None) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_gaussian_fill(0, 0, 8, 1.0, 9, FAKE, None) == DPF_ERR_UNSUPPORTED
    assert L.dpfused_gaussian_fill(0, 0, 8, math.inf, DPF_F32, FAKE, None) == DPF_ERR_INVALID_ARGUMENT


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.lib()


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "sample_gradient_clipping_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f


def test_seeded_projection_rejects_noise_drawn_from_its_blocks(L):
    """With sigma > 0 the noise must not reuse the projection's Philox blocks under the
    same seed: the noise would then be a scaled copy of P's entries."""
    X, G = _act(D=16), _act(D=8)                 # din = 16, dout = 8, r = 8
    f = L.dpfused_linear_clip_accumulate_projected_seeded

    def call(p_seed, p_off, seed, off, sigma=1.0):
        return f(ctypes.byref(X), ctypes.byref(G), None, 8, p_seed, p_off, math.nan, 1.0, sigma,
                 seed, off, FAKE, None, None)
    # P uses blocks [p_off, p_off + 32); the noise [off, off + 16)
    assert call(7, 0, 7, 0) == DPF_ERR_INVALID_ARGUMENT
    assert b"overlap" in L.dpfused_last_error()
    assert call(7, 0, 7, 31) == DPF_ERR_INVALID_ARGUMENT
    assert call(7, 20, 7, 5) == DPF_ERR_INVALID_ARGUMENT
    assert call(0, 0, 0, 0) == DPF_ERR_INVALID_ARGUMENT      # the all-default seeds
    # the range wraps modulo 2^64
    assert call(7, 2 ** 64 - 4, 7, 10) == DPF_ERR_INVALID_ARGUMENT


def test_projected_many_argument_checks(L):
    n = 2
    Xs = (DpfAct * n)(_act(), _act(D=16))
    Gs = (DpfAct * n)(_act(D=16), _act(D=8))
    Ps = (ctypes.c_void_p * n)(FAKE, FAKE)
    offs = (ctypes.c_uint64 * n)(0, 64)
    outs = (ctypes.c_void_p * n)(FAKE, FAKE)
    f = L.dpfused_linear_clip_accumulate_projected_many
    assert f(0, Xs, Gs, None, Ps, 8, 1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert f(65, Xs, Gs, None, Ps, 8, 1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert f(n, None, Gs, None, Ps, 8, 1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert f(n, Xs, Gs, None, None, 8, 1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert f(n, Xs, Gs, None, Ps, 8, 1.0, 1.0, 0, None, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert f(n, Xs, Gs, None, Ps, 0, 1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    assert f(n, Xs, Gs, None, Ps, 8, -1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_INVALID_ARGUMENT
    bad_g = (DpfAct * n)(_act(D=16), _act(T=5, D=8))
    assert f(n, Xs, bad_g, None, Ps, 8, 1.0, 1.0, 0, offs, outs, None, None) == \
        DPF_ERR_INVALID_ARGUMENT
    null_p = (ctypes.c_void_p * n)(FAKE, None)
    assert f(n, Xs, Gs, None, null_p, 8, 1.0, 1.0, 0, offs, outs, None, None) == \
        DPF_ERR_INVALID_ARGUMENT
    odd_p = (ctypes.c_void_p * n)(FAKE, FAKE + 4)
    assert f(n, Xs, Gs, None, odd_p, 8, 1.0, 1.0, 0, offs, outs, None, None) == DPF_ERR_UNSUPPORTED
    bad_out = (ctypes.c_void_p * n)(FAKE, FAKE + 4)
    assert f(n, Xs, Gs, None, Ps, 8, 1.0, 1.0, 0, offs, bad_out, None, None) == DPF_ERR_UNSUPPORTED
    # noise ranges: dout * r = 16 * 8 and 8 * 8 elements: 32 and 16 blocks
    for bad in ([0, 0], [0, 31], [10, 0]):
        o = (ctypes.c_uint64 * n)(*bad)
        assert f(n, Xs, Gs, None, Ps, 8, 1.0, 0.5, 0, o, outs, None, None) == \
            DPF_ERR_INVALID_ARGUMENT, bad
        assert b"overlap" in L.dpfused_last_error()


def test_group_rejects_overlapping_noise_ranges(L):
    n = 3
    Xs = (DpfAct * n)(_act(D=16), _act(D=16), _act(D=8))
    Gs = (DpfAct * n)(_act(D=16), _act(D=8), _act(D=8))       # 64, 32 and 16 noise blocks
    outs = (ctypes.c_void_p * n)(FAKE, FAKE, FAKE)
    f = L.dpfused_group_clip_accumulate
    for bad in ([0, 0, 200], [0, 63, 200], [0, 64, 95], [100, 0, 20], [0, 2 ** 64 - 8, 500]):
        offs = (ctypes.c_uint64 * n)(*bad)
        assert f(n, Xs, Gs, None, 1.0, 0.5, 0, offs, outs, None, None) == \
            DPF_ERR_INVALID_ARGUMENT, bad
        assert b"overlap" in L.dpfused_last_error()


def test_binding_default_group_offsets_are_disjoint():
    import sample_gradient_clipping_amd as dp
    shapes = [(5120, 5120), (13824, 5120), (7, 3), (1, 1), (2, 2)]
    offs = dp.consecutive_offsets(shapes)
    assert offs[0] == 0
    for l in range(1, len(shapes)):
        assert offs[l] == offs[l - 1] + dp_noise_blocks(shapes[l - 1][0] * shapes[l - 1][1])
    assert dp.consecutive_offsets([(3, 3)], start=9) == [9]


def dp_noise_blocks(n):
    return (n + 3) // 4


def test_binding_checks_caller_outputs():
    """Outputs the caller passes are written through raw pointers: the binding checks
    dtype, exact shape, contiguity and device before any call."""
    torch = pytest.importorskip("torch")
    import sample_gradient_clipping_amd as dp
    chk = dp._check_out
    dev = torch.device("cpu")
    good = torch.empty((4, 6), dtype=torch.float32)
    chk(good, (4, 6), "grad_out", dev)
    with pytest.raises(ValueError, match="float32"):
        chk(good.to(torch.bfloat16), (4, 6), "grad_out", dev)
    with pytest.raises(ValueError, match="shape"):
        chk(good, (6, 4), "grad_out", dev)
    with pytest.raises(ValueError, match="shape"):
        chk(good.reshape(24), (4, 6), "grad_out", dev)
    with pytest.raises(ValueError, match="contiguous"):
        chk(torch.empty((6, 4)).t(), (4, 6), "grad_out", dev)
    with pytest.raises(ValueError, match="on"):
        chk(torch.empty((4, 6), device="meta"), (4, 6), "grad_out", dev)
    with pytest.raises(TypeError):
        chk(np.zeros((4, 6), np.float32), (4, 6), "grad_out", dev)
    with pytest.raises(ValueError, match="float64"):
        chk(torch.empty(4), (4,), "out", dev, torch.float64)
    with pytest.raises(ValueError, match="on"):
        dp._same_device(torch.empty(2, device="meta"), dev, "G")


def test_memory_options(L):
    assert L.dpfused_get_option(b"staged_keep_bytes") == 0
    assert L.dpfused_get_option(b"workspace_keep_bytes") == 512 << 20
    assert L.dpfused_set_option(b"staged_keep_bytes", -1) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_set_option(b"workspace_call_high", 5) == DPF_ERR_INVALID_ARGUMENT
    assert L.dpfused_set_option(b"workspace_call_high", 0) == DPF_OK
    assert L.dpfused_get_option(b"workspace_call_high") == 0
    assert L.dpfused_get_option(b"workspace_call_bytes") >= 0
    assert L.dpfused_set_option(b"staged_keep_bytes", 1 << 30) == DPF_OK
    assert L.dpfused_get_option(b"staged_keep_bytes") == 1 << 30
    assert L.dpfused_set_option(b"staged_keep_bytes", 0) == DPF_OK


def test_noalloc_argument_checks(L):
    X, G = _act(), _act(D=16)
    f = L.dpfused_linear_clip_accumulate_noalloc
    call = lambda out=FAKE, C=1.0, sigma=1.0: f(ctypes.byref(X), ctypes.byref(G), None, C, sigma,
                                                 0, 0, out, None, None)
    assert call(out=None) == DPF_ERR_INVALID_ARGUMENT
    assert call(out=FAKE + 4) == DPF_ERR_UNSUPPORTED
    assert call(C=0.0) == DPF_ERR_INVALID_ARGUMENT
    assert call(sigma=-1.0) == DPF_ERR_INVALID_ARGUMENT
    bad = _act(T=5)
    assert f(ctypes.byref(bad), ctypes.byref(G), None, 1.0, 1.0, 0, 0, FAKE, None, None) == \
        DPF_ERR_INVALID_ARGUMENT
