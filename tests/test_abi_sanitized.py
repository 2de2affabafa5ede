"""Host-side argument validation of the C ABI under the host sanitizers.

Builds the library's host code with AddressSanitizer and UndefinedBehavior-
Sanitizer (the device code is built as usual; sanitizers never apply to it),
links tests/host/abi_checks.c against it, and runs that driver: every entry
point is called with bad arguments and must return the documented status
before anything is queued, with no sanitizer report.  CPU only; about half a
minute of compiling."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from sample_gradient_clipping_amd import build as b

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang"
# host-only sanitizer flags: each -fsanitize= right after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tools():
    try:
        return b._hipcc() and os.path.exists(CLANG)
    except RuntimeError:
        return False


@pytest.mark.skipif(not _tools(), reason="needs hipcc and the ROCm clang")
def test_abi_argument_checks_under_host_sanitizers(tmp_path):
    out = str(tmp_path)
    srcs = [s for s in sorted(os.listdir(b.CSRC)) if s.endswith(".hip")]

    def compile_one(src):
        obj = os.path.join(out, src + ".o")
        subprocess.run([b._hipcc(), *b.HIP_FLAGS, *HOST_SAN, "-g", "-I", b.INCLUDE, "-I", b.CSRC,
                        "-c", os.path.join(b.CSRC, src), "-o", obj],
                       check=True, capture_output=True)
        return obj

    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = os.path.join(out, "libdpfused_san.so")
    subprocess.run([b._hipcc(), "-shared", "-fPIC", f"--offload-arch={b.ARCH}", *HOST_SAN,
                    "-o", lib, *objs], check=True, capture_output=True)
    exe = os.path.join(out, "abi_checks")
    subprocess.run([CLANG, "-std=c11", "-g", "-fsanitize=address,undefined",
                    "-fno-omit-frame-pointer", "-I", b.INCLUDE,
                    os.path.join(HERE, "host", "abi_checks.c"), "-o", exe, f"-L{out}",
                    "-ldpfused_san", f"-Wl,-rpath,{out}", "-lm"], check=True, capture_output=True)
    # the HIP runtime's own allocations at exit are not this library's leaks
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    shutil.rmtree(out, ignore_errors=True)
