"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer: every
source is compiled with the host half instrumented (device code unchanged), linked into a
separate library in a temporary folder, and the C ABI checks of test_abi.py run against
it in a child Python with the sanitizer runtime preloaded.  Any report aborts the child.
No GPU: the ABI checks make only calls that fail validation or query sizes."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduction_rmsnorm_fwd_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]

CHILD = r'''
import ctypes, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import reduction_rmsnorm_fwd_amd as fo
lib = ctypes.CDLL({lib!r})
for name, (res, args) in fo.SIGNATURES.items():
    f = getattr(lib, name); f.restype = res; f.argtypes = args
fo._lib = lib
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {abi!r}]))
'''


def _runtime():
    rts = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return rts[-1] if rts else None


@pytest.mark.slow
def test_abi_checks_under_asan_and_ubsan(tmp_path):
    rt = _runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or the sanitizer runtime is not installed")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs = []
    for src in srcs:
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-I" + os.path.join(ROOT, "include"),
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, "-c", src, "-o", obj]
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE)))
    objs = []
    for src, obj, p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, f"{src}: {err.decode()[-2000:]}"
        objs.append(obj)
    lib = str(tmp_path / "libfo_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN[:4], "-shared-libsan",
                        "-o", lib, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    # the host code really is instrumented
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    child = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                         abi=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout
