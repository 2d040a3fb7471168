"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host code only (device
code is built as usual), and tests/abi_sanitize.c drives every entry point's
argument checks and workspace sizing on the CPU: out-of-bounds accesses,
use-after-free, signed overflow, misaligned or null dereferences in that code
stop the run.  Calls whose arguments pass every check stop at the device
query when no GPU is present."""
import glob
import os
import shutil
import subprocess

import pytest

from global_muse_rope_amd import build_lib as bl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
LLVM = "/opt/rocm/lib/llvm/bin/clang"
# sanitizer options for the host pass only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime_dir():
    dirs = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux"))
    return dirs[-1] if dirs else ""


def _build():
    os.makedirs(OUT, exist_ok=True)
    rt = "-Wl,-rpath," + _runtime_dir()
    lib = os.path.join(OUT, "libmuse_attn_san.so")
    srcs = [os.path.join(bl.SRC, s) for s in bl.SOURCES]
    deps = srcs + glob.glob(os.path.join(bl.SRC, "*.h")) + glob.glob(os.path.join(bl.INCLUDE, "*.h"))
    newest = max(os.path.getmtime(p) for p in deps)
    if not os.path.exists(lib) or os.path.getmtime(lib) < newest:
        objs = []
        for s in bl.SOURCES:
            obj = os.path.join(OUT, os.path.splitext(s)[0] + ".o")
            cmd = [bl.hipcc(), *bl.HIPCC_FLAGS, *bl.SOURCE_FLAGS.get(s, []), *SAN, "-O1", "-g", "-c",
                   os.path.join(bl.SRC, s), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            objs.append(obj)
        cmd = [bl.hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-fsanitize=address,undefined",
               "-shared-libsan", rt, *objs, "-o", lib, "-lhipblaslt"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
    exe = os.path.join(OUT, "abi_sanitize")
    drv = os.path.join(ROOT, "tests", "abi_sanitize.c")
    if not os.path.exists(exe) or os.path.getmtime(exe) < max(os.path.getmtime(lib), os.path.getmtime(drv)):
        cmd = [LLVM, "-O1", "-g", "-fsanitize=address,undefined", "-shared-libsan", "-fno-sanitize-recover=undefined",
               "-I" + bl.INCLUDE, drv, lib, "-Wl,-rpath," + OUT, rt, "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
    return exe


@pytest.mark.timeout(600)
def test_c_abi_host_code_under_sanitizers():
    if not (shutil.which(bl.hipcc()) or os.path.exists(bl.hipcc())) or not os.path.exists(LLVM):
        pytest.skip("the HIP toolchain is not installed")
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "OK" in r.stdout, out[-4000:]
