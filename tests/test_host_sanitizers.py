"""The host side of libisd under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every HIP source is compiled with the sanitizers on its host code only (the device code is
built as usual and never runs here) and linked with tests/host/abi_host_check.cpp, a driver
that exercises the C ABI's host paths: size queries, configuration validation, the binding
checks that build and free a context's host metadata, and the argument checks of every entry
point.  None of them reaches a HIP runtime call or a kernel launch.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "strided_decoding_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.slow
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_abi_host_paths_under_asan_and_ubsan():
    tmp = tempfile.mkdtemp(prefix="isd_san_")
    try:
        srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
        base = ["-O1", "-g", "-std=c++17", "-fPIC", "-Wno-unused-result", "-Wno-unused-value", "-I",
                os.path.join(ROOT, "include")]

        def compile_one(f):
            obj = os.path.join(tmp, f[:-4] + ".o")
            r = subprocess.run([HIPCC, "--offload-arch=gfx950"] + base + HOST_SAN +
                               ["-c", os.path.join(CSRC, f), "-o", obj], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return obj

        with cf.ThreadPoolExecutor(max_workers=min(6, len(srcs))) as ex:
            objs = list(ex.map(compile_one, srcs))
        drv = os.path.join(tmp, "abi_host_check.o")
        r = subprocess.run([HIPCC] + base + HOST_SAN + ["-x", "c++", "-c",
                                                        os.path.join(ROOT, "tests", "host", "abi_host_check.cpp"),
                                                        "-o", drv], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        exe = os.path.join(tmp, "abi_host_check")
        # link: the clang driver with the HIP runtime and the sanitizer runtimes (host code only)
        r = subprocess.run([CLANG, "--hip-link", "--offload-arch=gfx950", "-fsanitize=address,undefined", "-o", exe,
                            drv] + objs, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        assert "abi host checks passed" in r.stdout
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
