"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer: the library's host code is rebuilt with both
sanitizers (device code unchanged, gfx950) and linked with tests/c/abi_validation.c,
which calls every entry point with invalid arguments (and the host-only
queries with valid ones) and checks each status and error text.  Nothing
reaches the GPU, so this runs without one.  CPU only; takes ~20 s."""
import concurrent.futures as cf
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int2_rotated_kv_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_validation_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-std=c++17", "-O1", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(f):
        obj = os.path.join(OUT, f + ".o")
        r = subprocess.run([HIPCC] + flags + ["-c", os.path.join(CSRC, f), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    # the driver is host code only; it and the link use the same compiler (and
    # so the same sanitizer runtime) as the library objects
    drv = os.path.join(OUT, "abi_validation.o")
    host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
    r = subprocess.run([HIPCC, "-x", "c++", "-std=c++17", "-O1", "-g", "-fPIC", "-I", os.path.join(ROOT, "include")]
                       + host + ["-c", os.path.join(ROOT, "tests", "c", "abi_validation.c"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = os.path.join(OUT, "abi_validation")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950"] + host + ["-o", exe, drv] + objs,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "all checks passed" in r.stdout
