"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (all of the library's host code: validation, workspace layout, blob
and snapshot parsing, timing records) is compiled with g++ and
-fsanitize=address,undefined and linked, with the kernels' objects as built,
into tests/abi_sanitize.cpp's driver, which drives every refusal path and
parses corrupted and truncated blobs held in exactly-sized heap buffers.  The
driver makes no device call, so this runs without a GPU; a sanitizer report
or a failed check fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "compressed_kv_attention_compressor_amd")
CSRC = os.path.join(PKG, "csrc")
OBJS = [os.path.join(PKG, "_build", f"{n}.o") for n in ("proj_gemm", "pool", "decode", "indexer", "attention")]
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_host_code_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    if not all(os.path.exists(o) for o in OBJS):
        pytest.skip("kernel objects not built (run the build first)")
    inc = ["-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    api_o, drv_o, exe = str(tmp_path / "api.o"), str(tmp_path / "drv.o"), str(tmp_path / "abi_sanitize")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-w", "-D__HIP_PLATFORM_AMD__", *SAN, *inc, "-c",
          os.path.join(CSRC, "api.cpp"), "-o", api_o])
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, *inc, "-c", os.path.join(ROOT, "tests", "abi_sanitize.cpp"),
          "-o", drv_o])
    _run(["g++", *SAN, drv_o, api_o, *OBJS, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
          "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ALL OK" in r.stdout, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
