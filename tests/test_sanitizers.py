"""Host-side code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only, no GPU): the oracle (gcc, every entry point on small inputs) and the
library's host code in csrc/api.hip (compiled host-only with the
sanitizers, linked against the library's own kernel objects): the host and
file gathers with the worker pool, the training index, sizes, constants,
the host state release and the argument checks of the GPU entry points.
Drivers: tests/sanitize/."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(ROOT, "mixture_lookup_experts_amd", "_build")
ROCM = "/opt/rocm"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-o", exe, os.path.join(SAN, "oracle_driver.c"), "-lm"])
    r = run([exe], env=ENV)
    assert "oracle driver: ok" in r.stdout and "runtime error" not in r.stderr


def test_library_host_code_under_asan_ubsan(tmp_path):
    hipcc, clang = os.path.join(ROCM, "bin", "hipcc"), os.path.join(ROCM, "llvm", "bin", "clang++")
    kernels = [p for p in glob.glob(os.path.join(BUILD, "*.hip.o")) if not p.endswith("api.hip.o")]
    if not (os.path.exists(hipcc) and os.path.exists(clang)) or not kernels:
        pytest.skip("needs hipcc and the library's kernel objects (run the package build first)")
    api = str(tmp_path / "api_host.o")
    # host-only compile of the entry points, sanitizers on the host side only
    run([hipcc, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-c", os.path.join(ROOT, "mixture_lookup_experts_amd", "csrc", "api.hip"), "-o", api])
    drv = str(tmp_path / "driver.o")
    run([clang, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-c",
         os.path.join(SAN, "api_host_driver.cpp"), "-o", drv])
    objs = []
    for k in kernels:  # (kernel objects under names the linker takes as objects)
        dst = str(tmp_path / (os.path.basename(k).replace(".hip.o", "_k.o")))
        shutil.copy(k, dst)
        objs.append(dst)
    exe = str(tmp_path / "api_host_driver")
    run([clang, "-fsanitize=address,undefined", "-o", exe, drv, api, *objs, "-L" + os.path.join(ROCM, "lib"),
         "-lamdhip64", "-lpthread", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    r = run([exe, str(tmp_path)], env=ENV)
    assert "api host driver: ok" in r.stdout and "runtime error" not in r.stderr
