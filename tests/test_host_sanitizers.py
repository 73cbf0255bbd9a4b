"""The C-ABI's host code (argument validation, workspace planning, launch
sequencing in api.hip) under AddressSanitizer and UndefinedBehaviorSanitizer.

A second build of libsalad.so is made with api.hip's host pass instrumented
(-Xarch_host, so the GPU code is built as usual; undefined behaviour traps),
linked with clang's shared ASan runtime, and the host-side C-ABI tests run
against it in a child process that preloads that runtime.  No GPU is used:
every call in those tests returns from validation before any launch.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_linear_hybrid_st_amd")
BUILD = os.path.join(PKG, "_build")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_c_abi_host_code_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    objs = sorted(glob.glob(os.path.join(BUILD, "*.o")))
    if rt is None or not os.path.exists(CLANG):
        pytest.skip("clang's ASan runtime is not installed")
    if not any(o.endswith("api.hip.o") for o in objs):
        pytest.skip("libsalad.so has not been built (python -m sparse_linear_hybrid_st_amd.build)")
    api_o = str(tmp_path / "api_asan.o")
    compile_cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result",
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fsanitize-trap=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o]
    r = subprocess.run(compile_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lib = str(tmp_path / "libsalad_asan.so")
    others = [o for o in objs if not o.endswith("api.hip.o")]
    link_cmd = [CLANG, "-shared", "-fPIC", "-shared-libasan", "-fsanitize=address", "-o", lib, api_o,
                *others, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(link_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, SALAD_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verbosity=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py"),
                        os.path.join(ROOT, "tests", "test_zz_no_alloc.py")],
                       capture_output=True, text=True, env=env, cwd=str(tmp_path), timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" in out or "asan" in out.lower(), "the ASan runtime did not start"
    assert "passed" in r.stdout
