"""The C-ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only: no GPU code is built with them).

api.cpp, where every entry point validates its arguments before any launch,
is compiled with the host sanitizers (each -fsanitize= behind -Xarch_host, so
the device code is untouched) and linked with the library's other objects
from the in-tree build; then the ABI tests of test_abi_cpu.py (invalid
sizes, NULL and misaligned pointers, out-of-range enums, T = 0, workspace
queries, host refusal of the allocation-free entry point) run against that
library in a child process with the ASan runtime preloaded.  Any sanitizer
report fails the test.  Skipped when the ROCm toolchain, the sanitizer
runtime or the in-tree objects are missing."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_layer_bias_amd")
BUILD = os.path.join(PKG, "_build")
OTHER_OBJS = ["route.hip.o", "gemm_mfma.hip.o", "gemm_packed.hip.o", "gemm_fp8.hip.o",
              "gemm_simt.hip.o", "backward.hip.o"]


def _tools():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    objs = [os.path.join(BUILD, o) for o in OTHER_OBJS]
    if not os.path.exists(hipcc) or not rt or not all(os.path.exists(o) for o in objs):
        return None
    return hipcc, rt[-1], objs


def test_abi_validation_is_clean_under_asan_and_ubsan(tmp_path):
    tools = _tools()
    if tools is None:
        pytest.skip("needs hipcc, the clang ASan runtime and the in-tree build objects")
    hipcc, asan_rt, objs = tools
    obj = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libmoe_zc_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    compile_cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC",
                   "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   *san, "-c", os.path.join(PKG, "csrc", "api.cpp"), "-o", obj]
    r = subprocess.run(compile_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    link_cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC",
                "-Xarch_host", "-fsanitize=address,undefined", "-shared-libsan", "-o", lib, obj, *objs]
    r = subprocess.run(link_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    child = (
        "import sys, pytest\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import mixture_experts_layer_bias_amd._lib as L\n"
        f"L.LIB_PATH = {lib!r}\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
        f"{os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))\n")
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout
