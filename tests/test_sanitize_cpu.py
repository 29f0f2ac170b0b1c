"""Host AddressSanitizer + UndefinedBehaviorSanitizer build of the plan code.

api.cpp (validation, plan building, status and error text; host code only) is compiled with both
sanitizers, linked with stand-ins for the kernel tables (tests/sanitize/variant_stubs.cpp) and
driven through the C ABI's GPU-free paths by tests/sanitize/abi_errors.c: every bsg_problem
validation rule, the ABI-1 / ABI-2 struct sizes, unknown status codes, invalid plan handles and
the BSG_FORCE_ARCH refusal.  Any invalid access or undefined behaviour aborts the driver."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_precision_gemm_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
SANITIZERS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_error_paths_under_asan_and_ubsan(tmp_path):
    hip_compiler = os.path.join(ROCM, "bin", "hipcc")
    if not (os.path.exists(hip_compiler) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    # api.cpp needs the HIP headers, so it goes through the HIP compiler driver as host C++; each
    # sanitizer flag is marked for the host side.  The other two files are plain C / C++.
    host_only = [x for f in SANITIZERS for x in ("-Xarch_host", f)]
    common = ["-O1", "-g", "-fno-omit-frame-pointer", f"-I{INCLUDE}"]
    _run([hip_compiler, "-std=c++17", "-fPIC", *common, f"-I{CSRC}", *host_only, "-c",
          os.path.join(CSRC, "api.cpp"), "-o", str(tmp_path / "api.o")])
    _run([CLANG + "++", "-std=c++17", *common, *SANITIZERS, "-c", os.path.join(HERE, "variant_stubs.cpp"),
          "-o", str(tmp_path / "stubs.o")])
    _run([CLANG, "-std=c99", "-Wall", *common, *SANITIZERS, "-c", os.path.join(HERE, "abi_errors.c"),
          "-o", str(tmp_path / "drv.o")])
    exe = str(tmp_path / "abi_errors")
    _run([CLANG + "++", *SANITIZERS[:2], str(tmp_path / "api.o"), str(tmp_path / "stubs.o"), str(tmp_path / "drv.o"),
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    env = dict(os.environ, BSG_FORCE_ARCH="gfx942", ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env, timeout=120)
    assert "ok: 0 failures" in r.stdout, r.stdout
