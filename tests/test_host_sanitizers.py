"""The library's host code (the partitioner and the host AdamW with its thread
pool) under AddressSanitizer and UndefinedBehaviorSanitizer: a host-only
build of layout.cpp and offload.cpp (device entry points stubbed) runs the
host tests in a child process with the sanitizer runtime preloaded. Any
report aborts the child. Skipped where ROCm's clang or its sanitizer runtime
is missing. A second build of the same host code with GCC, the fallback host
compiler, runs the same tests."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fsdp_sharded_mixed_zero_amd", "csrc")
CLANG = "/opt/rocm/lib/llvm/bin/clang++"

# host tests that do not reach the (stubbed) device entry points
HOST_TESTS = ["tests/test_offload_cpu.py", "tests/test_oracle_layout.py", "tests/test_abi_cpu.py"]
DESELECT = "not device_calls_reject and not workspace_size_is_bounded and not empty_ranges"


def test_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not found")
    runtime = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("sanitizer runtime not found")
    lib = str(tmp_path / "libzero_host_sanitized.so")
    build = [CLANG, "-shared", "-fPIC", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
             "-std=c++17", "-fno-math-errno", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
             os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "offload.cpp"),
             os.path.join(ROOT, "tests", "sanitize", "device_stubs.cpp"), "-pthread", "-o", lib]
    r = subprocess.run(build, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=runtime, ZERO_MI355X_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "-k", DESELECT, *HOST_TESTS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


def test_host_code_built_with_gcc(tmp_path):
    """The same host-only build with GCC, the build's fallback host compiler
    (on GCC before 12 the host update has no AVX clones, only the baseline
    loop): the host tests pass against it."""
    import shutil

    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    lib = str(tmp_path / "libzero_host_gcc.so")
    build = [gxx, "-shared", "-fPIC", "-O3", "-std=c++17", "-Wall", "-Werror", "-fno-math-errno",
             "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-I", "/opt/rocm/include", os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "offload.cpp"),
             os.path.join(ROOT, "tests", "sanitize", "device_stubs.cpp"), "-pthread", "-o", lib]
    r = subprocess.run(build, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ZERO_MI355X_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "-k", DESELECT, *HOST_TESTS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


def test_sanitizer_catches_a_planted_overrun(tmp_path):
    """The harness above would pass just as well if the sanitizer never fired:
    a host library built the same way, with a one-element heap overrun, must
    abort the child with AddressSanitizer's report."""
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not found")
    runtime = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("sanitizer runtime not found")
    src = tmp_path / "overrun.cpp"
    src.write_text("#include <vector>\n"
                   "extern \"C\" int overrun(int n) {\n"
                   "  std::vector<int> v(n, 1);\n"
                   "  int s = 0;\n"
                   "  for (int i = 0; i <= n; ++i) s += v.data()[i];   // one past the end\n"
                   "  return s;\n"
                   "}\n")
    lib = str(tmp_path / "liboverrun.so")
    r = subprocess.run([CLANG, "-shared", "-fPIC", "-O1", "-g", "-fno-omit-frame-pointer",
                        "-fsanitize=address,undefined", "-shared-libsan", "-std=c++17", str(src), "-o", lib],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-c", f"import ctypes; print(ctypes.CDLL({lib!r}).overrun(8))"],
                       env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]
