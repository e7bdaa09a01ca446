"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two C drivers in tests/sanitizers/ are built with the sanitizers and run:
- the fp64 oracle (oracle/kda_oracle.c, built with gcc) on small inputs held in
  heap blocks of exactly their documented sizes, with its argument errors and
  the alpha = 1, beta = 0 closed form;
- the C ABI's host code (kda_api.cpp, built by hipcc with the sanitizers on its
  host side only) through argument checks, workspace quotes and plans over a
  grid of shapes and the window planning of kda_chunk_fwd_windowed(_ex), up to
  the first launch, which fails without a GPU.  The driver refuses to run where
  a GPU is visible (exit 77: skipped), since its device pointers are
  placeholders.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVERS = os.path.join(ROOT, "tests", "sanitizers")
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    exe = str(tmp_path / "oracle_san")
    rc, out = _run([gcc, "-std=c11", "-O1", "-g", "-fopenmp", *SAN, os.path.join(DRIVERS, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env={**os.environ, "OMP_NUM_THREADS": "4"})
    assert rc == 0 and "ok" in out, out


def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc, clang = f"{ROCM}/bin/hipcc", f"{ROCM}/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("the ROCm compilers are not installed")
    from linear_attention_sequence_gated_amd import build
    if build.is_stale():
        build.build()
    api = str(tmp_path / "kda_api_san.o")
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]   # device code is built as usual
    rc, out = _run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", *host_san, "-x", "hip", "-c",
                    os.path.join(ROOT, "linear_attention_sequence_gated_amd", "csrc", "kda_api.cpp"), "-o", api])
    assert rc == 0, out
    drv = str(tmp_path / "abi_driver.o")
    rc, out = _run([clang, "-std=c11", "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(DRIVERS, "abi_driver.c"), "-o", drv])
    assert rc == 0, out
    libdir = os.path.dirname(build.LIB)
    exe = str(tmp_path / "abi_san")
    # the sanitized entry points in the executable take precedence over the
    # library's; the launchers and planning helpers come from libkda.so
    rc, out = _run([f"{ROCM}/llvm/bin/clang++", "-fsanitize=address,undefined", drv, api, "-L", libdir, "-lkda",
                    f"-Wl,-rpath,{libdir}", f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    assert rc == 0, out
    # the HIP runtime keeps allocations until exit: leaks are not checked
    rc, out = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    if rc == 77:
        pytest.skip("a GPU is visible: the driver's placeholder pointers must not reach it")
    assert rc == 0 and "ok" in out, out
