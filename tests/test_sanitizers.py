"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no device).

* The oracle, nsa_oracle.c, built by gcc with -fsanitize=address,undefined, runs the oracle's
  pin tests and the parity-rule tests in a child process (the sanitizer runtime preloaded).
* The C ABI's host side (api.hip: argument and shape checks, workspace planning, status
  strings, the early returns of every entry point), its host code built by clang with the same
  sanitizers and linked with the kernel objects of build(), runs the ABI tests; no kernel is
  launched on those paths.
Any report aborts the child, which fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dynamic_block_sparse_fwd_amd", "csrc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(env_extra, tests):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *tests], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                           "-D_DEFAULT_SOURCE", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", lib,
                           os.path.join(ROOT, "oracle", "nsa_oracle.c"), "-lm"])
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    out = _child({"NSA_ORACLE_LIB": lib, "LD_PRELOAD": asan},
                 ["tests/test_oracle_pins.py", "tests/test_parity_rules.py"])
    print(out.strip().splitlines()[-1])


def _clang_asan_runtime():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def _built_objects():
    """The kernel translation units as build() compiled them (their device code is needed to
    load the library; their host side is launch wrappers only)."""
    objs = sorted(glob.glob(os.path.join(ROOT, "dynamic_block_sparse_fwd_amd", "_build",
                                         "*.hip.o")))
    return [o for o in objs if not o.endswith("api.hip.o")]


@pytest.mark.skipif(_clang_asan_runtime() is None, reason="clang's ASan runtime not installed")
@pytest.mark.skipif(not _built_objects(), reason="the library has not been built (build())")
def test_abi_host_side_under_asan_ubsan(tmp_path):
    api = str(tmp_path / "api_san.o")
    subprocess.check_call(
        ["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
         "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, "api.hip"), "-o", api],
        stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    lib = str(tmp_path / "libnsa_san.so")
    subprocess.check_call(["/opt/rocm/llvm/bin/clang++", "-shared", "-shared-libsan",
                           "-fsanitize=address,undefined", api, *_built_objects(),
                           "-L/opt/rocm/lib", "-lamdhip64", "-o", lib])
    out = _child({"NSA_LIBRARY": lib, "LD_PRELOAD": _clang_asan_runtime()},
                 ["tests/test_abi.py"])
    print(out.strip().splitlines()[-1])
