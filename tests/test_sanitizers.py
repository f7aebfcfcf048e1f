"""The oracle's pins and the library's host-side argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

- oracle.cpp is rebuilt with g++ -fsanitize=address,undefined and every oracle pin test runs
  against that build in a child process that preloads GCC's sanitizer runtime;
- the library is rebuilt for gfx950 with the sanitizers on the host pass only (each -fsanitize=
  right after -Xarch_host; the GPU code is built as usual and never runs here) and the C-ABI CPU
  tests run against that build in a child process that preloads clang's sanitizer runtime.
Undefined behaviour or a memory error aborts the child, which fails the test."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_decode_gqa_amd", "csrc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child_env(preload, **extra):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env["LD_PRELOAD"] = preload
    env.update(extra)
    return env


def test_oracle_pins_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run([gxx, "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.cpp"), "-o", str(lib)],
                   check=True)
    blob = lib.read_bytes()
    assert b"__asan_report" in blob and b"__ubsan_handle" in blob, "oracle build is not instrumented"
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    tests = sorted(os.path.join(ROOT, "tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py"))
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-q", "-x", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=_child_env(asan, ORACLE_LIB=str(lib)), capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout


def test_host_abi_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    rt = None
    for root, _, files in os.walk("/opt/rocm/lib/llvm/lib/clang"):
        if "libclang_rt.asan-x86_64.so" in files:
            rt = os.path.join(root, "libclang_rt.asan-x86_64.so")
    if rt is None:
        pytest.skip("clang's shared sanitizer runtime not found")
    srcs = [f for f in os.listdir(CSRC) if f.endswith((".cpp", ".hip"))]
    # the sanitizers go to the host pass only (each -fsanitize= right after -Xarch_host)
    flags = ["-O1", "-g", "-fPIC", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
             "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(f):
        out = tmp_path / (f + ".o")
        subprocess.run([hipcc, *flags, "-c", os.path.join(CSRC, f), "-o", str(out)], check=True,
                       capture_output=True)
        return str(out)

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = tmp_path / "libattn_decode_hostsan.so"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", str(lib)], check=True,
                   capture_output=True)
    blob = lib.read_bytes()
    assert b"__asan_report" in blob and b"__ubsan_handle" in blob, "library build is not instrumented"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitized_abi_driver.py"), str(lib)],
                       cwd=ROOT, env=_child_env(rt), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
