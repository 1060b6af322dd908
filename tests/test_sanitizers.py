"""Sanitizer builds on the CPU: the oracle and the host side of the C ABI under
AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts the run).

- oracle/oracle.c is compiled with gcc -fsanitize=address,undefined (OpenMP on)
  and every pin of tests/oracle_checks.py runs against that build, the ASan
  runtime preloaded into the child Python process.
- csrc/api.cpp (argument checks, workspace layouts, tuning cache) is compiled
  with the sanitizers on its host code only and linked with the library's other
  (device) objects; tests/c_abi_checks.c, a plain C program built with the same
  sanitizers, drives every refusal path, extreme sizes and a tuning-cache file
  round trip through it.  No GPU is touched: every call fails a host check.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "block_sparse_flash_mask_amd")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_pins_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", so, "-lm"])
    asan = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, OMP_NUM_THREADS="4", **SAN_ENV)
    r = _run([sys.executable, os.path.join(HERE, "oracle_checks.py"), so], env=env, cwd=HERE, timeout=900)
    assert r.stdout.strip().splitlines()[-1] == "[]", r.stdout[-2000:]


def test_c_abi_host_checks_under_asan_ubsan(tmp_path):
    from block_sparse_flash_mask_amd import build as hip_build
    if not all(os.path.exists(os.path.join(hip_build.BUILD, os.path.splitext(s)[0] + ".o"))
               for s in hip_build.SOURCES):
        hip_build.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "api_san.o")
    flags = [f for f in hip_build.FLAGS if f != "-O3"]
    _run([hip_build.hipcc(), "-x", "hip", *flags, "-O1", "-g", *san, "-c",
          os.path.join(hip_build.CSRC, "api.cpp"), "-o", api_o])
    others = [os.path.join(hip_build.BUILD, os.path.splitext(s)[0] + ".o") for s in hip_build.SOURCES
              if s != "api.cpp"]
    lib = str(tmp_path / "libbsattn_san.so")
    _run([hip_build.hipcc(), "--offload-arch=" + hip_build.ARCH, "-shared", "-fPIC", "-o", lib, api_o, *others,
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"])
    rt = os.path.dirname(_run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip())
    exe = str(tmp_path / "c_abi_checks")
    _run([CLANG, "-std=c11", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared-libasan",
          "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi_checks.c"), "-o", exe,
          "-L", str(tmp_path), "-lbsattn_san", "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + rt, "-lm"])
    r = _run([exe, str(tmp_path / "tune.json"), str(tmp_path / "missing.json")],
             env=dict(os.environ, **SAN_ENV), timeout=300)
    assert "all host checks returned their documented status" in r.stdout
