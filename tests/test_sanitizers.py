"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only).

* The fp64 oracle (oracle/kda_oracle.c) is built by gcc with
  -fsanitize=address,undefined -fno-sanitize-recover=all, and the oracle's pin
  and backward tests run against that build in a child process with gcc's
  ASan runtime preloaded: any invalid access, leak-free or not, or undefined
  operation in the oracle aborts the child.
* The C-ABI library's host code (argument validation, aliasing and size
  arithmetic, workspace layouts: kda_api.hip) is rebuilt with clang's
  sanitizers on the host side only (-Xarch_host; the device code and the other
  objects are the regular build's), and the C-ABI validation tests
  (test_abi_cpu.py) run against it the same way.
* A canary program per toolchain shows that its sanitizers are live: a
  one-past-the-end heap read and a signed overflow must each be reported.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_recurrent_attention_chunkwise_amd")
CANARY = os.path.join(ROOT, "tests", "sanitize", "canary.c")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, env=None, timeout=600):
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _check_canary(cc, tmp_path, extra=()):
    exe = str(tmp_path / ("canary_" + os.path.basename(cc)))
    r = _run([cc, "-g", "-O1"] + SAN + list(extra) + ["-o", exe, CANARY])
    assert r.returncode == 0, r.stderr
    assert _run([exe]).returncode == 0
    r = _run([exe, "heap"])   # ASan's report, or UBSan's object-size check first
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or
                                  "insufficient space" in r.stderr), r.stderr[-2000:]
    r = _run([exe, "overflow"])
    assert r.returncode != 0 and "signed integer overflow" in r.stderr, r.stderr[-2000:]


def _pytest_child(tests, env_extra, preload):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"   # the interpreter keeps its arenas
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
    cmd += [os.path.join(ROOT, "tests", t) for t in tests]
    r = _run(cmd, env=env, timeout=900)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    return out


def test_oracle_under_gcc_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    _check_canary("gcc", tmp_path)
    lib = str(tmp_path / "libkda_oracle_san.so")
    r = _run(["gcc", "-O1", "-g"] + SAN + ["-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                                           "-Wextra", "-o", lib,
                                           os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm"])
    assert r.returncode == 0, r.stderr
    asan = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    out = _pytest_child(["test_oracle_pins.py", "test_oracle_backward.py"],
                        {"KDA_ORACLE_LIB": lib}, asan)
    assert " passed" in out


def test_c_abi_validation_under_clang_sanitizers(tmp_path):
    rt = _clang_asan_runtime()
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and rt):
        pytest.skip("ROCm clang or its ASan runtime not found")
    others = [os.path.join(PKG, "_build", s + ".o") for s in
              ("kda_backward", "kda_conv", "kda_decode", "kda_prefill", "kda_prefill16", "kda_split")]
    if not all(os.path.exists(o) for o in others):
        pytest.fail("the library's objects are not built (run __graft_entry__.build())")
    _check_canary(CLANG, tmp_path)
    host = []
    for f in SAN:
        host += ["-Xarch_host", f]
    obj = str(tmp_path / "kda_api_san.o")
    lib = str(tmp_path / "libkda.so")
    common = ["--offload-arch=gfx950", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops"]
    r = _run([HIPCC] + common + ["-O1", "-g", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
                                 "-I" + os.path.join(PKG, "csrc")] + host +
             ["-c", os.path.join(PKG, "csrc", "kda_api.hip"), "-o", obj])
    assert r.returncode == 0, r.stderr
    r = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan"] + host +
             ["-o", lib, obj] + others)
    assert r.returncode == 0, r.stderr
    syms = _run(["nm", "-D", "--undefined-only", lib]).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms
    out = _pytest_child(["test_abi_cpu.py"], {"KDA_TEST_LIB": lib}, rt)
    assert " passed" in out
