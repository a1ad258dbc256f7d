"""Sanitized CPU builds (AddressSanitizer + UndefinedBehaviorSanitizer).

* The oracle, oracle/ssd_oracle.c, built with -fsanitize=address,undefined,
  runs its own pins (tests/test_oracle*.py: the dual form, the chunked form,
  closed forms, invariants, the gradient against finite differences) in a
  child process.
* The library's host code (argument checks, workspace arithmetic, status
  strings), built with the sanitizers on its host side only, runs the C-ABI
  tests (tests/test_abi.py), which make no GPU call.
* A planted out-of-bounds write in a throwaway C function shows that the
  sanitizer is active in such a child process.

Any sanitizer report aborts the child, which fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mamba_ssd_chunked_scan_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtimes():
    libs = [subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
            for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in libs):
        pytest.skip("gcc sanitizer runtimes are not installed")
    return " ".join(libs)


def _gcc_san_so(src, out):
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-fopenmp",
                           "-ffp-contract=off", "-fno-fast-math",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-shared", "-fPIC", "-o", out, src, "-lm"])


def _child(args, env_extra, timeout=600):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


def test_sanitizer_catches_planted_overflow(tmp_path):
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int planted(int n) { int *a = malloc(n * sizeof(int));\n"
                   "  for (int i = 0; i <= n; ++i) a[i] = i;\n"
                   "  int s = a[n - 1]; free(a); return s; }\n")
    so = str(tmp_path / "libplanted.so")
    _gcc_san_so(str(src), so)
    r = _child(["-c", f"import ctypes; ctypes.CDLL({so!r}).planted(8)"],
               {"LD_PRELOAD": _gcc_runtimes()})
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr


def test_oracle_pins_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "libssd_oracle_asan.so")
    _gcc_san_so(os.path.join(ROOT, "oracle", "ssd_oracle.c"), so)
    files = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle*.py")))
    r = _child(["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *files],
               {"LD_PRELOAD": _gcc_runtimes(), "SSD_ORACLE_LIB": so})
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout and "AddressSanitizer" not in r.stderr


def test_abi_checks_under_asan_ubsan(tmp_path):
    rts = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(HIPCC) or not rts:
        pytest.skip("hipcc or its sanitizer runtime is not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    flags = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
             "-I", CSRC, *san, "-Xarch_host", "-fno-omit-frame-pointer"]
    from mamba_ssd_chunked_scan_amd import build as libbuild
    procs, objs = [], []
    for src in libbuild.SOURCES:
        obj = str(tmp_path / (src + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        procs.append(subprocess.Popen([HIPCC, *flags, *lang, "-c", os.path.join(CSRC, src),
                                       "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT))
        objs.append(obj)
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out.decode()[-3000:]
    lib = str(tmp_path / "libssd.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san,
                           "-shared-libsan", "-o", lib, *objs],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    r = _child(["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                os.path.join(ROOT, "tests", "test_abi.py")],
               {"LD_PRELOAD": rts[0], "SSD_LIB": lib})
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout and "Sanitizer" not in r.stderr
