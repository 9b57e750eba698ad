"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

* The plan scheduler and the C-ABI layer (plan.cpp, api.cpp) are rebuilt
  with -fsanitize=address,undefined and linked with the library's own gfx950
  objects; the ABI / plan tests (tests/test_abi_plan.py: validation errors,
  coverage of every (request, kv head, token), cascade, append, tuning) run
  against that build.
* The oracle (oracle.c) is rebuilt the same way and its pins
  (tests/test_oracle.py) run against it.

Each runs in a child process with the sanitizer runtimes preloaded (Python
itself is not instrumented; leak checking is off for that reason).  Any
report aborts the child, so a non-zero exit fails the test."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _runtime():
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                           text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            pytest.skip(f"{name} not available")
        libs.append(p)
    return " ".join(libs)


def _env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime()
    env["ASAN_OPTIONS"] = ("detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:"
                           "abort_on_error=1")
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def _child(code, env):
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_plan_and_abi_under_sanitizers(tmp_path):
    from paged_kv_decode_fi_amd import build as b
    objs = [os.path.join(b.OUT_DIR, s + ".o") for s in b.HIP_SOURCES]
    if not all(os.path.exists(o) for o in objs):
        b.build()
    san_objs = []
    for src in b.CXX_SOURCES:
        o = str(tmp_path / (src + ".o"))
        subprocess.check_call(["g++", "-std=c++17", "-fPIC", "-Wall", *SAN,
                               "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(b.ROCM, "include"),
                               "-I", b.CSRC, "-I", b.INC, "-c", os.path.join(b.CSRC, src),
                               "-o", o])
        san_objs.append(o)
    lib = str(tmp_path / "libfi_decode_san.so")
    subprocess.check_call(["g++", "-shared", *SAN, *san_objs, *objs,
                           "-L", os.path.join(b.ROCM, "lib"), "-lamdhip64",
                           "-Wl,-rpath," + os.path.join(b.ROCM, "lib"), "-o", lib])
    code = f"""
import sys
sys.path.insert(0, {ROOT!r})
import paged_kv_decode_fi_amd as m
m.LIB_PATH = {lib!r}
import pytest
rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_abi_plan.py"])
maps = open("/proc/self/maps").read()
assert {lib!r} in maps and "libasan" in maps, "the sanitized library was not the one loaded"
sys.exit(rc)
"""
    out = _child(code, _env())
    assert " passed" in out


def test_oracle_under_sanitizers(tmp_path):
    import oracle
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
                           *SAN, oracle.SRC_PATH, "-o", lib, "-lm"])
    code = f"""
import sys
sys.path.insert(0, {ROOT!r})
import oracle
oracle.LIB_PATH = {lib!r}
oracle.build = lambda force=False: {lib!r}
import pytest
rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle.py"])
maps = open("/proc/self/maps").read()
assert {lib!r} in maps and "libasan" in maps, "the sanitized oracle was not the one loaded"
sys.exit(rc)
"""
    out = _child(code, _env())
    assert " passed" in out
