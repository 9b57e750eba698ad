"""Builds libfi_decode.so in-tree for gfx950.

    python -m paged_kv_decode_fi_amd.build

HIP sources go through hipcc --offload-arch=gfx950; the host-only plan
scheduler and the C-ABI layer are plain C++ (g++), linked into one shared
library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INC = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfi_decode.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["decode.hip", "prefix.hip", "prefix_rope.hip", "merge.hip", "noalloc.hip"]
CXX_SOURCES = ["plan.cpp", "api.cpp"]

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             # packed fp32 VALU forms are kept out of every kernel
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", CSRC, "-I", INC]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROCM, "include"), "-I", CSRC, "-I", INC]


def _run_all(cmds):
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
             for c in cmds]
    failed = []
    for c, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device feature flag: harmless
        text = "\n".join(ln for ln in text.splitlines()
                         if "packed-fp32-ops" not in ln)
        if p.returncode != 0:
            failed.append((c, text))
        elif text.strip():
            sys.stderr.write(text + "\n")
    if failed:
        msg = "\n\n".join(" ".join(c) + "\n" + t for c, t in failed)
        raise RuntimeError("build failed:\n" + msg)


def build(verbose: bool = False) -> str:
    """Compiles every source (always) and links libfi_decode.so."""
    os.makedirs(OUT_DIR, exist_ok=True)
    objs, cmds = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    cxx = shutil.which("g++") or "g++"
    for src in CXX_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        cmds.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    if verbose:
        for c in cmds:
            print(" ".join(c))
    _run_all(cmds)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run_all([[HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp,
               "-Wl,--no-undefined", "-Wl,-soname,libfi_decode.so"]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
