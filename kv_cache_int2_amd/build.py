"""Compile the OSCAR HIP library (liboscar.so) for gfx950 with hipcc.

Every call recompiles all sources (objects go to _build/ beside the package,
the library is written in place next to this file).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liboscar.so")
ARCH = os.environ.get("OSCAR_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


SAN_LIB = os.path.join(HERE, "liboscar_san.so")
# host-only sanitizers: every -fsanitize applies to the host compilation
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of hipcc's clang (preloaded into
    the Python process that loads the sanitized library)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return hits[-1]


def build_sanitized(verbose: bool = False) -> str:
    """liboscar_san.so: the host C++ (pool, planner, calibration, argument
    checks) built with AddressSanitizer and UndefinedBehaviorSanitizer, linked
    with the regular device objects.  For host tests on the CPU only."""
    hipcc = _hipcc()
    if not all(os.path.exists(os.path.join(BUILD, f + ".o")) for f in os.listdir(CSRC) if f.endswith(".hip")):
        build(verbose)
    san_dir = os.path.join(BUILD, "san")
    os.makedirs(san_dir, exist_ok=True)
    objs = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip"):
            objs.append(os.path.join(BUILD, f + ".o"))
        elif f.endswith(".cpp"):
            obj = os.path.join(san_dir, f + ".o")
            out = _run([hipcc, *COMMON, *SAN_FLAGS, "-c", os.path.join(CSRC, f), "-o", obj])
            if verbose and out.strip():
                print(out, file=sys.stderr)
            objs.append(obj)
    tmp = SAN_LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *SAN_FLAGS, "-shared-libasan", *objs, "-o", tmp])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    jobs = []
    for f in srcs:
        obj = os.path.join(BUILD, f + ".o")
        lang = ["-x", "hip"] if f.endswith(".hip") else []
        jobs.append((obj, [hipcc, *COMMON, *lang, "-c", os.path.join(CSRC, f), "-o", obj]))
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[j[0] for j in jobs], "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose=True))
    else:
        print(build(verbose=True))
