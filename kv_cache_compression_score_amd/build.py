"""Build libkvcc.so (all HIP sources under csrc/) for gfx950 with hipcc.

Usage: python -m kv_cache_compression_score_amd.build   (or build() from Python)
Objects go to _build/ next to this file; the library to libkvcc.so here.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvcc.so")

ARCH = "gfx950"
# Packed fp32 ops are disabled for all device code.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
         "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA results straight into VGPRs (no AGPR copies in the epilogues)
         "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


# Per-source extra flags.  The score kernels never carry NaNs (masked logits
# are -inf), so their device code drops the sNaN-quieting v_max that IEEE
# mode puts in front of every fmax of an MFMA result; infinities stay exact.
EXTRA = {"score.hip": ["-Xarch_device", "-fno-honor-nans"]}


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [_hipcc(), *FLAGS, *EXTRA.get(os.path.basename(s), []), "-c", s,
                                 "-o", o]) for s, o in zip(srcs, objs)]
        for f in futs:
            out = f.result()
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


# Host-checking build: the same library with AddressSanitizer and
# UndefinedBehaviorSanitizer on its host code only (argument validation,
# workspace planning, launch set-up); the device code is built as usual.
SAN_DIR = os.path.join(BUILD, "sanitized")
SAN_LIB = os.path.join(SAN_DIR, "libkvcc_sanitized.so")
SAN_FLAGS = FLAGS + ["-g", "-Xarch_host", "-fsanitize=address,undefined",
                     "-Xarch_host", "-fno-sanitize-recover=undefined",
                     "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime (it also carries the UBSan handlers),
    to be preloaded into a process that loads the sanitized library."""
    pat = os.path.join(os.path.dirname(os.path.dirname(_hipcc())), "llvm", "lib", "clang", "*",
                       "lib", "linux", "libclang_rt.asan-x86_64.so")
    found = sorted(glob.glob(pat))
    if not found:
        raise RuntimeError(f"no ASan runtime at {pat}")
    return found[-1]


def build_sanitized(force: bool = False) -> str:
    """Build the host-checking library (reused while it is newer than every
    source, header and this script, unless force)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    deps = srcs + glob.glob(os.path.join(CSRC, "*.hpp")) + \
        glob.glob(os.path.join(INCLUDE, "*.h")) + [os.path.abspath(__file__)]
    if not force and os.path.exists(SAN_LIB) and \
            os.path.getmtime(SAN_LIB) > max(os.path.getmtime(p) for p in deps):
        return SAN_LIB
    objs = [os.path.join(SAN_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        for f in [ex.submit(_run, [_hipcc(), *SAN_FLAGS, *EXTRA.get(os.path.basename(s), []),
                                   "-c", s, "-o", o]) for s, o in zip(srcs, objs)]:
            f.result()
    _run([_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Xarch_host",
          "-fsanitize=address,undefined", "-o", SAN_LIB, *objs])
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))
