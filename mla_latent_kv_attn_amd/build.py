"""Build libmla_attn.so in-tree with hipcc for gfx950.

Every HIP source under ``csrc/`` is compiled to an object (in parallel) and
linked into ``mla_latent_kv_attn_amd/libmla_attn.so``.  The benchmark's
calibration kernel (``calib/mfma_rate.hip``, not part of the library) is
built alongside into ``libmla_calib.so``.  The flags disable
packed-fp32 instruction selection (``-packed-fp32-ops``) so that fp32 math
is emitted as scalar VALU operations.

Usage: ``python -m mla_latent_kv_attn_amd.build [--asm]``; ``--asm`` also
writes the gfx950 assembly of each source next to its object for inspection.
"""

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla_attn.so")
CALIB_SRC = os.path.join(PKG, "calib", "mfma_rate.hip")
CALIB_LIB = os.path.join(PKG, "libmla_calib.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line.
    out = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)


def build(asm=False, verbose=False):
    """Compile and link the library (and the benchmark's calibration
    library); returns the library's path.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    calib_obj = os.path.join(BUILD_DIR, "calib_mfma_rate.o")

    def compile_one(pair):
        src, obj = pair
        out = _run([HIPCC, *COMMON_FLAGS, "-c", src, "-o", obj])
        if asm:
            _run([HIPCC, *COMMON_FLAGS, "--cuda-device-only", "-S", src, "-o", obj[:-2] + ".s"])
        return out

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        for out in ex.map(compile_one, zip(srcs + [CALIB_SRC], objs + [calib_obj])):
            if verbose and out.strip():
                print(out)
    _link(objs, LIB, verbose)
    _link([calib_obj], CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    path = build(asm="--asm" in sys.argv, verbose=True)
    print(path)
