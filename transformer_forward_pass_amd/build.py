"""Build libmak.so (gfx950) from csrc/*.hip with hipcc.

Every HIP source is compiled with packed-FP32 instructions disabled and
without floating-point contraction (the rounding schedule places every fp32
rounding explicitly)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmak.so")
OBJ_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


MICRO = os.path.join(HERE, "microbench")
MICRO_BIN = os.path.join(MICRO, "bin")


def build_microbench(verbose: bool = False) -> None:
    """Standalone measurement programs (sync_cost, mem_stream, copy_calib, bf16_convert, fp64_mfma)."""
    os.makedirs(MICRO_BIN, exist_ok=True)
    srcs = sorted(f for f in os.listdir(MICRO) if f.endswith(".hip"))

    def one(f):
        out = os.path.join(MICRO_BIN, f[:-4])
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=" + ARCH, "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
               "-o", out, os.path.join(MICRO, f)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (f, r.stderr))
        return out
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        outs = list(ex.map(one, srcs))
    if verbose:
        print("built", " ".join(os.path.basename(o) for o in outs))


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    build_microbench(verbose=True)
