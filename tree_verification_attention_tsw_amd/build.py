"""Builds libtsw.so (the gfx950 HIP kernels plus the C entry points of
include/tsw.h) in-tree with hipcc."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtsw.so")
SOURCES = [os.path.join(CSRC, "tsw_api.cpp"), os.path.join(CSRC, "tsw_kernels.hip")]
HEADERS = [os.path.join(CSRC, "tsw_internal.h"), os.path.join(INCLUDE, "tsw.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + INCLUDE, "-I" + CSRC,
]


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


def build(verbose=False):
    """Compile every source into libtsw.so (always rebuilds)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only target feature; that
    # warning is expected and harmless.
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l
                    and "not a recognized feature" not in l)
    if res.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed building libtsw.so")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
