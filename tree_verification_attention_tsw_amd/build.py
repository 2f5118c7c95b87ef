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
SOURCES = [os.path.join(CSRC, n) for n in ("tsw_api.cpp", "tsw_kernels.hip", "tsw_mfma.hip")]
HEADERS = [os.path.join(CSRC, n) for n in ("tsw_internal.h", "tsw_device.h")] + [
    os.path.join(INCLUDE, "tsw.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + INCLUDE, "-I" + CSRC,
]


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


def _filter(text):
    # hipcc's host pass does not know the device-only target feature; that
    # warning is expected and harmless.
    return "\n".join(l for l in text.splitlines()
                     if "packed-fp32-ops" not in l and "not a recognized feature" not in l)


def build(verbose=False):
    """Compile every source (in parallel) and link libtsw.so; always rebuilds."""
    import concurrent.futures as cf
    import tempfile

    with tempfile.TemporaryDirectory(prefix="tsw_build_") as tmpd:
        objs = [os.path.join(tmpd, os.path.basename(src) + ".o") for src in SOURCES]
        cmds = [[HIPCC] + FLAGS + ["-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with cf.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, stdout=subprocess.PIPE,
                                                           stderr=subprocess.STDOUT, text=True),
                                  cmds))
        for c, res in zip(cmds, results):
            out = _filter(res.stdout)
            if res.returncode != 0:
                sys.stderr.write(out + "\n")
                raise RuntimeError("hipcc failed: " + " ".join(c))
            if verbose and out.strip():
                print(out)
        tmp = LIB + ".tmp%d" % os.getpid()
        link = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp]
        res = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + "\n")
            raise RuntimeError("hipcc link failed")
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
