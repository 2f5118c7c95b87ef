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
# Matrix-core kernel shapes (waves, row groups, query blocks per wave); each
# one is its own object compiled from tsw_mfma_inst.hip, so they build in
# parallel.
MFMA_SHAPES = [(4, 1, 1), (4, 1, 2), (8, 2, 2), (8, 4, 2), (8, 4, 3), (8, 8, 2), (8, 8, 3)]
# (source, extra flags, object name)
UNITS = [(os.path.join(CSRC, n), [], n + ".o")
         for n in ("tsw_api.cpp", "tsw_kernels.hip", "tsw_mfma.hip", "tsw_accept.hip", "tsw_select.hip",
                   "tsw_stream.hip", "tsw_noalloc.hip")] + [
    (os.path.join(CSRC, "tsw_mfma_inst.hip"), ["-DTSW_W=%d" % w, "-DTSW_R=%d" % r, "-DTSW_NB=%d" % nb],
     "tsw_mfma_%d_%d_%d.o" % (w, r, nb)) for w, r, nb in MFMA_SHAPES]
SOURCES = sorted(set(u[0] for u in UNITS))
HEADERS = [os.path.join(CSRC, n) for n in ("tsw_internal.h", "tsw_device.h", "tsw_mfma_impl.h")] + [
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
        objs = [os.path.join(tmpd, name) for _, _, name in UNITS]
        cmds = [[HIPCC] + FLAGS + extra + ["-c", src, "-o", obj]
                for (src, extra, _), obj in zip(UNITS, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
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
