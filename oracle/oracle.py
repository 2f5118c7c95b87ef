"""ctypes binding of the float64 C oracle (tsw_oracle.c) -- TEST INFRASTRUCTURE.

The oracle is a plain statement of tree-verification attention in float64:
every (tree node, query head) row attends to the committed prefix (all of it,
or an index list) plus the node's own ancestor-or-self rows of the tree, with
an ordinary softmax.  Used only by tests, the smoke check and the benchmark's
CPU baseline; the GPU path never touches it.
"""
import ctypes
import os
import subprocess

import numpy as np

ORACLE_OK = 0
ORACLE_EINVAL = -1
ORACLE_EBADTREE = -2

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "tsw_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def lib_path():
    return _LIB


def compile_oracle(src, out):
    """gcc -O2 with IEEE semantics (no fast-math); OpenMP only over rows."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force=True):
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(SRC):
        return _LIB
    return compile_oracle(SRC, _LIB)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _as_input(x):
    """numpy float32 array, or a uint16 array of bfloat16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, 0
    if x.dtype == np.uint16:
        return x, 1
    raise TypeError("oracle inputs must be float32 or bfloat16 bits (uint16), got %s" % x.dtype)


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        i32, i64, vp, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.oracle_mask_build.argtypes = [vp, i32, vp, vp]
        lib.oracle_mask_build.restype = i32
        lib.oracle_tree_attn.argtypes = [i32, i32, i32, i32, i64, i32, vp, vp, vp, i64, vp, vp,
                                         i64, dbl, vp, i64, vp, vp, i32]
        lib.oracle_tree_attn.restype = i32
        lib.oracle_lse_merge.argtypes = [i32, i64, i32, vp, vp, vp, vp]
        lib.oracle_lse_merge.restype = i32
        self.lib = lib
        self.path = path

    def mask_build(self, parent):
        """parent[] -> (mask uint64[T], depth int32[T]); raises on a bad tree."""
        parent = np.ascontiguousarray(parent, dtype=np.int32)
        T = parent.shape[0]
        mask = np.zeros(max(T, 1), dtype=np.uint64)
        depth = np.zeros(max(T, 1), dtype=np.int32)
        rc = self.lib.oracle_mask_build(_ptr(parent), T, _ptr(mask), _ptr(depth))
        if rc != ORACLE_OK:
            raise ValueError("oracle_mask_build failed: %d" % rc)
        return mask[:T], depth[:T]

    def tree_attn(self, q, k, v, parent, n_prefix, scale, idx=None, rows=None, nthreads=1):
        """Float64 tree attention.

        q: [T, Hq, d]; k, v: [Hkv, cap, d] (cap >= n_prefix + T), same dtype
        (float32, or uint16 holding bfloat16 bits).  idx: optional sorted
        distinct positions < n_prefix (partial-KV variant).  rows: optional
        flat (node * Hq + head) row list.  Returns float64 (o, lse): o [T, Hq, d]
        and lse [T, Hq] for all rows, or o [n_rows, d], lse [n_rows] for a list.
        """
        q, dt = _as_input(q)
        k, dtk = _as_input(k)
        v, dtv = _as_input(v)
        if not (dt == dtk == dtv):
            raise TypeError("q, k, v must share a dtype")
        T, Hq, d = q.shape
        Hkv, cap, dk = k.shape
        if v.shape != k.shape or dk != d:
            raise ValueError("shape mismatch")
        parent = np.ascontiguousarray(parent, dtype=np.int32)
        if idx is not None:
            idx = np.ascontiguousarray(idx, dtype=np.int32)
        if rows is not None:
            rows = np.ascontiguousarray(rows, dtype=np.int32)
            n_out = rows.shape[0]
            o = np.zeros((n_out, d), dtype=np.float64)
            lse = np.zeros(n_out, dtype=np.float64)
        else:
            n_out = T * Hq
            o = np.zeros((T, Hq, d), dtype=np.float64)
            lse = np.zeros((T, Hq), dtype=np.float64)
        rc = self.lib.oracle_tree_attn(
            T, Hq, Hkv, d, int(n_prefix), dt, _ptr(q), _ptr(k), _ptr(v), cap * d, _ptr(parent),
            _ptr(idx), 0 if idx is None else idx.shape[0], float(scale),
            _ptr(rows), 0 if rows is None else n_out, _ptr(o), _ptr(lse), int(nthreads))
        if rc == ORACLE_EBADTREE:
            raise ValueError("bad tree")
        if rc != ORACLE_OK:
            raise ValueError("oracle_tree_attn failed: %d" % rc)
        return o, lse

    def lse_merge(self, part_o, part_lse):
        """Merge partial results: part_o [S, R, d], part_lse [S, R] (float64)."""
        part_o = np.ascontiguousarray(part_o, dtype=np.float64)
        part_lse = np.ascontiguousarray(part_lse, dtype=np.float64)
        S, R, d = part_o.shape
        o = np.zeros((R, d), dtype=np.float64)
        lse = np.zeros(R, dtype=np.float64)
        rc = self.lib.oracle_lse_merge(S, R, d, _ptr(part_o), _ptr(part_lse), _ptr(o), _ptr(lse))
        if rc != ORACLE_OK:
            raise ValueError("oracle_lse_merge failed: %d" % rc)
        return o, lse


_default = None


def default():
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(_LIB)
    return _default


def mask_build(parent):
    return default().mask_build(parent)


def tree_attn(*a, **kw):
    return default().tree_attn(*a, **kw)


def lse_merge(*a, **kw):
    return default().lse_merge(*a, **kw)
