"""ctypes binding of libtsw.so (include/tsw.h): argument marshalling only.

Torch tensors supply device memory and the current HIP stream; every step of
the computation runs in the library's kernels.  There is no fallback: if
libtsw.so is missing or fails to load, every call raises.
"""
import ctypes
import os
import re

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtsw.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "tsw.h")

TSW_OK = 0
DTYPE_F32, DTYPE_BF16 = 0, 1
IMPL = {"auto": 0, "valu": 1, "mfma": 2}


class TswError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s: %s (status %d)" % (what, status_str(status), status))
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("d", ctypes.c_int32), ("n_prefix", ctypes.c_int64), ("kv_head_stride", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("impl", ctypes.c_int32), ("scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


class PagedDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("d", ctypes.c_int32), ("page_rows", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("reserved", ctypes.c_int32),
    ]


_lib = None


def lib():
    """The loaded library; raises if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libtsw.so is not built (run __graft_entry__.build() or "
                           "python -m tree_verification_attention_tsw_amd.build); "
                           "there is no CPU fallback")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(AttnDesc)
    L.tsw_tree_mask_build.argtypes = [vp, i32, vp, vp]
    L.tsw_plan_splits.argtypes = [D, i64, ctypes.POINTER(i32)]
    L.tsw_workspace_size.argtypes = [D, i64, ctypes.POINTER(sz)]
    L.tsw_tree_attn_verify.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.tsw_tree_attn_partial.argtypes = [D, vp, vp, vp, vp, vp, i64, vp, vp, vp, sz, vp]
    L.tsw_tree_attn_split.argtypes = [D, vp, vp, vp, vp, vp, i64, i32, vp, vp, vp]
    L.tsw_lse_merge.argtypes = [i32, i64, i32, vp, vp, vp, vp, vp]
    PD = ctypes.POINTER(PagedDesc)
    L.tsw_paged_workspace_size.argtypes = [PD, vp, ctypes.POINTER(sz)]
    L.tsw_tree_attn_verify_paged.argtypes = [PD, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.tsw_paged_partial_workspace_size.argtypes = [PD, vp, vp, ctypes.POINTER(sz)]
    L.tsw_tree_attn_partial_paged.argtypes = [PD, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]
    L.tsw_select_workspace_size.argtypes = [i64, ctypes.POINTER(sz)]
    L.tsw_select_partial.argtypes = [D, vp, vp, vp, i64, i64, vp, vp, vp, sz, vp]
    L.tsw_verify_select_workspace_size.argtypes = [D, ctypes.POINTER(sz)]
    L.tsw_tree_attn_verify_select.argtypes = [D, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, sz, vp]
    L.tsw_context_penalty.argtypes = [vp, i32, vp, i64, i32, vp, vp, i64, i32, ctypes.c_float, vp]
    L.tsw_accept_greedy_penalized.argtypes = [vp, i32, vp, i64, i32, vp, vp, i64, i32, ctypes.c_float, vp, vp, sz,
                                              vp]
    L.tsw_accept_workspace_size.argtypes = [i32, i64, ctypes.POINTER(sz)]
    L.tsw_accept_greedy.argtypes = [vp, i32, vp, i64, i32, vp, vp, vp, sz, vp]
    L.tsw_kv_compact.argtypes = [vp, vp, i32, i64, i32, i32, i32, i64, i64, i32, vp, vp]
    L.tsw_read_stream.argtypes = [D, vp, vp, vp, vp]
    L.tsw_launch_floor.argtypes = [D, i64, vp, vp]
    L.tsw_tree_attn_verify_noalloc.argtypes = [D, vp, vp, vp, vp, vp, vp, vp]
    L.tsw_noalloc_scratch_bytes.argtypes = []
    L.tsw_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.tsw_status_str.argtypes = [ctypes.c_int]
    L.tsw_status_str.restype = ctypes.c_char_p
    for name in ("tsw_tree_mask_build", "tsw_plan_splits", "tsw_workspace_size",
                 "tsw_tree_attn_verify", "tsw_tree_attn_partial", "tsw_tree_attn_split",
                 "tsw_lse_merge", "tsw_accept_workspace_size", "tsw_accept_greedy",
                 "tsw_kv_compact", "tsw_paged_workspace_size", "tsw_tree_attn_verify_paged",
                 "tsw_select_workspace_size", "tsw_select_partial", "tsw_read_stream", "tsw_launch_floor",
                 "tsw_tree_attn_verify_noalloc", "tsw_paged_partial_workspace_size",
                 "tsw_tree_attn_partial_paged"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def declared_functions():
    """Names of the functions include/tsw.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tsw_\w+)\s*\(", text, re.M)))


def status_str(status):
    return lib().tsw_status_str(int(status)).decode()


def _check(rc, what):
    if rc != TSW_OK:
        raise TswError(rc, what)


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dev_ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def tree_mask(parent):
    """Host tree mask: (mask uint64[T], depth int32[T])."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    T = parent.shape[0]
    mask = np.zeros(max(T, 1), dtype=np.uint64)
    depth = np.zeros(max(T, 1), dtype=np.int32)
    _check(lib().tsw_tree_mask_build(_np_ptr(parent), T, _np_ptr(mask), _np_ptr(depth)),
           "tsw_tree_mask_build")
    return mask[:T], depth[:T]


def make_desc(q, k, n_prefix, scale=None, impl="auto"):
    """Descriptor for q [T, Hq, d] and a cache k [Hkv, rows, d]."""
    T, Hq, d = q.shape
    Hkv = k.shape[0]
    if q.dtype == torch.float32:
        dt = DTYPE_F32
    elif q.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    else:
        raise TypeError("q/k/v must be float32 or bfloat16, got %s" % q.dtype)
    desc = AttnDesc()
    desc.T, desc.Hq, desc.Hkv, desc.d = T, Hq, Hkv, d
    desc.n_prefix = int(n_prefix)
    desc.kv_head_stride = int(k.stride(0))
    desc.dtype = dt
    desc.impl = IMPL[impl]
    desc.scale = float(scale) if scale is not None else 1.0 / float(np.sqrt(d))
    desc.reserved = 0
    return desc


def _check_tensors(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [T, Hq, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v dtypes differ")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape and strides")
    if k.dim() != 3 or k.stride(2) != 1 or k.stride(1) != k.shape[2] or k.shape[2] != q.shape[2]:
        raise ValueError("k/v must be [Hkv, rows, d] with contiguous rows")


def _parent_arr(parent):
    return np.ascontiguousarray(parent, dtype=np.int32)


def plan_splits(q, k, n_prefix, n_idx=-1, scale=None, impl="auto"):
    desc = make_desc(q, k, n_prefix, scale, impl)
    n = ctypes.c_int32(0)
    _check(lib().tsw_plan_splits(ctypes.byref(desc), int(n_idx), ctypes.byref(n)), "tsw_plan_splits")
    return n.value


def workspace_size(q, k, n_prefix, n_idx=-1, scale=None, impl="auto"):
    desc = make_desc(q, k, n_prefix, scale, impl)
    n = ctypes.c_size_t(0)
    _check(lib().tsw_workspace_size(ctypes.byref(desc), int(n_idx), ctypes.byref(n)),
           "tsw_workspace_size")
    return n.value


def _workspace(q, k, n_prefix, n_idx, scale, impl, workspace):
    need = workspace_size(q, k, n_prefix, n_idx, scale, impl)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    return workspace


def tree_attn_verify(q, k, v, parent, n_prefix, scale=None, impl="auto", out=None, workspace=None):
    """Tree verification attention; returns (o [T, Hq, d] float32, lse [T, Hq] float32)."""
    _check_tensors(q, k, v)
    T, Hq, d = q.shape
    desc = make_desc(q, k, n_prefix, scale, impl)
    o, lse = out if out is not None else (
        torch.empty((T, Hq, d), dtype=torch.float32, device=q.device),
        torch.empty((T, Hq), dtype=torch.float32, device=q.device))
    ws = _workspace(q, k, n_prefix, -1, scale, impl, workspace)
    p = _parent_arr(parent)
    _check(lib().tsw_tree_attn_verify(ctypes.byref(desc), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v),
                                      _np_ptr(p), _dev_ptr(o), _dev_ptr(lse), _dev_ptr(ws),
                                      ws.numel(), _stream(q)), "tsw_tree_attn_verify")
    return o, lse


def tree_attn_partial(q, k, v, parent, idx, n_prefix, scale=None, impl="auto", out=None,
                      workspace=None):
    """Partial-KV (draft pass) attention over idx (int32 device tensor)."""
    _check_tensors(q, k, v)
    if idx.dtype != torch.int32 or not idx.is_cuda or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 GPU tensor")
    T, Hq, d = q.shape
    n_idx = idx.numel()
    desc = make_desc(q, k, n_prefix, scale, impl)
    o, lse = out if out is not None else (
        torch.empty((T, Hq, d), dtype=torch.float32, device=q.device),
        torch.empty((T, Hq), dtype=torch.float32, device=q.device))
    ws = _workspace(q, k, n_prefix, n_idx, scale, impl, workspace)
    p = _parent_arr(parent)
    _check(lib().tsw_tree_attn_partial(ctypes.byref(desc), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v),
                                       _np_ptr(p), _dev_ptr(idx) if n_idx else None, n_idx,
                                       _dev_ptr(o), _dev_ptr(lse), _dev_ptr(ws), ws.numel(),
                                       _stream(q)), "tsw_tree_attn_partial")
    return o, lse


def tree_attn_split(q, k, v, parent, n_prefix, n_splits, idx=None, scale=None, impl="auto",
                    out=None):
    """First phase only: per-split (part_o [S, T, Hq, d], part_lse [S, T, Hq])."""
    _check_tensors(q, k, v)
    T, Hq, d = q.shape
    desc = make_desc(q, k, n_prefix, scale, impl)
    po, pl = out if out is not None else (
        torch.empty((n_splits, T, Hq, d), dtype=torch.float32, device=q.device),
        torch.empty((n_splits, T, Hq), dtype=torch.float32, device=q.device))
    p = _parent_arr(parent)
    n_idx = idx.numel() if idx is not None else 0
    idx_ptr = _dev_ptr(idx) if idx is not None else None
    if idx is not None and n_idx == 0:
        idx_ptr = _dev_ptr(po)  # non-null marker for the partial variant; never read
    _check(lib().tsw_tree_attn_split(ctypes.byref(desc), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v),
                                     _np_ptr(p), idx_ptr, n_idx, int(n_splits), _dev_ptr(po),
                                     _dev_ptr(pl), _stream(q)), "tsw_tree_attn_split")
    return po, pl


def lse_merge(part_o, part_lse, out=None):
    """Merge partial results: part_o [S, ..., d], part_lse [S, ...] -> (o, lse)."""
    S = part_o.shape[0]
    d = part_o.shape[-1]
    rows = part_lse[0].numel()
    if not (part_o.is_contiguous() and part_lse.is_contiguous()):
        raise ValueError("partials must be contiguous")
    if part_o.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise TypeError("partials must be float32")
    o, lse = out if out is not None else (
        torch.empty(part_o.shape[1:], dtype=torch.float32, device=part_o.device),
        torch.empty(part_lse.shape[1:], dtype=torch.float32, device=part_o.device))
    _check(lib().tsw_lse_merge(S, rows, d, _dev_ptr(part_o), _dev_ptr(part_lse), _dev_ptr(o),
                               _dev_ptr(lse), _stream(part_o)), "tsw_lse_merge")
    return o, lse


class PreparedCall:
    """A C entry point with every argument marshalled once, for tight loops
    (benchmarks, serving): calling it costs one ctypes call."""

    def __init__(self, fn, args, what, keep):
        self._fn, self._args, self._what, self._keep = fn, args, what, keep

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != TSW_OK:
            raise TswError(rc, self._what)


def prepare_verify(q, k, v, parent, n_prefix, o, lse, workspace, idx=None, scale=None,
                   impl="auto", stream=None):
    """Bound tsw_tree_attn_verify (idx None) or tsw_tree_attn_partial call."""
    _check_tensors(q, k, v)
    desc = make_desc(q, k, n_prefix, scale, impl)
    p = _parent_arr(parent)
    st = ctypes.c_void_p(stream.cuda_stream if stream is not None
                         else torch.cuda.current_stream(q.device).cuda_stream)
    L = lib()
    if idx is None:
        args = (ctypes.byref(desc), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _np_ptr(p), _dev_ptr(o),
                _dev_ptr(lse), _dev_ptr(workspace), workspace.numel(), st)
        return PreparedCall(L.tsw_tree_attn_verify, args, "tsw_tree_attn_verify", (desc, p))
    args = (ctypes.byref(desc), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _np_ptr(p),
            _dev_ptr(idx) if idx.numel() else None, idx.numel(), _dev_ptr(o), _dev_ptr(lse),
            _dev_ptr(workspace), workspace.numel(), st)
    return PreparedCall(L.tsw_tree_attn_partial, args, "tsw_tree_attn_partial", (desc, p))


def prepare_split(q, k, v, parent, n_prefix, n_splits, part_o, part_lse, idx=None, scale=None,
                  impl="auto", stream=None):
    """Bound tsw_tree_attn_split call (first phase only)."""
    _check_tensors(q, k, v)
    desc = make_desc(q, k, n_prefix, scale, impl)
    p = _parent_arr(parent)
    st = ctypes.c_void_p(stream.cuda_stream if stream is not None
                         else torch.cuda.current_stream(q.device).cuda_stream)
    idx_ptr = _dev_ptr(idx) if idx is not None else None
    if idx is not None and idx.numel() == 0:
        idx_ptr = _dev_ptr(part_o)
    args = (ctypes.byref(desc), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _np_ptr(p), idx_ptr,
            0 if idx is None else idx.numel(), int(n_splits), _dev_ptr(part_o), _dev_ptr(part_lse),
            st)
    return PreparedCall(lib().tsw_tree_attn_split, args, "tsw_tree_attn_split", (desc, p))


def prepare_merge(part_o, part_lse, o, lse, stream=None):
    """Bound tsw_lse_merge call (second phase only)."""
    st = ctypes.c_void_p(stream.cuda_stream if stream is not None
                         else torch.cuda.current_stream(part_o.device).cuda_stream)
    args = (part_o.shape[0], part_lse[0].numel(), part_o.shape[-1], _dev_ptr(part_o),
            _dev_ptr(part_lse), _dev_ptr(o), _dev_ptr(lse), st)
    return PreparedCall(lib().tsw_lse_merge, args, "tsw_lse_merge", None)


# ------------------------------------------------------------ acceptance

def accept_workspace_size(T, vocab):
    n = ctypes.c_size_t(0)
    _check(lib().tsw_accept_workspace_size(int(T), int(vocab), ctypes.byref(n)),
           "tsw_accept_workspace_size")
    return n.value


def _logits_dtype(logits):
    if logits.dtype == torch.float32:
        return DTYPE_F32
    if logits.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError("logits must be float32 or bfloat16")


def _accept_args(parent, logits, draft, result, workspace, stream):
    if logits.dim() != 2 or not logits.is_cuda or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [T, vocab] GPU tensor")
    T, vocab = logits.shape
    if draft.dtype != torch.int32 or not draft.is_cuda or draft.numel() != T:
        raise ValueError("draft must be an int32 GPU tensor of T entries")
    p = _parent_arr(parent)
    if p.shape[0] != T:
        raise ValueError("parent must have T entries")
    if result is None:
        result = torch.empty(2 + 2 * T, dtype=torch.int32, device=logits.device)
    if workspace is None:
        workspace = torch.empty(max(accept_workspace_size(T, vocab), 256), dtype=torch.uint8,
                                device=logits.device)
    st = ctypes.c_void_p(stream.cuda_stream if stream is not None
                         else torch.cuda.current_stream(logits.device).cuda_stream)
    args = (_np_ptr(p), T, _dev_ptr(logits), vocab, _logits_dtype(logits), _dev_ptr(draft),
            _dev_ptr(result), _dev_ptr(workspace), workspace.numel(), st)
    return args, (p, result, workspace)


def _penalty_args(parent, logits, draft, recent, window, theta, stream):
    if logits.dim() != 2 or not logits.is_cuda or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [T, vocab] GPU tensor")
    T, vocab = logits.shape
    for name, x in (("draft", draft), ("recent", recent)):
        if x.dtype != torch.int32 or not x.is_cuda or not x.is_contiguous():
            raise ValueError(name + " must be a contiguous int32 GPU tensor")
    if draft.numel() != T:
        raise ValueError("draft must have T entries")
    p = _parent_arr(parent)
    if p.shape[0] != T:
        raise ValueError("parent must have T entries")
    st = ctypes.c_void_p(stream.cuda_stream if stream is not None
                         else torch.cuda.current_stream(logits.device).cuda_stream)
    args = (_np_ptr(p), T, _dev_ptr(logits), vocab, _logits_dtype(logits), _dev_ptr(draft),
            _dev_ptr(recent) if recent.numel() else None, recent.numel(), int(window), float(theta), st)
    return args, (p, logits, draft, recent)


def context_penalty(parent, logits, draft, recent, window, theta):
    """Contextual penalty on every node's logits, in place (before accept_greedy)."""
    args, _ = _penalty_args(parent, logits, draft, recent, window, theta, None)
    _check(lib().tsw_context_penalty(*args), "tsw_context_penalty")
    return logits


def prepare_penalty(parent, logits, draft, recent, window, theta, stream=None):
    args, keep = _penalty_args(parent, logits, draft, recent, window, theta, stream)
    return PreparedCall(lib().tsw_context_penalty, args, "tsw_context_penalty", keep)


def accept_greedy(parent, logits, draft, result=None, workspace=None):
    """Greedy acceptance; returns the int32 device result [2 + 2T]:
    (L, bonus, path[T] padded with -1, most likely token per node)."""
    args, keep = _accept_args(parent, logits, draft, result, workspace, None)
    _check(lib().tsw_accept_greedy(*args), "tsw_accept_greedy")
    return keep[1]


def _accept_penalized_args(parent, logits, draft, recent, window, theta, result, workspace, stream):
    args, keep = _accept_args(parent, logits, draft, result, workspace, stream)
    if recent.dtype != torch.int32 or not recent.is_cuda or not recent.is_contiguous():
        raise ValueError("recent must be a contiguous int32 GPU tensor")
    # (parent, T, logits, vocab, dtype, draft, result, workspace, bytes, stream) -> insert the penalty
    full = args[:6] + (_dev_ptr(recent) if recent.numel() else None, recent.numel(), int(window),
                       float(theta)) + args[6:]
    return full, keep + (recent,)


def accept_greedy_penalized(parent, logits, draft, recent, window, theta, result=None, workspace=None):
    """Greedy acceptance on the contextually penalised logits (logits unchanged)."""
    args, keep = _accept_penalized_args(parent, logits, draft, recent, window, theta, result, workspace, None)
    _check(lib().tsw_accept_greedy_penalized(*args), "tsw_accept_greedy_penalized")
    return keep[1]


def prepare_accept_penalized(parent, logits, draft, recent, window, theta, result, workspace, stream=None):
    args, keep = _accept_penalized_args(parent, logits, draft, recent, window, theta, result, workspace, stream)
    return PreparedCall(lib().tsw_accept_greedy_penalized, args, "tsw_accept_greedy_penalized", keep)


def prepare_accept(parent, logits, draft, result, workspace, stream=None):
    args, keep = _accept_args(parent, logits, draft, result, workspace, stream)
    return PreparedCall(lib().tsw_accept_greedy, args, "tsw_accept_greedy", keep)


def _compact_args(k, v, n_prefix, T, result, stream):
    if k.shape != v.shape or k.dtype != v.dtype or not (k.is_cuda and v.is_cuda):
        raise ValueError("k and v must be GPU tensors of one shape and dtype")
    if k.dim() == 3:
        n_layers, layer_stride = 1, 0
        Hkv, rows, d = k.shape
        hs = k.stride(0)
    elif k.dim() == 4:
        n_layers, Hkv, rows, d = k.shape
        layer_stride, hs = k.stride(0), k.stride(1)
        if v.stride(0) != layer_stride:
            raise ValueError("k and v must share strides")
    else:
        raise ValueError("k, v must be [Hkv, rows, d] or [layers, Hkv, rows, d]")
    if k.stride(-1) != 1 or k.stride(-2) != d or v.stride(-1) != 1 or v.stride(-2) != d \
            or v.stride(-3) != hs:
        raise ValueError("k and v rows must be contiguous with equal head strides")
    if rows < int(n_prefix) + int(T):
        raise ValueError("the caches need n_prefix + T rows")
    dt = DTYPE_F32 if k.dtype == torch.float32 else DTYPE_BF16
    st = ctypes.c_void_p(stream.cuda_stream if stream is not None
                         else torch.cuda.current_stream(k.device).cuda_stream)
    return (_dev_ptr(k), _dev_ptr(v), n_layers, layer_stride, Hkv, d, dt, hs, int(n_prefix), int(T),
            _dev_ptr(result), st)


def kv_compact(k, v, n_prefix, T, result):
    """Move the accepted path's K/V rows in place (see tsw_kv_compact)."""
    _check(lib().tsw_kv_compact(*_compact_args(k, v, n_prefix, T, result, None)), "tsw_kv_compact")


def prepare_compact(k, v, n_prefix, T, result, stream=None):
    return PreparedCall(lib().tsw_kv_compact, _compact_args(k, v, n_prefix, T, result, stream),
                        "tsw_kv_compact", (k, v, result))


# ------------------------------------------------------------ paged batch

def make_paged_desc(q, k_pages, block_table, scale=None):
    """Descriptor for q [B, T, Hq, d], a page pool [n_pages, Hkv, page_rows, d]
    and a block table [B, max_pages]."""
    B, T, Hq, d = q.shape
    _, Hkv, page_rows, d2 = k_pages.shape
    if d2 != d or block_table.shape[0] != B:
        raise ValueError("shape mismatch between q, pages and block table")
    return PagedDesc(B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, page_rows=page_rows,
                     max_pages=block_table.shape[1],
                     dtype=DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F32,
                     scale=float(scale) if scale is not None else 1.0 / float(np.sqrt(d)), reserved=0)


def _paged_lengths(n_prefix):
    return np.ascontiguousarray(np.asarray(n_prefix, dtype=np.int64))


def paged_workspace_size(q, k_pages, block_table, n_prefix, scale=None):
    desc = make_paged_desc(q, k_pages, block_table, scale)
    npf = _paged_lengths(n_prefix)
    n = ctypes.c_size_t(0)
    _check(lib().tsw_paged_workspace_size(ctypes.byref(desc), _np_ptr(npf), ctypes.byref(n)),
           "tsw_paged_workspace_size")
    return n.value


def _paged_args(q, k_pages, v_pages, block_table, n_prefix, parent, o, lse, workspace, scale, stream):
    for t in (q, k_pages, v_pages):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q and the page pools must be contiguous GPU tensors")
    if block_table.dtype != torch.int32 or not block_table.is_cuda or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 GPU tensor")
    desc = make_paged_desc(q, k_pages, block_table, scale)
    npf = _paged_lengths(n_prefix)
    p = _parent_arr(parent)
    st = ctypes.c_void_p(stream.cuda_stream if stream is not None
                         else torch.cuda.current_stream(q.device).cuda_stream)
    args = (ctypes.byref(desc), _dev_ptr(q), _dev_ptr(k_pages), _dev_ptr(v_pages), _dev_ptr(block_table),
            _np_ptr(npf), _np_ptr(p), _dev_ptr(o), _dev_ptr(lse), _dev_ptr(workspace), workspace.numel(), st)
    return args, (desc, npf, p)


def tree_attn_verify_paged(q, k_pages, v_pages, block_table, n_prefix, parent, scale=None, out=None,
                           workspace=None):
    """Paged batch verification; returns (o [B, T, Hq, d], lse [B, T, Hq])."""
    B, T, Hq, d = q.shape
    o, lse = out if out is not None else (
        torch.empty((B, T, Hq, d), dtype=torch.float32, device=q.device),
        torch.empty((B, T, Hq), dtype=torch.float32, device=q.device))
    if workspace is None:
        workspace = torch.empty(max(paged_workspace_size(q, k_pages, block_table, n_prefix, scale), 256),
                                dtype=torch.uint8, device=q.device)
    args, _keep = _paged_args(q, k_pages, v_pages, block_table, n_prefix, parent, o, lse, workspace, scale,
                              None)
    _check(lib().tsw_tree_attn_verify_paged(*args), "tsw_tree_attn_verify_paged")
    return o, lse


def prepare_verify_paged(q, k_pages, v_pages, block_table, n_prefix, parent, o, lse, workspace, scale=None,
                         stream=None):
    args, keep = _paged_args(q, k_pages, v_pages, block_table, n_prefix, parent, o, lse, workspace, scale,
                             stream)
    return PreparedCall(lib().tsw_tree_attn_verify_paged, args, "tsw_tree_attn_verify_paged", keep)


def paged_partial_workspace_size(q, k_pages, block_table, n_prefix, n_idx, scale=None):
    desc = make_paged_desc(q, k_pages, block_table, scale)
    npf, nif = _paged_lengths(n_prefix), _paged_lengths(n_idx)
    n = ctypes.c_size_t(0)
    _check(lib().tsw_paged_partial_workspace_size(ctypes.byref(desc), _np_ptr(npf), _np_ptr(nif),
                                                  ctypes.byref(n)), "tsw_paged_partial_workspace_size")
    return n.value


def _paged_partial_args(q, k_pages, v_pages, block_table, n_prefix, parent, idx, n_idx, o, lse, workspace, scale,
                        stream):
    """idx: int32 GPU tensor [B, idx_stride] (sequence b's list in row b), or
    None when every n_idx[b] is 0."""
    args, keep = _paged_args(q, k_pages, v_pages, block_table, n_prefix, parent, o, lse, workspace, scale, stream)
    if idx is not None:
        if idx.dtype != torch.int32 or not idx.is_cuda or not idx.is_contiguous() or idx.dim() != 2:
            raise ValueError("idx must be a contiguous 2-D int32 GPU tensor [B, idx_stride]")
        stride = idx.shape[1]
    else:
        stride = 0
    nif = _paged_lengths(n_idx)
    # (desc, q, k, v, table, n_prefix, parent, idx, idx_stride, n_idx, o, lse, ws, ws_bytes, stream)
    args = args[:7] + (_dev_ptr(idx) if idx is not None else None, stride, _np_ptr(nif)) + args[7:]
    return args, keep + (nif, idx)


def tree_attn_partial_paged(q, k_pages, v_pages, block_table, n_prefix, parent, idx, n_idx, scale=None, out=None,
                            workspace=None):
    """Paged batch draft pass over per-sequence index lists; returns
    (o [B, T, Hq, d], lse [B, T, Hq])."""
    B, T, Hq, d = q.shape
    o, lse = out if out is not None else (
        torch.empty((B, T, Hq, d), dtype=torch.float32, device=q.device),
        torch.empty((B, T, Hq), dtype=torch.float32, device=q.device))
    if workspace is None:
        workspace = torch.empty(max(paged_partial_workspace_size(q, k_pages, block_table, n_prefix, n_idx, scale),
                                    256), dtype=torch.uint8, device=q.device)
    args, _keep = _paged_partial_args(q, k_pages, v_pages, block_table, n_prefix, parent, idx, n_idx, o, lse,
                                      workspace, scale, None)
    _check(lib().tsw_tree_attn_partial_paged(*args), "tsw_tree_attn_partial_paged")
    return o, lse


def prepare_partial_paged(q, k_pages, v_pages, block_table, n_prefix, parent, idx, n_idx, o, lse, workspace,
                          scale=None, stream=None):
    args, keep = _paged_partial_args(q, k_pages, v_pages, block_table, n_prefix, parent, idx, n_idx, o, lse,
                                     workspace, scale, stream)
    return PreparedCall(lib().tsw_tree_attn_partial_paged, args, "tsw_tree_attn_partial_paged", keep)


# ------------------------------------------------------------ partial-cache selection

def select_workspace_size(n_prefix):
    n = ctypes.c_size_t(0)
    _check(lib().tsw_select_workspace_size(int(n_prefix), ctypes.byref(n)), "tsw_select_workspace_size")
    return n.value


def _select_args(q, k, lse, n_prefix, n_keep, n_idx, idx, importance, workspace, scale, stream):
    _check_tensors(q, k, k)
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 GPU tensor")
    desc = make_desc(q, k, n_prefix, scale)
    n_out = min(int(n_idx), int(n_prefix))
    if idx is None:
        idx = torch.empty(max(n_out, 1), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = torch.empty(select_workspace_size(n_prefix), dtype=torch.uint8, device=q.device)
    st = ctypes.c_void_p(stream.cuda_stream if stream is not None
                         else torch.cuda.current_stream(q.device).cuda_stream)
    args = (ctypes.byref(desc), _dev_ptr(q), _dev_ptr(k), _dev_ptr(lse), int(n_keep), int(n_idx), _dev_ptr(idx),
            _dev_ptr(importance), _dev_ptr(workspace), workspace.numel() if workspace is not None else 0, st)
    return args, (desc, idx, importance, workspace), n_out


def select_partial(q, k, lse, n_prefix, n_keep, n_idx, scale=None, importance=None, idx=None, workspace=None):
    """Index list for the next draft pass: (idx int32 [min(n_idx, n_prefix)], importance or None)."""
    args, keep, n_out = _select_args(q, k, lse, n_prefix, n_keep, n_idx, idx, importance, workspace, scale, None)
    _check(lib().tsw_select_partial(*args), "tsw_select_partial")
    return keep[1][:n_out], importance


def prepare_select(q, k, lse, n_prefix, n_keep, n_idx, idx, importance=None, workspace=None, scale=None,
                   stream=None):
    args, keep, _ = _select_args(q, k, lse, n_prefix, n_keep, n_idx, idx, importance, workspace, scale, stream)
    return PreparedCall(lib().tsw_select_partial, args, "tsw_select_partial", keep)


def verify_select_workspace_size(q, k, n_prefix, scale=None, impl="auto"):
    desc = make_desc(q, k, n_prefix, scale, impl)
    n = ctypes.c_size_t(0)
    _check(lib().tsw_verify_select_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "tsw_verify_select_workspace_size")
    return n.value


def _verify_select_args(q, k, v, parent, n_prefix, n_keep, n_idx, o, lse, idx, importance, workspace, scale,
                        impl, stream):
    _check_tensors(q, k, v)
    T, Hq, d = q.shape
    desc = make_desc(q, k, n_prefix, scale, impl)
    if o is None:
        o = torch.empty((T, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    n_out = min(int(n_idx), int(n_prefix))
    if idx is None:
        idx = torch.empty(max(n_out, 1), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = torch.empty(verify_select_workspace_size(q, k, n_prefix, scale, impl), dtype=torch.uint8,
                                device=q.device)
    p = _parent_arr(parent)
    st = ctypes.c_void_p(stream.cuda_stream if stream is not None
                         else torch.cuda.current_stream(q.device).cuda_stream)
    args = (ctypes.byref(desc), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _np_ptr(p), _dev_ptr(o), _dev_ptr(lse),
            int(n_keep), int(n_idx), _dev_ptr(idx), _dev_ptr(importance), _dev_ptr(workspace), workspace.numel(),
            st)
    return args, (desc, p, o, lse, idx, importance, workspace), n_out


def tree_attn_verify_select(q, k, v, parent, n_prefix, n_keep, n_idx, scale=None, impl="auto", out=None,
                            idx=None, importance=None, workspace=None):
    """Verification plus the next draft pass's index list from the same pass:
    (o, lse, idx [min(n_idx, n_prefix)], importance or None)."""
    o, lse = out if out is not None else (None, None)
    args, keep, n_out = _verify_select_args(q, k, v, parent, n_prefix, n_keep, n_idx, o, lse, idx, importance,
                                            workspace, scale, impl, None)
    _check(lib().tsw_tree_attn_verify_select(*args), "tsw_tree_attn_verify_select")
    return keep[2], keep[3], keep[4][:n_out], importance


def prepare_verify_select(q, k, v, parent, n_prefix, n_keep, n_idx, o, lse, idx, importance=None,
                          workspace=None, scale=None, impl="auto", stream=None):
    args, keep, _ = _verify_select_args(q, k, v, parent, n_prefix, n_keep, n_idx, o, lse, idx, importance,
                                        workspace, scale, impl, stream)
    return PreparedCall(lib().tsw_tree_attn_verify_select, args, "tsw_tree_attn_verify_select", keep)


def read_stream(q, k, v, n_prefix, sink, scale=None, stream=None):
    """Read-stream ceiling for the cache a verify call with these shapes reads
    (a measurement aid): streams K and V rows 0 .. n_prefix + T - 1 through
    the LDS-DMA ring.  sink: a device tensor of at least 64 bytes."""
    _check_tensors(q, k, v)
    desc = make_desc(q, k, n_prefix, scale)
    st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(q)
    _check(lib().tsw_read_stream(ctypes.byref(desc), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sink), st),
           "tsw_read_stream")


def prepare_read_stream(q, k, v, n_prefix, sink, scale=None, stream=None):
    _check_tensors(q, k, v)
    desc = make_desc(q, k, n_prefix, scale)
    st = ctypes.c_void_p((stream or torch.cuda.current_stream(q.device)).cuda_stream)
    args = (ctypes.byref(desc), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sink), st)
    return PreparedCall(lib().tsw_read_stream, args, "tsw_read_stream", keep=(desc,))


def prepare_launch_floor(q, k, n_prefix, n_idx=None, scale=None, impl="auto", stream=None):
    """Bound tsw_launch_floor call (a measurement aid): an empty kernel on
    the split grid of the verify (n_idx None) or partial call."""
    desc = make_desc(q, k, n_prefix, scale, impl)
    st = ctypes.c_void_p((stream or torch.cuda.current_stream(q.device)).cuda_stream)
    args = (ctypes.byref(desc), -1 if n_idx is None else int(n_idx), None, st)
    return PreparedCall(lib().tsw_launch_floor, args, "tsw_launch_floor", keep=(desc,))


def noalloc_scratch_bytes():
    """Bytes of the library's own partials array used by tree_attn_verify_noalloc."""
    return int(lib().tsw_noalloc_scratch_bytes())


def tree_attn_verify_noalloc(q, k, v, parent, n_prefix, o, lse, scale=None, impl="auto", stream=None):
    """tree_attn_verify without a workspace: the library's own device array
    holds the split partials.  o [T, Hq, d] and lse [T, Hq] float32 are
    written in place (the call allocates nothing)."""
    _check_tensors(q, k, v)
    desc = make_desc(q, k, n_prefix, scale, impl)
    p = _parent_arr(parent)
    st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(q)
    _check(lib().tsw_tree_attn_verify_noalloc(ctypes.byref(desc), _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _np_ptr(p),
                                              _dev_ptr(o), _dev_ptr(lse), st), "tsw_tree_attn_verify_noalloc")
    return o, lse
