"""The C-ABI library without a GPU: it loads, exports every function the
public header declares, builds tree masks bit-exactly, and rejects bad
arguments with the documented status codes before touching HIP."""
import ctypes

import numpy as np
import pytest

import oracle
import tree_verification_attention_tsw_amd as tsw
from tree_verification_attention_tsw_amd import workloads as wl
from tree_verification_attention_tsw_amd import build as tsw_build

TSW_OK, EINVAL, EBADTREE, EBADINDEX, EUNSUP, ENOSPACE, EHIP = 0, -1, -2, -3, -4, -5, -6
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: argument checks run first


@pytest.fixture(scope="module")
def L():
    if tsw_build.stale():
        tsw_build.build()
    return tsw.lib()


def test_exports_every_declared_symbol(L):
    names = tsw.declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in (TSW_OK, EINVAL, EBADTREE, EBADINDEX, EUNSUP, ENOSPACE, EHIP):
        assert tsw.status_str(s)
    assert tsw.status_str(-99) == "unknown status"


@pytest.mark.parametrize("T", [1, 2, 13, 40, 63, 64])
def test_mask_ternary_matches_oracle(L, T):
    parent = wl.kary_tree_parent(T, 3)
    m1, d1 = tsw.tree_mask(parent)
    m2, d2 = oracle.mask_build(parent)
    assert np.array_equal(m1, m2) and np.array_equal(d1, d2)


def test_mask_random_and_chain_match_oracle(L):
    for seed in range(50):
        T = 1 + (seed * 7) % 64
        for parent in (wl.random_tree_parent(T, seed), wl.chain_parent(T)):
            m1, d1 = tsw.tree_mask(parent)
            m2, d2 = oracle.mask_build(parent)
            assert np.array_equal(m1, m2) and np.array_equal(d1, d2)


def test_mask_closed_form_totals(L):
    for n, total in ((13, 34), (40, 142)):
        m, _ = tsw.tree_mask(wl.kary_tree_parent(n, 3))
        assert sum(bin(int(x)).count("1") for x in m) == total


@pytest.mark.parametrize("parent,code", [
    ([0], EBADTREE), ([-1, 1], EBADTREE), ([-1, 0, 3], EBADTREE), ([-1, -1], EBADTREE),
    ([-1, 0, 0, 2, 5], EBADTREE)])
def test_mask_rejects_bad_trees(L, parent, code):
    p = np.array(parent, dtype=np.int32)
    mask = np.zeros(64, dtype=np.uint64)
    assert L.tsw_tree_mask_build(p.ctypes.data_as(ctypes.c_void_p), len(parent),
                                 mask.ctypes.data_as(ctypes.c_void_p), None) == code


def test_mask_rejects_sizes(L):
    p = np.full(65, 0, dtype=np.int32)
    p[0] = -1
    mask = np.zeros(65, dtype=np.uint64)
    args = (p.ctypes.data_as(ctypes.c_void_p), None, mask.ctypes.data_as(ctypes.c_void_p), None)
    assert L.tsw_tree_mask_build(args[0], 0, args[2], None) == EINVAL
    assert L.tsw_tree_mask_build(args[0], 65, args[2], None) == EINVAL
    assert L.tsw_tree_mask_build(None, 3, args[2], None) == EINVAL
    assert L.tsw_tree_mask_build(args[0], 3, None, None) == EINVAL


def _desc(**kw):
    d = tsw.AttnDesc()
    d.T, d.Hq, d.Hkv, d.d = 13, 4, 2, 128
    d.n_prefix = 100
    d.kv_head_stride = (100 + 13) * 128
    d.dtype = tsw.DTYPE_BF16
    d.impl = 0
    d.scale = 0.088
    d.reserved = 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


PARENT = np.ascontiguousarray(wl.kary_tree_parent(13, 3))


def _verify(L, desc, parent=PARENT, q=FAKE, o=FAKE, ws=FAKE):
    return L.tsw_tree_attn_verify(ctypes.byref(desc), q, FAKE, FAKE,
                                  parent.ctypes.data_as(ctypes.c_void_p), o, FAKE, ws, 1 << 30, None)


@pytest.mark.parametrize("field,value,code", [
    ("T", 0, EINVAL), ("T", 65, EINVAL), ("Hq", 3, EINVAL), ("Hkv", 0, EINVAL),
    ("d", 96, EUNSUP), ("dtype", 7, EUNSUP), ("impl", 9, EUNSUP), ("reserved", 1, EINVAL),
    ("scale", 0.0, EINVAL), ("scale", -1.0, EINVAL), ("scale", float("nan"), EINVAL),
    ("scale", float("inf"), EINVAL), ("n_prefix", -1, EINVAL),
    ("kv_head_stride", (100 + 13) * 128 - 1, EINVAL)])
def test_desc_errors(L, field, value, code):
    assert _verify(L, _desc(**{field: value})) == code


def test_mfma_forced_on_unsupported_shape(L):
    # float32 inputs have no matrix-core kernel here
    assert _verify(L, _desc(impl=2, dtype=tsw.DTYPE_F32)) == EUNSUP
    # more than 24 query blocks of 16 rows (384 rows) per kv head
    assert _verify(L, _desc(impl=2, T=64, Hq=56, Hkv=8, d=128,
                            kv_head_stride=(100 + 64) * 128),
                   parent=np.ascontiguousarray(wl.kary_tree_parent(64, 3))) == EUNSUP



def test_query_rows_per_kv_head_limit(L):
    # at most 4096 query rows (T * Hq / Hkv) share one kv head
    par = np.ascontiguousarray(wl.kary_tree_parent(64, 3))
    assert _verify(L, _desc(T=64, Hq=128, Hkv=1, kv_head_stride=(100 + 64) * 128), parent=par) == EUNSUP


def test_null_pointers_and_bad_tree(L):
    d = _desc()
    assert _verify(L, d, q=None) == EINVAL
    assert _verify(L, d, o=None) == EINVAL
    bad = np.array([-1, 0, 5] + [0] * 10, dtype=np.int32)
    assert _verify(L, d, parent=bad) == EBADTREE


def test_partial_index_errors(L):
    d = _desc()
    p = PARENT.ctypes.data_as(ctypes.c_void_p)
    call = lambda n: L.tsw_tree_attn_partial(ctypes.byref(d), FAKE, FAKE, FAKE, p, FAKE, n,
                                             FAKE, FAKE, FAKE, 1 << 30, None)
    assert call(-1) == EBADINDEX
    assert call(101) == EBADINDEX


def test_split_and_merge_argument_errors(L):
    d = _desc()
    p = PARENT.ctypes.data_as(ctypes.c_void_p)
    assert L.tsw_tree_attn_split(ctypes.byref(d), FAKE, FAKE, FAKE, p, None, 0, 0, FAKE, FAKE,
                                 None) == EINVAL
    assert L.tsw_tree_attn_split(ctypes.byref(d), FAKE, FAKE, FAKE, p, FAKE, 101, 4, FAKE,
                                 FAKE, None) == EBADINDEX
    assert L.tsw_lse_merge(0, 10, 128, FAKE, FAKE, FAKE, FAKE, None) == EINVAL
    assert L.tsw_lse_merge(2, -1, 128, FAKE, FAKE, FAKE, FAKE, None) == EINVAL
    assert L.tsw_lse_merge(2, 10, 128, None, FAKE, FAKE, FAKE, None) == EINVAL
    # zero rows is a no-op that needs no device
    assert L.tsw_lse_merge(2, 0, 128, None, None, None, None, None) == TSW_OK


def test_contiguous_part_size_limit(L):
    # a matrix-core part of a contiguous cache reads its rows through 32-bit
    # buffer offsets: more than 2^23 keys in one part is refused on the host
    npre = (1 << 23) + 100
    d = _desc(n_prefix=npre, kv_head_stride=(npre + 13) * 128, impl=tsw.IMPL["mfma"])
    p = PARENT.ctypes.data_as(ctypes.c_void_p)
    assert L.tsw_tree_attn_split(ctypes.byref(d), FAKE, FAKE, FAKE, p, None, 0, 1, FAKE, FAKE,
                                 None) == EUNSUP


def test_null_workspace(L):
    assert _verify(L, _desc(), ws=None) == EINVAL


def test_accept_argument_errors(L):
    p = PARENT.ctypes.data_as(ctypes.c_void_p)
    call = lambda **kw: L.tsw_accept_greedy(
        kw.get("parent", p), kw.get("T", 13), kw.get("logits", FAKE), kw.get("vocab", 1000),
        kw.get("dtype", 0), kw.get("draft", FAKE), kw.get("result", FAKE), kw.get("ws", FAKE),
        1 << 20, None)
    assert call(T=0) == EINVAL
    assert call(T=65) == EINVAL
    assert call(vocab=0) == EINVAL
    assert call(vocab=1 << 31) == EINVAL
    assert call(parent=None) == EINVAL
    bad = np.array([-1, 0, 5] + [0] * 10, dtype=np.int32)
    assert call(parent=bad.ctypes.data_as(ctypes.c_void_p)) == EBADTREE
    assert call(dtype=5) == EUNSUP
    assert call(logits=None) == EINVAL
    assert call(draft=None) == EINVAL
    assert call(result=None) == EINVAL
    assert call(ws=None) == EINVAL
    assert call(ws=ctypes.c_void_p(0x10004)) == EINVAL      # not 8-byte aligned
    n = ctypes.c_size_t(0)
    assert L.tsw_accept_workspace_size(0, 100, ctypes.byref(n)) == EINVAL
    assert L.tsw_accept_workspace_size(13, 0, ctypes.byref(n)) == EINVAL
    assert L.tsw_accept_workspace_size(13, 100, None) == EINVAL


def test_compact_argument_errors(L):
    def call(**kw):
        a = dict(k=FAKE, v=FAKE, layers=2, layer_stride=8 * 200 * 128, Hkv=8, d=128, dtype=1,
                 hs=200 * 128, n_prefix=100, T=40, result=FAKE)
        a.update(kw)
        return L.tsw_kv_compact(a["k"], a["v"], a["layers"], a["layer_stride"], a["Hkv"], a["d"],
                                a["dtype"], a["hs"], a["n_prefix"], a["T"], a["result"], None)
    assert call(k=None) == EINVAL
    assert call(result=None) == EINVAL
    assert call(T=0) == EINVAL
    assert call(T=65) == EINVAL
    assert call(layers=0) == EINVAL
    assert call(Hkv=0) == EINVAL
    assert call(d=96) == EUNSUP
    assert call(dtype=3) == EUNSUP
    assert call(n_prefix=-1) == EINVAL
    assert call(hs=100 * 128) == EINVAL                       # rows < n_prefix + T
    assert call(layer_stride=8 * 200 * 128 - 1) == EINVAL     # layers overlap
    assert call(k=ctypes.c_void_p(0x10008)) == EINVAL         # not 16-byte aligned


def _pdesc(**kw):
    d = tsw.PagedDesc(B=3, T=13, Hq=8, Hkv=2, d=128, page_rows=16, max_pages=20, dtype=tsw.DTYPE_BF16,
                      scale=0.088, reserved=0)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _paged(L, desc, npf=(100, 200, 0), q=FAKE, table=FAKE, ws=FAKE):
    n = np.ascontiguousarray(np.asarray(npf, dtype=np.int64))
    return L.tsw_tree_attn_verify_paged(ctypes.byref(desc), q, FAKE, FAKE, table,
                                        n.ctypes.data_as(ctypes.c_void_p),
                                        PARENT.ctypes.data_as(ctypes.c_void_p), FAKE, FAKE, ws, 1 << 30,
                                        None)


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, EINVAL), ("B", 65, EINVAL), ("T", 0, EINVAL), ("Hq", 3, EINVAL), ("d", 64, EUNSUP),
    ("dtype", 0, EUNSUP), ("page_rows", 24, EINVAL), ("page_rows", 8, EINVAL), ("page_rows", 8192, EINVAL),
    ("max_pages", 13, EINVAL), ("scale", 0.0, EINVAL), ("reserved", 1, EINVAL), ("Hq", 64, EUNSUP)])
def test_paged_desc_errors(L, field, value, code):
    npf = (100, 200, 0)
    if field == "Hq" and value == 64:       # 13 * 32 = 416 rows per kv head: no matrix shape
        assert _paged(L, _pdesc(Hq=64, Hkv=2), npf) == code
        return
    assert _paged(L, _pdesc(**{field: value}), npf) == code


def test_paged_argument_errors(L):
    assert _paged(L, _pdesc(), npf=(100, -1, 0)) == EINVAL
    assert _paged(L, _pdesc(), q=None) == EINVAL
    assert _paged(L, _pdesc(), table=None) == EINVAL
    assert _paged(L, _pdesc(), q=ctypes.c_void_p(0x10008)) == EINVAL
    n = ctypes.c_size_t(0)
    assert L.tsw_paged_workspace_size(ctypes.byref(_pdesc(B=0)), None, ctypes.byref(n)) == EINVAL


def _ppaged(L, desc, npf=(100, 200, 0), nif=(50, 200, 0), idx=FAKE, stride=256, q=FAKE, ws=FAKE):
    n = np.ascontiguousarray(np.asarray(npf, dtype=np.int64))
    ni = np.ascontiguousarray(np.asarray(nif, dtype=np.int64)) if nif is not None else None
    return L.tsw_tree_attn_partial_paged(ctypes.byref(desc), q, FAKE, FAKE, FAKE,
                                         n.ctypes.data_as(ctypes.c_void_p),
                                         PARENT.ctypes.data_as(ctypes.c_void_p), idx, stride,
                                         ni.ctypes.data_as(ctypes.c_void_p) if ni is not None else None,
                                         FAKE, FAKE, ws, 1 << 30, None)


def test_paged_partial_argument_errors(L):
    """The paged draft pass rejects bad index-list lengths and pointers
    before any HIP call (as the verify call does its shape errors)."""
    assert _ppaged(L, _pdesc(), nif=None) == EINVAL                      # no n_idx
    assert _ppaged(L, _pdesc(), nif=(50, 201, 0)) == EBADINDEX           # n_idx > n_prefix
    assert _ppaged(L, _pdesc(), nif=(-1, 0, 0)) == EBADINDEX
    assert _ppaged(L, _pdesc(), stride=199) == EINVAL                    # a list longer than its row
    assert _ppaged(L, _pdesc(), idx=None) == EINVAL                      # lists but no idx
    assert _ppaged(L, _pdesc(), q=None) == EINVAL
    assert _ppaged(L, _pdesc(B=0)) == EINVAL
    assert _ppaged(L, _pdesc(d=64)) == EUNSUP
    assert _ppaged(L, _pdesc(), npf=(100, -1, 0)) == EINVAL
    n = ctypes.c_size_t(0)
    npf = np.asarray([100, 200, 0], dtype=np.int64)
    bad = np.asarray([0, 300, 0], dtype=np.int64)
    assert L.tsw_paged_partial_workspace_size(ctypes.byref(_pdesc()), npf.ctypes.data_as(ctypes.c_void_p),
                                              bad.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n)) == EBADINDEX
    assert L.tsw_paged_partial_workspace_size(ctypes.byref(_pdesc()), npf.ctypes.data_as(ctypes.c_void_p),
                                              None, ctypes.byref(n)) == EINVAL


def test_select_argument_errors(L):
    def call(desc=None, q=FAKE, k=FAKE, lse=FAKE, n_keep=128, n_idx=4096, idx=FAKE, imp=None, ws=FAKE):
        d = desc if desc is not None else _desc()
        return L.tsw_select_partial(ctypes.byref(d), q, k, lse, n_keep, n_idx, idx, imp, ws, 1 << 30, None)
    assert call(n_keep=-1) == EBADINDEX
    assert call(n_idx=-1) == EBADINDEX
    assert call(q=None) == EINVAL
    assert call(lse=None) == EINVAL
    assert call(idx=None) == EINVAL
    assert call(ws=None) == EINVAL                        # no workspace
    assert call(k=ctypes.c_void_p(0x10008)) == EINVAL     # not 16-byte aligned
    assert call(desc=_desc(Hq=128, Hkv=8)) == EUNSUP     # more query heads than the kernel holds
    assert call(desc=_desc(d=96)) == EUNSUP
    n = ctypes.c_size_t(0)
    assert L.tsw_select_workspace_size(-1, ctypes.byref(n)) == EINVAL
    assert L.tsw_select_workspace_size(1000, ctypes.byref(n)) == TSW_OK and n.value >= 4000


def test_verify_select_argument_errors(L):
    def call(desc=None, q=FAKE, k=FAKE, v=FAKE, parent=PARENT, o=FAKE, lse=FAKE, n_keep=128, n_idx=4096,
             idx=FAKE, ws=FAKE):
        d = desc if desc is not None else _desc()
        p = parent.ctypes.data_as(ctypes.c_void_p) if parent is not None else None
        return L.tsw_tree_attn_verify_select(ctypes.byref(d), q, k, v, p, o, lse, n_keep, n_idx, idx, None, ws,
                                             1 << 30, None)
    assert call(n_keep=-1) == EBADINDEX
    assert call(n_idx=-1) == EBADINDEX
    assert call(q=None) == EINVAL
    assert call(v=None) == EINVAL
    assert call(parent=None) == EINVAL
    assert call(o=None) == EINVAL
    assert call(idx=None) == EINVAL
    assert call(ws=None) == EINVAL
    assert call(ws=ctypes.c_void_p(0x10080)) == EINVAL    # workspace not 256-byte aligned
    assert call(k=ctypes.c_void_p(0x10008)) == EINVAL
    bad = PARENT.copy()
    bad[5] = 7                                            # a parent after its child
    assert call(parent=bad) == EBADTREE
    assert call(desc=_desc(Hq=128, Hkv=8)) == EUNSUP
    assert call(desc=_desc(d=96)) == EUNSUP
    assert L.tsw_verify_select_workspace_size(ctypes.byref(_desc()), None) == EINVAL


def test_penalty_argument_errors(L):
    p = PARENT.ctypes.data_as(ctypes.c_void_p)

    def call(parent=p, T=13, logits=FAKE, vocab=1000, dtype=0, draft=FAKE, recent=FAKE, n_recent=10, window=64,
             theta=1.2):
        return L.tsw_context_penalty(parent, T, logits, vocab, dtype, draft, recent, n_recent, window, theta, None)
    assert call(window=-1) == EINVAL
    assert call(window=8193) == EINVAL
    assert call(theta=0.5) == EINVAL                      # would raise repeated tokens
    assert call(theta=float("nan")) == EINVAL
    assert call(theta=float("inf")) == EINVAL
    assert call(n_recent=-1) == EINVAL
    assert call(logits=None) == EINVAL
    assert call(draft=None) == EINVAL
    assert call(recent=None) == EINVAL
    assert call(dtype=5) == EUNSUP
    assert call(T=0) == EINVAL
    bad = PARENT.copy()
    bad[5] = 7
    assert call(parent=bad.ctypes.data_as(ctypes.c_void_p)) == EBADTREE
    assert call(window=0) == TSW_OK                       # nothing to do: no launch, no device needed
    assert call(theta=1.0) == TSW_OK


def test_accept_penalized_argument_errors(L):
    p = PARENT.ctypes.data_as(ctypes.c_void_p)

    def call(window=64, theta=1.2, recent=FAKE, n_recent=10, ws=FAKE):
        return L.tsw_accept_greedy_penalized(p, 13, FAKE, 1000, 0, FAKE, recent, n_recent, window, theta, FAKE, ws,
                                             1 << 20, None)
    assert call(window=-1) == EINVAL
    assert call(window=8193) == EINVAL
    assert call(theta=0.9) == EINVAL
    assert call(theta=float("nan")) == EINVAL
    assert call(recent=None) == EINVAL
    assert call(n_recent=-2) == EINVAL
    assert call(ws=None) == EINVAL


def test_read_stream_argument_errors(L):
    d = _desc()
    assert L.tsw_read_stream(ctypes.byref(d), None, FAKE, FAKE, None) == EINVAL
    assert L.tsw_read_stream(ctypes.byref(d), FAKE, FAKE, None, None) == EINVAL
    d32 = _desc(dtype=tsw.DTYPE_F32)
    assert L.tsw_read_stream(ctypes.byref(d32), FAKE, FAKE, FAKE, None) == EUNSUP
    d64 = _desc(d=64, kv_head_stride=(100 + 13) * 64)
    assert L.tsw_read_stream(ctypes.byref(d64), FAKE, FAKE, FAKE, None) == EUNSUP
    odd = ctypes.c_void_p(0x10008)
    assert L.tsw_read_stream(ctypes.byref(d), odd, FAKE, FAKE, None) == EINVAL



def test_launch_floor_argument_errors(L):
    """The launch-floor aid checks its descriptor before any HIP call."""
    assert L.tsw_launch_floor(ctypes.byref(_desc(T=0)), -1, None, None) == EINVAL
    assert L.tsw_launch_floor(ctypes.byref(_desc(Hq=3)), -1, None, None) == EINVAL
    assert L.tsw_launch_floor(ctypes.byref(_desc()), 101, None, None) == EBADINDEX     # n_idx > n_prefix
