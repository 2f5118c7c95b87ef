"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
identical seeded inputs.  Tolerances: max-abs 1e-5 on O and LSE for float32
inputs, 4e-3 for bfloat16 inputs with float32 accumulation; tree masks are
compared bit-exactly.  Every workload, the 100K-token ones included, is
compared on every (node, head) row."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_tsw_amd as tsw
from tree_verification_attention_tsw_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 4e-3}
NTHREADS = min(16, len(os.sched_getaffinity(0)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsw.lib()
    return torch.device("cuda:0")


def gen(shape, seed, dtype, device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def check(o, lse, o_ref, lse_ref, tol, what):
    o = o.detach().cpu().double().numpy()
    lse = lse.detach().cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what + ": non-finite output"
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse - lse_ref)))
    say("%s: max|dO| %.3g max|dLSE| %.3g" % (what, eo, el))
    assert eo <= tol and el <= tol, (what, eo, el)


def run_case(T, Hq, Hkv, d, n_prefix, dtype, parent, idx=None, impl="auto", seed=0,
             cap_extra=0, head_pad=0, rows=None, k_override=None):
    """Generate inputs, run the GPU path, compare with the oracle."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    cap = n_prefix + T + cap_extra
    q = gen((T, Hq, d), seed + 1, tdt)
    kb = gen((Hkv, cap + head_pad, d), seed + 2, tdt)
    vb = gen((Hkv, cap + head_pad, d), seed + 3, tdt)
    if k_override is not None:
        kb = k_override(kb)
    k, v = kb[:, :cap], vb[:, :cap]
    say("case T=%d Hq=%d Hkv=%d d=%d n_prefix=%d %s idx=%s impl=%s" % (
        T, Hq, Hkv, d, n_prefix, dtype, None if idx is None else len(idx), impl))
    if idx is None:
        o, lse = tsw.tree_attn_verify(q, k, v, parent, n_prefix, impl=impl)
    else:
        it = torch.from_numpy(np.asarray(idx, dtype=np.int32)).to(q.device)
        o, lse = tsw.tree_attn_partial(q, k, v, parent, it, n_prefix, impl=impl)
    torch.cuda.synchronize()
    qn, kn, vn = wl.oracle_view(q), wl.oracle_view(k.contiguous()), wl.oracle_view(v.contiguous())
    o_ref, lse_ref = oracle.tree_attn(qn, kn, vn, parent, n_prefix, 1.0 / np.sqrt(d), idx=idx,
                                      rows=rows, nthreads=NTHREADS)
    if rows is not None:
        o_s = o.reshape(T * Hq, d)[torch.as_tensor(rows, device=o.device).long()]
        l_s = lse.reshape(T * Hq)[torch.as_tensor(rows, device=o.device).long()]
        check(o_s, l_s, o_ref, lse_ref, TOL[dtype], "sampled rows")
    else:
        check(o, lse, o_ref, lse_ref, TOL[dtype], "all rows")
    return q, k, v, o, lse


# ------------------------------------------------------------ the workloads

def test_workload_tiny_mha_f32():
    w = wl.WORKLOADS["tiny_mha_f32"]
    q, k, v = wl.make_qkv(w, device="cuda")
    for impl in ("auto", "valu"):
        o, lse = tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix, impl=impl)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v),
                                        w.parent(), w.n_prefix, w.scale(), nthreads=NTHREADS)
        check(o, lse, o_ref, l_ref, TOL["f32"], "tiny %s" % impl)


@pytest.mark.parametrize("impl", ["auto", "valu"])
def test_workload_gqa8b_8k(impl):
    w = wl.WORKLOADS["gqa8b_8k"]
    q, k, v = wl.make_qkv(w, device="cuda")
    o, lse = tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix, impl=impl)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v),
                                    w.parent(), w.n_prefix, w.scale(), nthreads=NTHREADS)
    check(o, lse, o_ref, l_ref, TOL["bf16"], "gqa8b_8k %s" % impl)


@pytest.mark.parametrize("name", ["gqa8b_100k", "mha7b_100k", "gqa14b_100k"])
def test_workload_100k_all_rows(name):
    """The 100K-token workloads at full size in the launch configuration the
    bench times: every (node, head) row of O and LSE against the oracle."""
    w = wl.WORKLOADS[name]
    q, k, v = wl.make_qkv(w, device="cuda")
    o, lse = tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix)
    torch.cuda.synchronize()
    say("%s: %d rows x %d keys against the oracle (%d threads)" % (name, w.n_nodes * w.Hq, w.n_prefix + w.n_nodes,
                                                                  NTHREADS))
    o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v),
                                    w.parent(), w.n_prefix, w.scale(), nthreads=NTHREADS)
    check(o, lse, o_ref, l_ref, TOL["bf16"], name)


def test_workload_partial32_layers():
    w = wl.WORKLOADS["partial32_gqa8b_100k"]
    for layer in (0, 13, 31):
        q, k, v = wl.make_qkv(w, layer=layer, device="cuda")
        idx = wl.make_index_set(w, layer)
        assert len(idx) == 4096 and list(idx[:128]) == list(range(128))
        assert np.all(np.diff(idx) > 0) and idx[-1] < w.n_prefix
        it = torch.from_numpy(idx).to(q.device)
        o, lse = tsw.tree_attn_partial(q, k, v, w.parent(), it, w.n_prefix)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v),
                                        w.parent(), w.n_prefix, w.scale(), idx=idx,
                                        nthreads=NTHREADS)
        check(o, lse, o_ref, l_ref, TOL["bf16"], "partial layer %d" % layer)
        del q, k, v
        torch.cuda.empty_cache()


# ------------------------------------------------------------ shapes / edges

# Query rows per kv head M = T * G select the matrix-core shape (blocks of 16
# rows: 1-2, 3-4, 5-8, 9-12, 13-16, 17-24); each shape is covered, with
# ragged M and with row groups that own one block fewer than the others.
# 13 blocks (M = 193..208) take the shared-block arrangement: (40, 5), (52, 4)
# (13 full blocks), (41, 5), (49, 4) with two kv heads.
MFMA_SHAPES = [
    (1, 1, 1), (13, 1, 1), (16, 2, 1), (4, 8, 8), (40, 1, 1), (13, 4, 1), (40, 2, 1),
    (23, 4, 1), (40, 3, 1), (33, 4, 1), (40, 4, 1), (47, 4, 1), (64, 3, 1), (40, 5, 1),
    (52, 4, 1), (41, 5, 1), (49, 4, 2),
    (64, 4, 1), (61, 4, 1), (53, 5, 1), (50, 7, 1), (64, 6, 2),
]


@pytest.mark.parametrize("T,G,Hkv", MFMA_SHAPES)
def test_mfma_shapes(T, G, Hkv):
    run_case(T, G * Hkv, Hkv, 128, 1000 + 37, "bf16", wl.random_tree_parent(T, T * G),
             impl="mfma", seed=T * 100 + G)


@pytest.mark.parametrize("n_prefix", [0, 1, 31, 32, 63, 64, 65, 127, 129, 255, 4097])
def test_ragged_prefix(n_prefix):
    run_case(40, 8, 2, 128, n_prefix, "bf16", wl.kary_tree_parent(40, 3), seed=n_prefix)


@pytest.mark.parametrize("T", [1, 2, 3, 17, 63, 64])
def test_tree_sizes(T):
    run_case(T, 4, 1, 128, 777, "bf16", wl.random_tree_parent(T, T), seed=7 * T)


def test_chain_tree():
    run_case(64, 4, 2, 128, 513, "bf16", wl.chain_parent(64), seed=11)


@pytest.mark.parametrize("dtype,d,impl", [("f32", 64, "auto"), ("f32", 128, "auto"),
                                          ("bf16", 64, "auto"), ("bf16", 128, "valu")])
def test_valu_kernel(dtype, d, impl):
    run_case(13, 8, 2, d, 700, dtype, wl.kary_tree_parent(13, 3), impl=impl, seed=d)
    run_case(40, 4, 4, d, 300, dtype, wl.random_tree_parent(40, 3), impl=impl, seed=d + 1)



@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_largest_query_group(dtype, d):
    """4096 query rows on one kv head (64 nodes x 64 query heads), the most a
    call takes: past the matrix-core shapes, on the vector-ALU kernel."""
    run_case(64, 64, 1, d, 700, dtype, wl.random_tree_parent(64, 31), seed=31 + d)


def test_head_stride_padding():
    run_case(13, 8, 4, 128, 2000, "bf16", wl.kary_tree_parent(13, 3), head_pad=333, seed=5)
    run_case(13, 4, 4, 64, 500, "f32", wl.kary_tree_parent(13, 3), head_pad=17, seed=6)


def test_rows_beyond_cache_are_not_read():
    # cache rows past n_prefix + T are poisoned; they must not leak
    run_case(13, 8, 2, 128, 900, "bf16", wl.kary_tree_parent(13, 3), cap_extra=100, seed=8,
             k_override=lambda kb: kb.index_fill_(1, torch.arange(900 + 13, kb.shape[1],
                                                                  device=kb.device), float("nan")))


@pytest.mark.parametrize("n_splits", [1, 3, 7])
def test_ragged_splits_do_not_read_past_their_rows(n_splits):
    """Every split of a contiguous cache reads its own rows (and the last
    split the tree rows) through a buffer over exactly those rows: the
    ragged end of each slice and the tree tile's padding read as zeros.
    K and V rows past n_prefix + T hold NaN and must not leak, whatever
    the split count (ragged slices in every split)."""
    T, Hq, Hkv, d, npre, extra = 13, 8, 2, 128, 1001, 200
    parent = wl.kary_tree_parent(T, 3)
    q = gen((T, Hq, d), 71, torch.bfloat16)
    k = gen((Hkv, npre + T + extra, d), 72, torch.bfloat16)
    v = gen((Hkv, npre + T + extra, d), 73, torch.bfloat16)
    k[:, npre + T:] = float("nan")
    v[:, npre + T:] = float("nan")
    po, pl = tsw.tree_attn_split(q, k, v, parent, npre, n_splits, impl="mfma")
    o, lse = tsw.lse_merge(po, pl)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k[:, :npre + T]),
                                    wl.oracle_view(v[:, :npre + T]), parent, npre, 1 / np.sqrt(d),
                                    nthreads=NTHREADS)
    check(o, lse, o_ref, l_ref, TOL["bf16"], "ragged splits %d" % n_splits)


@pytest.mark.parametrize("n_idx", [0, 1, 100, 4096, 5000])
def test_partial_sizes(n_idx):
    npre = 20000
    idx = wl.retained_index_set(npre, n_idx, min(128, n_idx), n_idx)
    run_case(4, 32, 8, 128, npre, "bf16", wl.chain_parent(4), idx=idx, seed=n_idx)
    run_case(13, 8, 2, 128, npre, "bf16", wl.kary_tree_parent(13, 3), idx=idx, seed=n_idx + 1)


@pytest.mark.parametrize("n_prefix", [1000, 2500])
def test_mfma_partial_forced(n_prefix):
    idx = wl.retained_index_set(n_prefix, n_prefix // 2, 128, 7)
    run_case(4, 32, 8, 128, n_prefix, "bf16", wl.chain_parent(4), idx=idx, impl="mfma", seed=71)
    run_case(40, 32, 8, 128, n_prefix, "bf16", wl.kary_tree_parent(40, 3), idx=idx, impl="mfma",
             seed=72)


def test_partial_valu_and_f32():
    npre = 3000
    idx = wl.retained_index_set(npre, 700, 64, 3)
    run_case(4, 8, 2, 128, npre, "bf16", wl.chain_parent(4), idx=idx, impl="valu", seed=21)
    run_case(13, 4, 4, 64, npre, "f32", wl.kary_tree_parent(13, 3), idx=idx, seed=22)


def test_partial_all_positions_equals_verify():
    T, Hq, Hkv, d, npre = 40, 32, 8, 128, 6000
    q = gen((T, Hq, d), 31, torch.bfloat16)
    k = gen((Hkv, npre + T, d), 32, torch.bfloat16)
    v = gen((Hkv, npre + T, d), 33, torch.bfloat16)
    parent = wl.kary_tree_parent(T, 3)
    o1, l1 = tsw.tree_attn_verify(q, k, v, parent, npre)
    idx = torch.arange(npre, dtype=torch.int32, device=q.device)
    o2, l2 = tsw.tree_attn_partial(q, k, v, parent, idx, npre)
    torch.cuda.synchronize()
    assert float((o1 - o2).abs().max()) <= 1e-5
    assert float((l1 - l2).abs().max()) <= 1e-5


def test_partial_unselected_rows_poisoned():
    """Rows outside the index list hold NaN: the result stays finite and
    matches the oracle (which never reads them)."""
    T, Hq, Hkv, d, npre = 4, 32, 8, 128, 30000
    idx = wl.retained_index_set(npre, 4096, 128, 99)
    sel = np.zeros(npre + T, dtype=bool)
    sel[idx] = True
    sel[npre:] = True
    bad = torch.from_numpy(np.nonzero(~sel)[0]).cuda()
    q = gen((T, Hq, d), 41, torch.bfloat16)
    k = gen((Hkv, npre + T, d), 42, torch.bfloat16).index_fill_(1, bad, float("nan"))
    v = gen((Hkv, npre + T, d), 43, torch.bfloat16).index_fill_(1, bad, float("nan"))
    parent = wl.chain_parent(T)
    o, lse = tsw.tree_attn_partial(q, k, v, parent, torch.from_numpy(idx).cuda(), npre)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v),
                                    parent, npre, 1 / np.sqrt(d), idx=idx, nthreads=NTHREADS)
    check(o, lse, o_ref, l_ref, TOL["bf16"], "poisoned partial")


def test_non_ancestor_tree_rows_do_not_leak():
    """Tree rows that are not ancestors get a huge key along the query
    direction: the output must not change."""
    T, Hq, Hkv, d, npre = 40, 8, 2, 128, 2000
    parent = wl.kary_tree_parent(T, 3)
    q = gen((T, Hq, d), 51, torch.bfloat16)
    k = gen((Hkv, npre + T, d), 52, torch.bfloat16)
    v = gen((Hkv, npre + T, d), 53, torch.bfloat16)
    o1, l1 = tsw.tree_attn_verify(q, k, v, parent, npre)
    mask, _ = tsw.tree_mask(parent)
    # node 39 (a leaf) sees only its own ancestors; poison every other tree row
    k2 = k.clone()
    anc = [j for j in range(T) if (int(mask[39]) >> j) & 1]
    others = [j for j in range(T) if j not in anc]
    k2[:, [npre + j for j in others], :] = 1e4
    o2, l2 = tsw.tree_attn_verify(q, k2, v, parent, npre)
    torch.cuda.synchronize()
    # Nodes 39 and 0 see none of the poisoned rows.  (The poisoned scores
    # send the last split's work-group through the exact two-pass path, which
    # rounds each p to bf16 relative to the row maximum instead of 2^0: the
    # unaffected rows may differ by that rounding, about 2^-9 of their
    # values, while a leaked 1e4 key would move them by the size of V.)
    for node in (39, 0):
        assert float((o1[node] - o2[node]).abs().max()) <= 1e-3
        assert float((l1[node] - l2[node]).abs().max()) <= 1e-3
    # nodes that do see poisoned rows change; all rows must match the oracle
    o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k2), wl.oracle_view(v),
                                    parent, npre, 1 / np.sqrt(d), nthreads=NTHREADS)
    check(o2, l2, o_ref, l_ref, TOL["bf16"], "poisoned tree rows")


@pytest.mark.parametrize("n_splits", [1, 2, 3, 7, 64, 300])
def test_split_then_merge(n_splits):
    """The two-phase API with caller-chosen split counts (including splits
    with no keys) merges to the oracle result."""
    T, Hq, Hkv, d, npre = 40, 32, 8, 128, 5000
    parent = wl.kary_tree_parent(T, 3)
    q = gen((T, Hq, d), 61, torch.bfloat16)
    k = gen((Hkv, npre + T, d), 62, torch.bfloat16)
    v = gen((Hkv, npre + T, d), 63, torch.bfloat16)
    po, pl = tsw.tree_attn_split(q, k, v, parent, npre, n_splits)
    o, lse = tsw.lse_merge(po, pl)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v),
                                    parent, npre, 1 / np.sqrt(d), nthreads=NTHREADS)
    check(o, lse, o_ref, l_ref, TOL["bf16"], "split %d" % n_splits)


# Loads are issued in groups of 128 keys (1, 2 or 4 tiles of 128, 64 or 32
# keys by shape); whole groups run unrolled and the rest of a split's tiles
# one at a time.  Two splits with an explicit count put 1-3 tiles after the
# last whole group (plus ragged ends and the tree's tiles in the last split)
# for every group size.
GROUP_CASES = [
    # (T, G, Hkv, tile keys, tiles per split)
    (13, 1, 1, 128, 3),     # 1 block: 128-key tiles, one tile per group
    (40, 2, 1, 64, 7),      # 5 blocks: 64-key tiles, two per group
    (40, 4, 1, 64, 5),      # 10 blocks
    (40, 5, 1, 32, 11),     # 13 blocks: 32-key tiles, four per group
    (53, 5, 1, 32, 9),      # 17 blocks
    (64, 4, 1, 32, 6),      # 16 blocks
]


@pytest.mark.parametrize("T,G,Hkv,tk,tiles", GROUP_CASES)
@pytest.mark.parametrize("ragged", [0, 5])
def test_load_group_remainders(T, G, Hkv, tk, tiles, ragged):
    d = 128
    npre = 2 * tiles * tk - ragged
    parent = wl.random_tree_parent(T, T * G + tiles)
    q = gen((T, G * Hkv, d), 90 + T, torch.bfloat16)
    k = gen((Hkv, npre + T, d), 91 + T, torch.bfloat16)
    v = gen((Hkv, npre + T, d), 92 + T, torch.bfloat16)
    po, pl = tsw.tree_attn_split(q, k, v, parent, npre, 2, impl="mfma")
    o, lse = tsw.lse_merge(po, pl)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v),
                                    parent, npre, 1 / np.sqrt(d), nthreads=NTHREADS)
    check(o, lse, o_ref, l_ref, TOL["bf16"], "T=%d G=%d tiles=%d ragged=%d" % (T, G, tiles, ragged))


@pytest.mark.parametrize("S,R,d,misaligned", [(9, 300, 128, False), (9, 301, 128, False), (40, 7, 128, False),
                                             (17, 301, 128, True), (9, 300, 64, False)])
def test_lse_merge_against_oracle(S, R, d, misaligned):
    """Both merge kernels: two rows per wavefront (d = 128, 16-byte aligned;
    an odd row count leaves the last wavefront half empty; more than 32
    splits take a second round of LSE lanes) and one row per wavefront (an
    output 4 bytes off 16-byte alignment, d = 64).  Empty splits and rows
    whose every split is empty included."""
    rng = np.random.default_rng(5 + S + R)
    po = rng.standard_normal((S, R, d)).astype(np.float32)
    pl = (rng.standard_normal((S, R)) * 5).astype(np.float32)
    pl[2] = -np.inf
    pl[5, :R // 3] = -np.inf
    pl[:, R - 1] = -np.inf
    out = None
    if misaligned:
        buf = torch.empty(R * d + 1, dtype=torch.float32, device="cuda")
        out = (buf[1:].view(R, d), torch.empty(R, dtype=torch.float32, device="cuda"))
    o, lse = tsw.lse_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), out=out)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.lse_merge(po.astype(np.float64), pl.astype(np.float64))
    # the row with every split empty: LSE -inf and a zero row on both sides
    assert l_ref[R - 1] == -np.inf and np.all(o_ref[R - 1] == 0.0)
    assert float(lse[R - 1]) == -np.inf and bool(torch.all(o[R - 1] == 0.0))
    check(o[:R - 1], lse[:R - 1], o_ref[:R - 1], l_ref[:R - 1], 1e-5, "merge S=%d R=%d d=%d" % (S, R, d))


def test_deterministic():
    w = wl.WORKLOADS["gqa8b_8k"]
    q, k, v = wl.make_qkv(w, device="cuda")
    o0, l0 = tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix)
    for _ in range(5):
        o1, l1 = tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_small_workspace_rejected():
    w = wl.WORKLOADS["gqa8b_8k"]
    q, k, v = wl.make_qkv(w, device="cuda")
    need = tsw.workspace_size(q, k, w.n_prefix)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=q.device)
    with pytest.raises(tsw.TswError) as e:
        tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix, workspace=ws)
    assert e.value.status == -5


def test_planner_fills_the_chip():
    import ctypes
    w = wl.WORKLOADS["gqa8b_100k"]
    desc = tsw.AttnDesc(T=w.n_nodes, Hq=w.Hq, Hkv=w.Hkv, d=w.d, n_prefix=w.n_prefix,
                        kv_head_stride=w.cap * w.d, dtype=tsw.DTYPE_BF16, impl=0,
                        scale=w.scale(), reserved=0)
    n = ctypes.c_int32(0)
    assert tsw.lib().tsw_plan_splits(ctypes.byref(desc), -1, ctypes.byref(n)) == 0
    s = n.value
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say("CUs %d splits %d" % (cus, s))
    assert s * w.Hkv <= cus and s * w.Hkv > cus // 2


@pytest.mark.parametrize("Hq", [32, 40])
@pytest.mark.parametrize("where", ["first_tile", "late_tile", "tree_row"])
def test_large_logit_headroom(where, Hq):
    """A key whose score is ~60 nats above every other score.  When it is
    not in a split's first tile, the fast pass flags its rows and the
    work-group reruns the split with exact row maxima; either way the
    result must match the oracle.  Hq = 40 (13 query blocks per kv head)
    puts flagged rows in the block the four waves share."""
    T, Hkv, d, npre = 40, 8, 128, 4096
    parent = wl.kary_tree_parent(T, 3)
    q = gen((T, Hq, d), 81, torch.bfloat16)
    k = gen((Hkv, npre + T, d), 82, torch.bfloat16)
    v = gen((Hkv, npre + T, d), 83, torch.bfloat16)
    pos = {"first_tile": 0, "late_tile": 3000, "tree_row": npre + 7}[where]
    # every query of head 0 is the same vector u; one key of kv head 0 is
    # 10.5 u, so that key scores 10.5 |u|^2 / sqrt(d) ~ 60 nats for all of them
    u = gen((d,), 84, torch.float32)
    u = (u / u.norm() * 8.0).to(torch.bfloat16)
    q[:, 0, :] = u
    k[0, pos] = (u.float() * 10.5).to(torch.bfloat16)
    o, lse = tsw.tree_attn_verify(q, k, v, parent, npre)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v),
                                    parent, npre, 1 / np.sqrt(d), nthreads=NTHREADS)
    if where != "tree_row":
        assert float(np.min(l_ref[:, 0])) - float(np.median(l_ref)) > 45.0
    check(o, lse, o_ref, l_ref, TOL["bf16"], "large logit %s" % where)


def test_hip_graph_replays_match_eager():
    """Verify and partial calls captured in one HIP graph: every replay, with
    eager work and synchronisations in between, equals the eager result bit
    for bit (the library records only kernel launches)."""
    T, Hq, Hkv, d, npre = 40, 32, 8, 128, 6000
    parent = wl.kary_tree_parent(T, 3)
    q = gen((T, Hq, d), 91, torch.bfloat16)
    k = gen((Hkv, npre + T, d), 92, torch.bfloat16)
    v = gen((Hkv, npre + T, d), 93, torch.bfloat16)
    qp = gen((4, Hq, d), 94, torch.bfloat16)
    kp = gen((Hkv, npre + 4, d), 95, torch.bfloat16)
    vp = gen((Hkv, npre + 4, d), 96, torch.bfloat16)
    chain = wl.chain_parent(4)
    idx = torch.from_numpy(np.sort(np.random.default_rng(9).choice(npre, 1500, replace=False))
                           .astype(np.int32)).cuda()
    o_e, l_e = tsw.tree_attn_verify(q, k, v, parent, npre)
    op_e, lp_e = tsw.tree_attn_partial(qp, kp, vp, chain, idx, npre)
    torch.cuda.synchronize()

    cs = torch.cuda.Stream()
    o = torch.empty_like(o_e); lse = torch.empty_like(l_e)
    op = torch.empty_like(op_e); lp = torch.empty_like(lp_e)
    ws = torch.empty(max(tsw.workspace_size(q, k, npre), 256), dtype=torch.uint8, device=q.device)
    wsp = torch.empty(max(tsw.workspace_size(qp, kp, npre, idx.numel()), 256), dtype=torch.uint8,
                      device=q.device)
    c1 = tsw.prepare_verify(q, k, v, parent, npre, o, lse, ws, stream=cs)
    c2 = tsw.prepare_verify(qp, kp, vp, chain, npre, op, lp, wsp, idx=idx, stream=cs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        c1()
        c2()
    for rep in range(4):
        for t in (o, lse, op, lp):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # eager work between replays reuses the same kernels
        tsw.tree_attn_verify(q, k, v, parent, npre)
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, l_e), rep
        assert torch.equal(op, op_e) and torch.equal(lp, lp_e), rep
    say("graph replays: 4 x bit-identical")


@pytest.mark.parametrize("impl,npre", [("mfma", 5000), ("valu", 700), ("auto", 100)])
def test_v_ones_gives_exactly_one(impl, npre):
    """V = 1 everywhere: every output element is 1 up to float32 rounding of
    the normalisation, because the row sum is taken over the same (rounded)
    weights that multiply V; the LSE still matches the oracle."""
    T, Hq, Hkv, d = 40, 32, 8, 128
    parent = wl.kary_tree_parent(T, 3)
    q = gen((T, Hq, d), 71, torch.bfloat16)
    k = gen((Hkv, npre + T, d), 72, torch.bfloat16)
    v = torch.ones((Hkv, npre + T, d), dtype=torch.bfloat16, device=q.device)
    o, lse = tsw.tree_attn_verify(q, k, v, parent, npre, impl=impl)
    torch.cuda.synchronize()
    err = float((o - 1.0).abs().max())
    say("V=1 %s: max|O-1| %.3g" % (impl, err))
    assert err <= 2e-6
    o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v),
                                    parent, npre, 1 / np.sqrt(d), nthreads=NTHREADS)
    check(o, lse, o_ref, l_ref, TOL["bf16"], "V=1 %s" % impl)
