"""GPU parity of the paged batch call: every sequence's rows against the
float64 oracle on that sequence's cache, rebuilt contiguously from the pages
(K and V pages shuffled in the pool, sequences of different lengths)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_tsw_amd as tsw
from tree_verification_attention_tsw_amd import workloads as wl

pytestmark = pytest.mark.gpu
TOL = 4e-3
NTHREADS = min(16, len(os.sched_getaffinity(0)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsw.lib()


def make_batch(lengths, T, Hq, Hkv, page_rows, seed, spare_pages=7):
    d = 128
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    need = [-(-(n + T) // page_rows) for n in lengths]
    n_pages = sum(need) + spare_pages
    kp = torch.randn((n_pages, Hkv, page_rows, d), generator=g, device="cuda").to(torch.bfloat16)
    vp = torch.randn((n_pages, Hkv, page_rows, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((len(lengths), T, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    perm = np.random.default_rng(seed).permutation(n_pages).astype(np.int32)
    max_pages = max(need) + 2
    table = np.full((len(lengths), max_pages), -1, dtype=np.int32)    # unused entries are never read
    at = 0
    for b, k in enumerate(need):
        table[b, :k] = perm[at:at + k]
        at += k
    return q, kp, vp, torch.from_numpy(table).cuda(), table


def contiguous(pool, table_row, rows, page_rows):
    """[Hkv, rows, d] cache of one sequence, gathered from its pages."""
    pages = torch.from_numpy(table_row[: -(-rows // page_rows)].astype(np.int64)).cuda()
    x = pool[pages]                                   # [k, Hkv, page_rows, d]
    return x.permute(1, 0, 2, 3).reshape(pool.shape[1], -1, pool.shape[3])[:, :rows].contiguous()


def check_batch(lengths, T, Hq, Hkv, page_rows, seed, parent=None):
    parent = parent if parent is not None else wl.kary_tree_parent(T, 3)
    q, kp, vp, table_t, table = make_batch(lengths, T, Hq, Hkv, page_rows, seed)
    say("paged B=%d T=%d Hq=%d Hkv=%d page=%d lengths=%s" % (len(lengths), T, Hq, Hkv, page_rows, lengths))
    o, lse = tsw.tree_attn_verify_paged(q, kp, vp, table_t, lengths, parent)
    torch.cuda.synchronize()
    for b, n in enumerate(lengths):
        k = contiguous(kp, table[b], n + T, page_rows)
        v = contiguous(vp, table[b], n + T, page_rows)
        o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q[b]), wl.oracle_view(k), wl.oracle_view(v), parent, n,
                                        1 / np.sqrt(128), nthreads=NTHREADS)
        eo = float(np.max(np.abs(o[b].cpu().double().numpy() - o_ref)))
        el = float(np.max(np.abs(lse[b].cpu().double().numpy() - l_ref)))
        say("  seq %d n_prefix %d: max|dO| %.3g max|dLSE| %.3g" % (b, n, eo, el))
        assert eo <= TOL and el <= TOL, (b, n, eo, el)


def test_paged_single_sequence():
    check_batch([5000], 40, 32, 8, 16, 1)


def test_paged_mixed_lengths():
    # a length on a page boundary, tree rows crossing a page, a short one
    check_batch([4096, 3001, 777, 12000, 300], 40, 32, 8, 16, 2)


def test_paged_large_pages_and_mha():
    check_batch([2500, 6400], 13, 16, 16, 256, 3)


def test_paged_gqa14b_shape():
    check_batch([3333, 1500, 9000], 40, 40, 8, 64, 4)


def test_paged_random_tree_T64():
    check_batch([2000, 4500], 64, 8, 2, 32, 5, parent=wl.random_tree_parent(64, 5))


def test_paged_twenty_query_blocks():
    # 64 nodes x 5 query heads = 320 rows per kv head (the 17-24 block shape)
    check_batch([3000, 1700], 64, 20, 4, 16, 9, parent=wl.random_tree_parent(64, 9))


def test_paged_odd_rows_per_sequence():
    # 13 nodes x 5 query heads = 65 rows per sequence: the segmented merge
    # cannot pair rows across sequences and takes its row-per-wave kernel
    check_batch([1500, 700, 2049], 13, 5, 1, 16, 8)


def test_paged_many_sequences():
    check_batch([400 + 137 * b for b in range(16)], 13, 32, 8, 16, 6)



def test_paged_sixty_four_sequences():
    """The largest batch a call takes (64 sequences: the per-sequence length
    and split tables are full), lengths from 0 up, every row compared."""
    rng = np.random.default_rng(64)
    lengths = [0, 1, 63, 64, 65] + [int(x) for x in rng.integers(0, 1500, 59)]
    check_batch(lengths, 13, 8, 2, 16, 64, parent=wl.random_tree_parent(13, 64))


def test_paged_matches_contiguous_call():
    """One sequence in pages vs the same cache contiguous: same definition,
    two kernels; both within the tolerance of each other."""
    T, Hq, Hkv = 40, 32, 8
    parent = wl.kary_tree_parent(T, 3)
    q, kp, vp, table_t, table = make_batch([20000], T, Hq, Hkv, 16, 7)
    o, lse = tsw.tree_attn_verify_paged(q, kp, vp, table_t, [20000], parent)
    k = contiguous(kp, table[0], 20000 + T, 16)
    v = contiguous(vp, table[0], 20000 + T, 16)
    o2, l2 = tsw.tree_attn_verify(q[0].contiguous(), k, v, parent, 20000)
    torch.cuda.synchronize()
    assert float((o[0] - o2).abs().max()) <= TOL and float((lse[0] - l2).abs().max()) <= TOL


def test_paged_bench_workload_all_rows():
    """The paged bench workload at its full size and in its launch
    configuration (eight GQA-8B sequences of 25600 ... 4800 committed tokens,
    16-row pages of a permuted pool): every (node, head) row of every
    sequence against the oracle."""
    w = wl.PAGED_WORKLOADS["paged_gqa8b_b8"]
    q, kp, vp, table_t = wl.make_paged_inputs(w, "cuda")
    parent = w.parent()
    o, lse = tsw.tree_attn_verify_paged(q, kp, vp, table_t, list(w.lengths), parent)
    torch.cuda.synchronize()
    table = table_t.cpu().numpy()
    T = w.n_nodes
    for b, n in enumerate(w.lengths):
        k = contiguous(kp, table[b], n + T, w.page_rows)
        v = contiguous(vp, table[b], n + T, w.page_rows)
        o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q[b]), wl.oracle_view(k), wl.oracle_view(v), parent, n,
                                        1 / np.sqrt(128), nthreads=NTHREADS)
        eo = float(np.max(np.abs(o[b].cpu().double().numpy() - o_ref)))
        el = float(np.max(np.abs(lse[b].cpu().double().numpy() - l_ref)))
        say("  bench workload seq %d n_prefix %d: max|dO| %.3g max|dLSE| %.3g (all rows)" % (b, n, eo, el))
        assert eo <= TOL and el <= TOL, (b, n, eo, el)


# ------------------------------------------------------------ paged draft pass

def index_lists(lengths, n_idx, seed, pad=3):
    """Per-sequence sorted index lists (the first 64 positions kept) in the
    rows of one int32 tensor with a few unused entries per row."""
    stride = max(max(n_idx), 1) + pad
    out = np.full((len(lengths), stride), -1, dtype=np.int32)
    for b, (n, k) in enumerate(zip(lengths, n_idx)):
        out[b, :k] = wl.retained_index_set(n, k, 64, seed * 100 + b)
    return out


def check_partial_batch(lengths, n_idx, T, Hq, Hkv, page_rows, seed, parent=None, no_lists=False):
    parent = parent if parent is not None else wl.kary_tree_parent(T, 3)
    q, kp, vp, table_t, table = make_batch(lengths, T, Hq, Hkv, page_rows, seed)
    lists = index_lists(lengths, n_idx, seed)
    say("paged draft pass B=%d T=%d Hq=%d Hkv=%d page=%d lengths=%s n_idx=%s" %
        (len(lengths), T, Hq, Hkv, page_rows, lengths, n_idx))
    idx_t = None if no_lists else torch.from_numpy(lists).cuda()
    o, lse = tsw.tree_attn_partial_paged(q, kp, vp, table_t, lengths, parent, idx_t, n_idx)
    torch.cuda.synchronize()
    for b, (n, k) in enumerate(zip(lengths, n_idx)):
        kc = contiguous(kp, table[b], n + T, page_rows)
        vc = contiguous(vp, table[b], n + T, page_rows)
        o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q[b]), wl.oracle_view(kc), wl.oracle_view(vc), parent, n,
                                        1 / np.sqrt(128), idx=lists[b, :k], nthreads=NTHREADS)
        eo = float(np.max(np.abs(o[b].cpu().double().numpy() - o_ref)))
        el = float(np.max(np.abs(lse[b].cpu().double().numpy() - l_ref)))
        say("  seq %d n_prefix %d n_idx %d: max|dO| %.3g max|dLSE| %.3g" % (b, n, k, eo, el))
        assert eo <= TOL and el <= TOL, (b, n, k, eo, el)


def test_paged_partial_mixed_lengths():
    # a whole cache as the list, an empty list, a list past one split's
    # 4096-entry slice, tree rows crossing a page
    check_partial_batch([4096, 3001, 777, 12000, 300], [1000, 3001, 0, 9000, 300], 40, 32, 8, 16, 11)


def test_paged_partial_large_pages_and_mha():
    check_partial_batch([2500, 6400], [2000, 5000], 13, 16, 16, 256, 12)


def test_paged_partial_all_lists_empty():
    """n_idx = 0 for every sequence, no index tensor: the tree rows only."""
    check_partial_batch([1000, 2000, 50], [0, 0, 0], 13, 8, 2, 32, 13, no_lists=True)


def test_paged_partial_draft_chain_many_sequences():
    lengths = [600 + 311 * b for b in range(16)]
    check_partial_batch(lengths, [min(n, 256 + 97 * b) for b, n in enumerate(lengths)], 4, 32, 8, 16, 14,
                        parent=wl.chain_parent(4))



def test_paged_partial_sixty_four_sequences():
    """The draft pass on the largest batch: 64 sequences, lists from empty
    to the whole cache."""
    rng = np.random.default_rng(65)
    lengths = [0, 1, 64, 129] + [int(x) for x in rng.integers(0, 2000, 60)]
    n_idx = [n if b % 5 == 0 else int(rng.integers(0, n + 1)) for b, n in enumerate(lengths)]
    check_partial_batch(lengths, n_idx, 4, 32, 8, 32, 65, parent=wl.chain_parent(4))


def test_paged_partial_random_tree_T64():
    check_partial_batch([2000, 4500], [1500, 4500], 64, 8, 2, 32, 15, parent=wl.random_tree_parent(64, 15))


def test_paged_partial_gqa14b_shape():
    check_partial_batch([3333, 9000], [3000, 4096], 40, 40, 8, 64, 16)


def test_paged_partial_matches_contiguous_call():
    """One sequence in pages vs the same cache and list contiguous: same
    definition, two kernels; both within the tolerance of each other."""
    T, Hq, Hkv, n, k = 4, 32, 8, 20000, 4096
    parent = wl.chain_parent(T)
    q, kp, vp, table_t, table = make_batch([n], T, Hq, Hkv, 16, 17)
    lists = index_lists([n], [k], 17)
    o, lse = tsw.tree_attn_partial_paged(q, kp, vp, table_t, [n], parent, torch.from_numpy(lists).cuda(), [k])
    kc = contiguous(kp, table[0], n + T, 16)
    vc = contiguous(vp, table[0], n + T, 16)
    idx = torch.from_numpy(lists[0, :k].copy()).cuda()
    o2, l2 = tsw.tree_attn_partial(q[0].contiguous(), kc, vc, parent, idx, n)
    torch.cuda.synchronize()
    assert float((o[0] - o2).abs().max()) <= TOL and float((lse[0] - l2).abs().max()) <= TOL


def test_paged_partial_bench_workload_all_rows():
    """The paged draft-pass bench workload at its full size and in its launch
    configuration (eight GQA-8B sequences of 25600 ... 4800 committed tokens,
    4096-position lists, four chained nodes, 16-row pages of a permuted
    pool): every (node, head) row of every sequence against the oracle."""
    w = wl.PAGED_WORKLOADS["paged_partial_gqa8b_b8"]
    q, kp, vp, table_t = wl.make_paged_inputs(w, "cuda")
    lists_t = wl.make_paged_index_lists(w, "cuda")
    parent = w.parent()
    o, lse = tsw.tree_attn_partial_paged(q, kp, vp, table_t, list(w.lengths), parent, lists_t, w.index_lengths())
    torch.cuda.synchronize()
    table, lists = table_t.cpu().numpy(), lists_t.cpu().numpy()
    T = w.n_nodes
    for b, (n, k) in enumerate(zip(w.lengths, w.index_lengths())):
        kc = contiguous(kp, table[b], n + T, w.page_rows)
        vc = contiguous(vp, table[b], n + T, w.page_rows)
        o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q[b]), wl.oracle_view(kc), wl.oracle_view(vc), parent, n,
                                        1 / np.sqrt(128), idx=lists[b, :k], nthreads=NTHREADS)
        eo = float(np.max(np.abs(o[b].cpu().double().numpy() - o_ref)))
        el = float(np.max(np.abs(lse[b].cpu().double().numpy() - l_ref)))
        say("  draft bench workload seq %d n_prefix %d n_idx %d: max|dO| %.3g max|dLSE| %.3g (all rows)"
            % (b, n, k, eo, el))
        assert eo <= TOL and el <= TOL, (b, n, eo, el)


def test_paged_partial_max_batch_and_degenerate_rows():
    """64 sequences (the most a call takes), T = 1 (plain decoding), lengths
    from 0 (no committed positions: the node attends to itself only) up, and
    index lists from empty to the whole cache."""
    lengths = [(37 * b) % 700 for b in range(64)]
    lengths[0], lengths[1] = 0, 1
    n_idx = [min(n, (53 * b) % 400) for b, n in enumerate(lengths)]
    n_idx[5] = lengths[5]
    check_partial_batch(lengths, n_idx, 1, 16, 4, 16, 18, parent=wl.chain_parent(1))


def test_paged_verify_max_batch_and_empty_prefix():
    lengths = [(41 * b) % 900 for b in range(64)]
    lengths[0] = 0
    check_batch(lengths, 4, 16, 4, 32, 19, parent=wl.chain_parent(4))
