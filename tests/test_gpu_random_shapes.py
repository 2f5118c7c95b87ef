"""GPU parity on seeded random shapes: the HIP path (through the C ABI)
against the float64 oracle on every (node, head) row, for shapes drawn at
random rather than picked by hand.  Each case draws a tree (random, chain or
3-ary), the head grouping, the head dim and precision, the committed length
(edge values mixed in), the kernel (bf16 cases also on the vector-ALU
kernel), and for the draft pass an index list, for the split phase an
explicit split count (over the whole cache or an index list), for the paged
calls a batch of lengths and a page size.  Tolerances as in the other
parity tests: max-abs 4e-3 for bfloat16 inputs, 1e-5 for float32."""
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
EDGE_LENGTHS = [0, 1, 31, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1023, 4096]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsw.lib()
    return torch.device("cuda:0")


def draw_tree(rng, T, seed):
    kind = rng.integers(3)
    if kind == 0:
        return wl.random_tree_parent(T, seed), "random"
    if kind == 1:
        return wl.chain_parent(T), "chain"
    return wl.kary_tree_parent(T, 3), "3-ary"


def draw_length(rng, hi):
    if rng.random() < 0.35:
        return int(rng.choice([n for n in EDGE_LENGTHS if n <= hi]))
    return int(rng.integers(0, hi + 1))


def gen(shape, g, dtype):
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dtype)


def compare(o, lse, o_ref, lse_ref, tol, what):
    o = o.detach().cpu().double().numpy()
    lse = lse.detach().cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what + ": non-finite output"
    eo = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    el = float(np.max(np.abs(lse - lse_ref))) if lse.size else 0.0
    say("  %s: max|dO| %.3g max|dLSE| %.3g" % (what, eo, el))
    assert eo <= tol and el <= tol, (what, eo, el)


# ------------------------------------------------------------ contiguous cache

@pytest.mark.parametrize("case", range(48))
def test_random_contiguous(case):
    seed = 9100 + case
    rng = np.random.default_rng(seed)
    T = int(rng.choice([1, 2, 3, 4, 13, 40, 64]) if rng.random() < 0.5 else rng.integers(1, 65))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 9))
    # float32 runs the vector-ALU path; keep its oracle work small
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    d = 128 if (dtype == "bf16" and rng.random() < 0.85) else int(rng.choice([64, 128]))
    while T * G * Hkv > 2048:
        G = max(1, G // 2)
        if T * G * Hkv > 2048:
            T = max(1, T // 2)
    Hq = G * Hkv
    n_prefix = draw_length(rng, 6000 if dtype == "bf16" else 1500)
    parent, tree = draw_tree(rng, T, seed)
    mode = rng.choice(["verify", "partial", "split"])
    # bf16 with d = 128 also runs on the vector-ALU kernel when asked to
    impl = str(rng.choice(["auto", "valu"])) if (dtype == "bf16" and d == 128 and rng.random() < 0.3) else "auto"
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    cap = n_prefix + T + int(rng.integers(0, 3))
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = gen((T, Hq, d), g, tdt)
    k = gen((Hkv, cap, d), g, tdt)
    v = gen((Hkv, cap, d), g, tdt)
    idx = None
    if mode == "partial" or (mode == "split" and rng.random() < 0.5):
        n_idx = int(rng.integers(0, n_prefix + 1)) if rng.random() < 0.8 else n_prefix
        idx = wl.retained_index_set(n_prefix, n_idx, int(rng.choice([0, 4, 64])), seed)
    say("case %d: %s T=%d (%s) Hq=%d Hkv=%d d=%d %s impl=%s n_prefix=%d cap=%d%s" % (
        case, mode, T, tree, Hq, Hkv, d, dtype, impl, n_prefix, cap,
        "" if idx is None else " n_idx=%d" % len(idx)))
    it = None if idx is None else torch.from_numpy(idx.astype(np.int32)).cuda()
    if mode == "verify":
        o, lse = tsw.tree_attn_verify(q, k, v, parent, n_prefix, impl=impl)
    elif mode == "partial":
        o, lse = tsw.tree_attn_partial(q, k, v, parent, it, n_prefix, impl=impl)
    else:
        n_splits = int(rng.integers(1, 41))
        say("  n_splits=%d" % n_splits)
        po, pl = tsw.tree_attn_split(q, k, v, parent, n_prefix, n_splits, idx=it, impl=impl)
        o, lse = tsw.lse_merge(po, pl)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v), parent, n_prefix,
                                      1.0 / np.sqrt(d), idx=idx, nthreads=NTHREADS)
    compare(o, lse, o_ref, lse_ref, TOL[dtype], "all rows")


# ------------------------------------------------------------ paged pool

def paged_inputs(rng, lengths, T, Hq, Hkv, page_rows, seed):
    d = 128
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    need = [-(-(n + T) // page_rows) for n in lengths]
    n_pages = sum(need) + int(rng.integers(0, 5))
    kp = gen((n_pages, Hkv, page_rows, d), g, torch.bfloat16)
    vp = gen((n_pages, Hkv, page_rows, d), g, torch.bfloat16)
    q = gen((len(lengths), T, Hq, d), g, torch.bfloat16)
    perm = rng.permutation(n_pages).astype(np.int32)
    table = np.full((len(lengths), max(need) + int(rng.integers(0, 3))), -1, dtype=np.int32)
    at = 0
    for b, k in enumerate(need):
        table[b, :k] = perm[at:at + k]
        at += k
    return q, kp, vp, table


def sequence_cache(pool, table_row, rows, page_rows):
    pages = torch.from_numpy(table_row[: -(-rows // page_rows)].astype(np.int64)).cuda()
    x = pool[pages]
    return x.permute(1, 0, 2, 3).reshape(pool.shape[1], -1, pool.shape[3])[:, :rows].contiguous()


@pytest.mark.parametrize("case", range(24))
def test_random_paged(case):
    seed = 9700 + case
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 65))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 9))
    while T * G > 384:                       # the matrix-core shapes' limit
        G -= 1
    G = max(G, 1)
    if T * G > 384:
        T = 384 // G
    Hq = G * Hkv
    B = int(rng.integers(1, 6))
    page_rows = int(rng.choice([16, 32, 64, 128, 256]))
    lengths = [draw_length(rng, 5000) for _ in range(B)]
    parent, tree = draw_tree(rng, T, seed)
    draft = case % 2 == 1
    q, kp, vp, table = paged_inputs(rng, lengths, T, Hq, Hkv, page_rows, seed)
    table_t = torch.from_numpy(table).cuda()
    lists, n_idx = None, None
    if draft:
        n_idx = [int(rng.integers(0, n + 1)) for n in lengths]
        stride = max(max(n_idx), 1) + int(rng.integers(0, 4))
        lists = np.full((B, stride), -1, dtype=np.int32)
        for b, (n, k) in enumerate(zip(lengths, n_idx)):
            lists[b, :k] = wl.retained_index_set(n, k, int(rng.choice([0, 64])), seed * 10 + b)
    say("case %d: paged %s B=%d T=%d (%s) Hq=%d Hkv=%d page=%d lengths=%s%s" % (
        case, "draft pass" if draft else "verify", B, T, tree, Hq, Hkv, page_rows, lengths,
        "" if not draft else " n_idx=%s" % n_idx))
    if draft:
        o, lse = tsw.tree_attn_partial_paged(q, kp, vp, table_t, lengths, parent, torch.from_numpy(lists).cuda(),
                                             n_idx)
    else:
        o, lse = tsw.tree_attn_verify_paged(q, kp, vp, table_t, lengths, parent)
    torch.cuda.synchronize()
    for b, n in enumerate(lengths):
        kc = sequence_cache(kp, table[b], n + T, page_rows)
        vc = sequence_cache(vp, table[b], n + T, page_rows)
        idx = lists[b, :n_idx[b]] if draft else None
        o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q[b]), wl.oracle_view(kc), wl.oracle_view(vc), parent, n,
                                        1.0 / np.sqrt(128), idx=idx, nthreads=NTHREADS)
        compare(o[b], lse[b], o_ref, l_ref, TOL["bf16"], "sequence %d (n_prefix %d)" % (b, n))
