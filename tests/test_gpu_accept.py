"""GPU parity of greedy acceptance and accepted-path compaction (through the
C ABI) against the numpy oracle: path, bonus token and per-node tokens
bit-exact; compacted caches bit-exact, every other row untouched."""
import sys

import numpy as np
import pytest
import torch

import oracle.accept as acc
import pins_accept as P
import tree_verification_attention_tsw_amd as tsw
from tree_verification_attention_tsw_amd import workloads as wl

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsw.lib()
    return torch.device("cuda:0")


def run_accept(parent, logits_np, draft, dtype):
    """logits_np float32 [T, V]; returns (GPU result numpy, oracle path, bonus, targets)."""
    lt = torch.from_numpy(np.ascontiguousarray(logits_np)).cuda()
    if dtype == "bf16":
        lt = lt.to(torch.bfloat16)
        ref_in = lt.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        ref_in = logits_np
    dt = torch.from_numpy(np.asarray(draft, dtype=np.int32)).cuda()
    res = tsw.accept_greedy(parent, lt, dt)
    torch.cuda.synchronize()
    path, bonus, target = acc.accept_greedy(parent, ref_in, draft)
    return res.cpu().numpy(), path, bonus, target


def check(res, path, bonus, target, T):
    L = len(path)
    assert res[0] == L and res[1] == bonus, (res[:2], L, bonus)
    assert list(res[2:2 + L]) == list(path)
    assert all(x == -1 for x in res[2 + L:2 + T])
    assert list(res[2 + T:2 + 2 * T]) == list(target)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_golden_fixture(dtype):
    g = P.read_golden()
    res, path, bonus, target = run_accept(g["parent"], g["logits"], g["draft"], dtype)
    assert list(path) == g["path"]
    check(res, path, bonus, target, len(g["parent"]))


@pytest.mark.parametrize("T,V,dtype,tree", [
    (1, 5, "f32", "chain"), (4, 1000, "bf16", "chain"), (13, 32003, "f32", "ternary"),
    (13, 32003, "bf16", "ternary"), (40, 128256, "f32", "ternary"), (40, 128256, "bf16", "ternary"),
    (64, 50000, "f32", "random"), (23, 7, "f32", "random")])
def test_random_trees(T, V, dtype, tree):
    for seed in range(3):
        rng = np.random.default_rng(1000 * T + seed)
        parent = {"chain": wl.chain_parent, "ternary": lambda n: wl.kary_tree_parent(n, 3),
                  "random": lambda n: wl.random_tree_parent(n, seed)}[tree](T)
        logits = rng.standard_normal((T, V)).astype(np.float32)
        if dtype == "bf16":   # decide on the values the kernel sees
            logits = torch.from_numpy(logits).to(torch.bfloat16).float().numpy()
        # ties for the maximum in different slices of the row: the first wins
        for i in range(T):
            m = float(logits[i].max()) + 1.0
            for j in sorted(rng.choice(V, size=min(3, V), replace=False)):
                logits[i, j] = m
        draft = rng.integers(0, V, size=T).astype(np.int32)
        for i in range(1, T):
            if rng.random() < 0.75:
                draft[i] = P.first_max(logits[int(parent[i])])
        say("accept T=%d V=%d %s %s seed=%d" % (T, V, dtype, tree, seed))
        res, path, bonus, target = run_accept(parent, logits, draft, dtype)
        check(res, path, bonus, target, T)


def test_unaligned_logits_view():
    # a row pitch that breaks 16-byte alignment takes the scalar path
    T, V = 13, 1001
    base = torch.randn(T * V + 1, device="cuda")
    lt = base[1:].view(T, V)
    parent = wl.kary_tree_parent(T, 3)
    ln = lt.cpu().numpy()
    draft = np.array([0] + [P.first_max(ln[int(parent[i])]) for i in range(1, T)], dtype=np.int32)
    res = tsw.accept_greedy(parent, lt, torch.from_numpy(draft).cuda()).cpu().numpy()
    path, bonus, target = acc.accept_greedy(parent, ln, draft)
    check(res, path, bonus, target, T)


def _caches(layers, Hkv, rows, d, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    k = torch.randn((layers, Hkv, rows, d), generator=g, device="cuda").to(tdt)
    v = torch.randn((layers, Hkv, rows, d), generator=g, device="cuda").to(tdt)
    return k, v


def _np(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("layers,Hkv,d,dtype,T", [(3, 2, 128, "bf16", 40), (1, 4, 64, "f32", 13),
                                                  (2, 8, 128, "f32", 64), (32, 8, 128, "bf16", 40)])
def test_compact_matches_oracle(layers, Hkv, d, dtype, T):
    n_prefix = 777
    rows = n_prefix + T + 5
    k, v = _caches(layers, Hkv, rows, d, dtype, T + d)
    k0, v0 = _np(k), _np(v)
    rng = np.random.default_rng(T)
    parent = wl.kary_tree_parent(T, 3) if T != 64 else wl.random_tree_parent(T, 5)
    V = 97
    logits = rng.standard_normal((T, V)).astype(np.float32)
    draft = np.array([0] + [P.first_max(logits[int(parent[i])]) for i in range(1, T)], dtype=np.int32)
    res = tsw.accept_greedy(parent, torch.from_numpy(logits).cuda(), torch.from_numpy(draft).cuda())
    tsw.kv_compact(k if layers > 1 else k[0], v if layers > 1 else v[0], n_prefix, T, res)
    torch.cuda.synchronize()
    path, _, _ = acc.accept_greedy(parent, logits, draft)
    say("compact layers=%d Hkv=%d d=%d %s path=%s" % (layers, Hkv, d, dtype, path))
    assert len(path) > 1
    assert np.array_equal(_np(k), acc.kv_compact(k0, n_prefix, path))
    assert np.array_equal(_np(v), acc.kv_compact(v0, n_prefix, path))


def test_compact_overlapping_rows():
    # path [0, 2, 5] on a 6-node tree: row n+2 is read (node 2) and written (k = 2)
    parent = np.array([-1, 0, 0, 1, 1, 2], dtype=np.int32)
    logits = np.zeros((6, 8), dtype=np.float32)
    logits[0, 3] = 1.0
    logits[2, 6] = 1.0
    draft = np.array([0, 1, 3, 0, 0, 6], dtype=np.int32)
    n_prefix = 10
    k, v = _caches(2, 3, n_prefix + 6, 128, "bf16", 3)
    k0, v0 = _np(k), _np(v)
    res = tsw.accept_greedy(parent, torch.from_numpy(logits).cuda(), torch.from_numpy(draft).cuda())
    tsw.kv_compact(k, v, n_prefix, 6, res)
    torch.cuda.synchronize()
    assert res.cpu().numpy()[:5].tolist() == [3, 0, 0, 2, 5]     # node 5 logits all 0: bonus 0
    assert np.array_equal(_np(k), acc.kv_compact(k0, n_prefix, [0, 2, 5]))
    assert np.array_equal(_np(v), acc.kv_compact(v0, n_prefix, [0, 2, 5]))


def test_compact_clamps_bad_result():
    # a result that did not come from tsw_accept_greedy: L and node indices
    # out of range are clamped, so only rows n_prefix .. n_prefix+T-1 change
    T, n_prefix = 5, 20
    k, v = _caches(1, 2, n_prefix + T + 8, 64, "f32", 9)
    k0 = k.clone()
    res = torch.tensor([100, 0, 0, 4000, -7, 3, 1] + [0] * (2 * T - 5), dtype=torch.int32, device="cuda")
    tsw.kv_compact(k, v, n_prefix, T, res)
    torch.cuda.synchronize()
    assert torch.equal(k[:, :, :n_prefix], k0[:, :, :n_prefix])
    assert torch.equal(k[:, :, n_prefix + T:], k0[:, :, n_prefix + T:])
    assert torch.equal(k[0, :, n_prefix + 1], k0[0, :, n_prefix + T - 1])   # 4000 -> T-1
    assert torch.equal(k[0, :, n_prefix + 2], k0[0, :, n_prefix + 0])       # -7 -> 0


@pytest.mark.parametrize("case", range(12))
def test_accept_compact_random_shapes(case):
    """Seeded random shapes for acceptance followed by compaction: tree
    (random, chain, 3-ary) of 1-64 nodes, vocabulary, layers, kv heads, head
    dim, precision, committed length and spare rows; drafts follow the
    parent's argmax with a drawn probability, so paths of many lengths occur.
    The result and every cache byte are compared with the oracle."""
    rng = np.random.default_rng(9900 + case)
    T = int(rng.integers(1, 65))
    kind = rng.integers(3)
    parent = (wl.random_tree_parent(T, 9900 + case) if kind == 0 else
              wl.chain_parent(T) if kind == 1 else wl.kary_tree_parent(T, 3))
    V = int(rng.choice([3, 97, 5001, 32000]))
    layers = int(rng.integers(1, 9))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    n_prefix = int(rng.integers(0, 3001))
    rows = n_prefix + T + int(rng.integers(0, 11))
    follow = float(rng.uniform(0.3, 1.0))
    logits = rng.standard_normal((T, V)).astype(np.float32)
    draft = np.array([0] + [P.first_max(logits[int(parent[i])]) if rng.random() < follow
                            else int(rng.integers(0, V)) for i in range(1, T)], dtype=np.int32)
    k, v = _caches(layers, Hkv, rows, d, dtype, 9900 + case)
    k0, v0 = _np(k), _np(v)
    res = tsw.accept_greedy(parent, torch.from_numpy(logits).cuda(), torch.from_numpy(draft).cuda())
    tsw.kv_compact(k, v, n_prefix, T, res)
    torch.cuda.synchronize()
    path, bonus, target = acc.accept_greedy(parent, logits, draft)
    say("accept+compact random case %d: T=%d V=%d layers=%d Hkv=%d d=%d %s n_prefix=%d path=%s" % (
        case, T, V, layers, Hkv, d, dtype, n_prefix, list(path)))
    check(res.cpu().numpy(), path, bonus, target, T)
    assert np.array_equal(_np(k), acc.kv_compact(k0, n_prefix, path))
    assert np.array_equal(_np(v), acc.kv_compact(v0, n_prefix, path))
