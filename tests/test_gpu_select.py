"""GPU parity of partial-cache selection.  What is claimed, and checked:
the importance values within relative 1e-4 of the float64 oracle; the index
list identical to the oracle's selection run on the kernel's own importance
values (the ranking decision taken in the kernel's float32 precision);
against the float64 ranking, only consistency outside a 1e-3 relative band
around the cut (every kept position at least (1 - 1e-3) times as important
as every dropped one); and the list feeding the partial-cache attention."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.select as sel
import tree_verification_attention_tsw_amd as tsw
from tree_verification_attention_tsw_amd import workloads as wl

pytestmark = pytest.mark.gpu
NTHREADS = min(16, len(os.sched_getaffinity(0)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsw.lib()


def gen(shape, seed, dtype):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda").to(dtype)


def run(T, Hq, Hkv, d, n_prefix, n_keep, n_idx, dtype, seed, zero_k=False):
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = gen((T, Hq, d), seed, tdt)
    k = gen((Hkv, n_prefix + T, d), seed + 1, tdt)
    v = gen((Hkv, n_prefix + T, d), seed + 2, tdt)
    if zero_k:
        k.zero_()
    parent = wl.kary_tree_parent(T, 3)
    _, lse = tsw.tree_attn_verify(q, k, v, parent, n_prefix)
    imp = torch.empty(max(n_prefix, 1), dtype=torch.float32, device="cuda")
    idx, _ = tsw.select_partial(q, k, lse, n_prefix, n_keep, n_idx, importance=imp)
    torch.cuda.synchronize()
    say("select T=%d Hq=%d Hkv=%d d=%d n_prefix=%d keep=%d n_idx=%d %s" % (T, Hq, Hkv, d, n_prefix, n_keep,
                                                                         n_idx, dtype))
    imp_gpu = imp[:n_prefix].cpu().numpy().astype(np.float64)
    imp_ref = sel.importance(wl.oracle_view(q), wl.oracle_view(k), lse.cpu().numpy(), n_prefix, 1 / np.sqrt(d))
    if n_prefix:
        rel = float(np.max(np.abs(imp_gpu - imp_ref) / np.maximum(imp_ref, 1e-30)))
        say("  importance max rel err %.3g" % rel)
        assert rel <= 1e-4
    got = idx.cpu().numpy().tolist()
    assert got == sel.select(imp_gpu, n_prefix, n_keep, n_idx).tolist()
    # away from the cut the float64 ranking agrees
    chosen = set(got[min(n_keep, len(got)):])
    rest = [p for p in range(min(n_keep, n_prefix), n_prefix) if p not in chosen]
    if chosen and rest:
        assert min(imp_ref[list(chosen)]) >= max(imp_ref[rest]) * (1 - 1e-3)
    return q, k, v, idx


@pytest.mark.parametrize("T,Hq,Hkv,d,n_prefix,n_keep,n_idx,dtype", [
    (40, 32, 8, 128, 102400, 128, 4096, "bf16"),
    (40, 40, 8, 128, 20000, 128, 4096, "bf16"),
    (13, 32, 32, 128, 9000, 64, 1000, "bf16"),
    (13, 4, 4, 64, 3000, 16, 500, "f32"),
    (4, 8, 2, 128, 257, 0, 100, "bf16"),
    (4, 8, 2, 128, 300, 128, 4096, "bf16"),       # the whole prefix
    (4, 8, 2, 128, 300, 200, 100, "bf16"),        # more kept than asked
    (4, 8, 2, 128, 300, 10, 0, "bf16"),           # nothing asked
])
def test_select_matches_oracle(T, Hq, Hkv, d, n_prefix, n_keep, n_idx, dtype):
    run(T, Hq, Hkv, d, n_prefix, n_keep, n_idx, dtype, 3 + n_prefix)


def test_select_ties_take_lowest_positions():
    # K = 0: every position has the same importance, so the lowest win
    _, _, _, idx = run(13, 8, 2, 128, 5000, 100, 700, "bf16", 5, zero_k=True)
    assert idx.cpu().numpy().tolist() == list(range(700))


def test_selected_list_feeds_partial_attention():
    T, Hq, Hkv, d, n = 4, 32, 8, 128, 30000
    q, k, v, idx = run(T, Hq, Hkv, d, n, 128, 4096, "bf16", 11)
    chain = wl.chain_parent(T)
    o, lse = tsw.tree_attn_partial(q, k, v, chain, idx, n)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.tree_attn(wl.oracle_view(q), wl.oracle_view(k), wl.oracle_view(v), chain, n,
                                    1 / np.sqrt(d), idx=idx.cpu().numpy(), nthreads=NTHREADS)
    assert float(np.max(np.abs(o.cpu().double().numpy() - o_ref))) <= 4e-3
    assert float(np.max(np.abs(lse.cpu().double().numpy() - l_ref))) <= 4e-3


def check_selection(imp_gpu, imp_ref, idx, n_prefix, n_keep, n_idx):
    if n_prefix:
        rel = float(np.max(np.abs(imp_gpu - imp_ref) / np.maximum(imp_ref, 1e-30)))
        say("  importance max rel err %.3g" % rel)
        assert rel <= 1e-4
    got = idx.cpu().numpy().tolist()
    assert got == sel.select(imp_gpu, n_prefix, n_keep, n_idx).tolist()


@pytest.mark.parametrize("T,Hq,Hkv,d,n_prefix,n_keep,n_idx,dtype", [
    (40, 32, 8, 128, 102400, 128, 4096, "bf16"),  # root scores from the split kernel
    (40, 40, 8, 128, 20003, 128, 4096, "bf16"),   # ragged prefix end, G = 5
    (64, 20, 4, 128, 7001, 64, 1000, "bf16"),     # 320 rows per kv head: 20 query blocks
    (13, 32, 32, 128, 9000, 64, 1000, "bf16"),    # G = 1
    (4, 32, 1, 128, 5000, 16, 300, "bf16"),       # G = 32: importance from K
    (13, 4, 4, 64, 3000, 16, 500, "f32"),         # vector-ALU verification
    (4, 8, 2, 128, 300, 128, 4096, "bf16"),       # the whole prefix
    (4, 8, 2, 128, 300, 200, 100, "bf16"),        # more kept than asked
    (4, 8, 2, 128, 300, 10, 0, "bf16"),           # nothing asked
])
def test_verify_select_matches_verify_and_oracle(T, Hq, Hkv, d, n_prefix, n_keep, n_idx, dtype):
    """The combined call gives verification's o and lse bit for bit, and the
    selection to the same bar as the separate call."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    seed = 7 + n_prefix
    q = gen((T, Hq, d), seed, tdt)
    k = gen((Hkv, n_prefix + T, d), seed + 1, tdt)
    v = gen((Hkv, n_prefix + T, d), seed + 2, tdt)
    parent = wl.kary_tree_parent(T, 3)
    imp = torch.full((max(n_prefix, 1),), float("nan"), dtype=torch.float32, device="cuda")
    o, lse, idx, _ = tsw.tree_attn_verify_select(q, k, v, parent, n_prefix, n_keep, n_idx, importance=imp)
    o_ref, lse_ref = tsw.tree_attn_verify(q, k, v, parent, n_prefix)
    torch.cuda.synchronize()
    say("verify_select T=%d Hq=%d Hkv=%d d=%d n_prefix=%d keep=%d n_idx=%d %s" % (T, Hq, Hkv, d, n_prefix,
                                                                                n_keep, n_idx, dtype))
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    imp_gpu = imp[:n_prefix].cpu().numpy().astype(np.float64)
    imp_ref = sel.importance(wl.oracle_view(q), wl.oracle_view(k), lse.cpu().numpy(), n_prefix, 1 / np.sqrt(d))
    check_selection(imp_gpu, imp_ref, idx, n_prefix, n_keep, n_idx)


def test_verify_select_repeated_calls_share_workspace():
    """Two calls in a row on one workspace (the digit totals are cleared by
    each call), the second smaller."""
    T, Hq, Hkv, d = 40, 32, 8, 128
    ws = torch.empty(tsw.verify_select_workspace_size(gen((T, Hq, d), 1, torch.bfloat16),
                                                      gen((Hkv, 60040, d), 2, torch.bfloat16), 60000),
                     dtype=torch.uint8, device="cuda")
    for n_prefix, seed in ((60000, 21), (33333, 22)):
        q = gen((T, Hq, d), seed, torch.bfloat16)
        k = gen((Hkv, n_prefix + T, d), seed + 1, torch.bfloat16)
        v = gen((Hkv, n_prefix + T, d), seed + 2, torch.bfloat16)
        parent = wl.kary_tree_parent(T, 3)
        imp = torch.empty(n_prefix, dtype=torch.float32, device="cuda")
        need = tsw.verify_select_workspace_size(q, k, n_prefix)
        assert need <= ws.numel()
        _, lse, idx, _ = tsw.tree_attn_verify_select(q, k, v, parent, n_prefix, 128, 4096, importance=imp,
                                                     workspace=ws)
        torch.cuda.synchronize()
        say("verify_select repeat n_prefix=%d" % n_prefix)
        imp_gpu = imp.cpu().numpy().astype(np.float64)
        imp_ref = sel.importance(wl.oracle_view(q), wl.oracle_view(k), lse.cpu().numpy(), n_prefix,
                                 1 / np.sqrt(d))
        check_selection(imp_gpu, imp_ref, idx, n_prefix, 128, 4096)


@pytest.mark.parametrize("case", range(20))
def test_select_random_shapes(case):
    """Seeded random shapes: tree size, head grouping (up to 32 query heads
    per kv head, so both importance sources run: the verification kernel's
    root scores and a pass over K), precision, committed length (tile edges
    mixed in), kept prefix and list size; even cases the separate selection
    call, odd cases the combined call (verification's o and lse bit for bit
    against the plain call)."""
    rng = np.random.default_rng(9300 + case)
    T = int(rng.integers(1, 65))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 32]))
    Hkv = int(rng.choice([h for h in (1, 2, 4, 8) if h * G <= 64]))
    Hq = G * Hkv
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    d = 128 if dtype == "bf16" else int(rng.choice([64, 128]))
    if rng.random() < 0.3:
        n_prefix = int(rng.choice([0, 1, 63, 64, 65, 255, 256, 257, 4095, 4096, 4097]))
    else:
        n_prefix = int(rng.integers(0, 20001))
    n_keep = int(rng.choice([0, 1, 16, 64, 128, 300]))
    n_idx = int(rng.integers(0, n_prefix + 200))
    seed = 9300 + 17 * case
    if case % 2 == 0:
        run(T, Hq, Hkv, d, n_prefix, n_keep, n_idx, dtype, seed)
        return
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = gen((T, Hq, d), seed, tdt)
    k = gen((Hkv, n_prefix + T, d), seed + 1, tdt)
    v = gen((Hkv, n_prefix + T, d), seed + 2, tdt)
    parent = wl.random_tree_parent(T, seed)
    imp = torch.full((max(n_prefix, 1),), float("nan"), dtype=torch.float32, device="cuda")
    say("verify_select random case %d: T=%d Hq=%d Hkv=%d d=%d n_prefix=%d keep=%d n_idx=%d %s" % (
        case, T, Hq, Hkv, d, n_prefix, n_keep, n_idx, dtype))
    o, lse, idx, _ = tsw.tree_attn_verify_select(q, k, v, parent, n_prefix, n_keep, n_idx, importance=imp)
    o_ref, lse_ref = tsw.tree_attn_verify(q, k, v, parent, n_prefix)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    imp_gpu = imp[:n_prefix].cpu().numpy().astype(np.float64)
    imp_ref = sel.importance(wl.oracle_view(q), wl.oracle_view(k), lse.cpu().numpy(), n_prefix, 1 / np.sqrt(d))
    check_selection(imp_gpu, imp_ref, idx, n_prefix, n_keep, n_idx)
