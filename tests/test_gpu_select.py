"""GPU parity of partial-cache selection: importance against the float64
oracle (relative 1e-4), the index list bit-exact against the oracle's
selection applied to the kernel's own importance values (the decision taken
in the kernel's precision), consistency with the float64 ranking away from
the cut, and the list feeding the partial-cache attention."""
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
