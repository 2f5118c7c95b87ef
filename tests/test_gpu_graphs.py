"""A whole decoding step captured in one HIP graph: verification fused with
the next draft pass's selection, penalised greedy acceptance, compaction of
the accepted rows, a draft pass over the selected list, and the paged
verification and draft pass of a batch.  Every replay, with the caches
restored and eager work and synchronisations in between, must equal the
eager run bit for bit (the library records kernel launches only: no memory
sets, no copies, no host synchronisation)."""
import sys

import numpy as np
import pytest
import torch

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


def rnd(shape, g, dtype=torch.bfloat16):
    return torch.randn(shape, generator=g, device="cuda").to(dtype)


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).cuda()


def test_decoding_step_in_one_graph():
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    rng = np.random.default_rng(4242)
    T, Hq, Hkv, d, npre, vocab = 40, 32, 8, 128, 6000, 5000
    n_keep, n_idx, Td = 64, 1000, 4
    parent = wl.kary_tree_parent(T, 3)
    chain = wl.chain_parent(Td)
    q = rnd((T, Hq, d), g)
    k = rnd((Hkv, npre + T + Td, d), g)
    v = rnd((Hkv, npre + T + Td, d), g)
    qd = rnd((Td, Hq, d), g)
    logits = torch.randn((T, vocab), generator=g, device="cuda")
    best = logits.argmax(dim=1).cpu().numpy()
    draft = i32([0] + [int(best[parent[i]]) if rng.random() < 0.8 else int(rng.integers(vocab))
                       for i in range(1, T)])
    recent = i32(rng.integers(0, vocab, 700))
    # paged batch
    lengths, page_rows, B = [3000, 129, 4500], 64, 3
    need = [-(-(n + T) // page_rows) for n in lengths]
    n_pages = sum(need) + 3
    kp, vp = rnd((n_pages, Hkv, page_rows, d), g), rnd((n_pages, Hkv, page_rows, d), g)
    qb = rnd((B, T, Hq, d), g)
    perm = rng.permutation(n_pages).astype(np.int32)
    table = np.full((B, max(need)), -1, dtype=np.int32)
    at = 0
    for b, c in enumerate(need):
        table[b, :c] = perm[at:at + c]
        at += c
    table_t = i32(table)
    n_idx_b = [1200, 0, 2048]
    lists = np.full((B, max(n_idx_b) + 1), -1, dtype=np.int32)
    for b, (n, c) in enumerate(zip(lengths, n_idx_b)):
        lists[b, :c] = wl.retained_index_set(n, c, 64, 77 + b)
    lists_t = i32(lists)

    k_saved, v_saved = k.clone(), v.clone()
    cs = torch.cuda.Stream()
    f32 = dict(dtype=torch.float32, device="cuda")
    o, lse = torch.empty((T, Hq, d), **f32), torch.empty((T, Hq), **f32)
    idx = torch.empty(min(n_idx, npre), dtype=torch.int32, device="cuda")
    imp = torch.empty(npre, **f32)
    res = torch.empty(2 + 2 * T, dtype=torch.int32, device="cuda")
    od, ld = torch.empty((Td, Hq, d), **f32), torch.empty((Td, Hq), **f32)
    ob, lb = torch.empty((B, T, Hq, d), **f32), torch.empty((B, T, Hq), **f32)
    obd, lbd = torch.empty((B, T, Hq, d), **f32), torch.empty((B, T, Hq), **f32)
    ws_acc = torch.empty(max(tsw.accept_workspace_size(T, vocab), 256), dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(max(tsw.workspace_size(qd, k, npre + T, idx.numel()), 256), dtype=torch.uint8,
                       device="cuda")
    ws_b = torch.empty(max(tsw.paged_workspace_size(qb, kp, table_t, lengths), 256), dtype=torch.uint8,
                       device="cuda")
    ws_bd = torch.empty(max(tsw.paged_partial_workspace_size(qb, kp, table_t, lengths, n_idx_b), 256),
                        dtype=torch.uint8, device="cuda")
    outs = (o, lse, idx, imp, res, od, ld, ob, lb, obd, lbd)

    calls = [
        tsw.prepare_verify_select(q, k, v, parent, npre, n_keep, n_idx, o, lse, idx, importance=imp, stream=cs),
        tsw.prepare_accept_penalized(parent, logits, draft, recent, 256, 1.3, res, ws_acc, stream=cs),
        tsw.prepare_compact(k, v, npre, T, res, stream=cs),
        # the draft pass after the step: the selected positions, then Td new
        # rows after the committed ones (here simply rows npre + T ..)
        tsw.prepare_verify(qd, k, v, chain, npre + T, od, ld, ws_d, idx=idx, stream=cs),
        tsw.prepare_verify_paged(qb, kp, vp, table_t, lengths, parent, ob, lb, ws_b, stream=cs),
        tsw.prepare_partial_paged(qb, kp, vp, table_t, lengths, parent, lists_t, n_idx_b, obd, lbd, ws_bd,
                                  stream=cs),
    ]

    def restore_and_poison():
        k.copy_(k_saved)
        v.copy_(v_saved)
        for t in outs:
            if t.dtype == torch.int32:
                t.fill_(-77)
            else:
                t.fill_(float("nan"))

    # eager run of the same sequence on the capture stream
    restore_and_poison()
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        for c in calls:
            c()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs] + [k.clone(), v.clone()]
    r = res.cpu().numpy()
    say("eager step: accepted path length %d, bonus %d, %d positions selected" % (r[0], r[1], idx.numel()))
    assert r[0] >= 1 and bool(torch.isfinite(o).all()) and bool(torch.isfinite(od).all())

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cs):
        for c in calls:
            c()
    for rep in range(4):
        restore_and_poison()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        tsw.tree_attn_verify(q, k_saved, v_saved, parent, npre)     # eager work between replays
        torch.cuda.synchronize()
        got = list(outs) + [k, v]
        for i, (a, b) in enumerate(zip(got, want)):
            same = torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 \
                else torch.equal(a, b)
            assert same, (rep, i)
    say("decoding-step graph: 4 replays bit-identical to the eager run")
