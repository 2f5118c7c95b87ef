"""Pins for the float64 oracle: checks against facts that do not come from the
oracle itself (closed forms, brute force over explicit sequences, library
attention, invariances, a hand-written fixture).

Each pin takes an oracle object (oracle.Oracle) so that the same checks can be
run against deliberately mutated oracle builds; a pin signals failure by
raising AssertionError (or any exception).

Page facts used (page title, part of page):
 * tree-based verification, lossless: each candidate must get exactly what the
   target model would compute for it alone -- "TokenSwift - A framework for
   accelerating ..." (aiboss88), technical principles; and the Tencent Cloud
   article "90分钟生成10万Token ..." (优势与特点, 无损的输出质量).
 * verification sees the full KV cache -- Tencent Cloud article, figure text
   under 技术原理.
 * the draft pass is the same model with a partial cache that keeps the
   initial positions -- aiboss88 page, dynamic KV cache update; Tencent Cloud
   article, 无损的输出质量.
 * the tree is 3-ary -- "From Hours to Minutes ..." (arxivlens), Technical
   Contribution.
"""
import math
import os

import numpy as np
import torch

from tree_verification_attention_tsw_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def _rand(shape, seed, dtype=np.float32):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape).astype(dtype)


def _path(parent, i):
    """Root-to-node path of node i (by walking parents, then reversing)."""
    p = []
    while i != -1:
        p.append(int(i))
        i = int(parent[i])
    return p[::-1]


def _explicit_sequence_attention(q, k, v, parent, n_prefix, scale, idx=None):
    """Brute force: for node i build the sequence (prefix rows, then the rows
    of the root-to-i path) and attend with the last query of that sequence."""
    T, Hq, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    qd, kd, vd = (x.astype(np.float64) for x in (q, k, v))
    pre = np.arange(n_prefix) if idx is None else np.asarray(idx)
    o = np.zeros((T, Hq, d))
    lse = np.zeros((T, Hq))
    for i in range(T):
        seq = np.concatenate([pre, n_prefix + np.array(_path(parent, i))]).astype(np.int64)
        for h in range(Hq):
            g = h // G
            ks, vs = kd[g, seq], vd[g, seq]
            s = scale * (ks @ qd[i, h])
            w = np.exp(s - s.max())
            o[i, h] = (w / w.sum()) @ vs
            lse[i, h] = s.max() + math.log(w.sum())
    return o, lse


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)), what
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol * max(1.0, np.max(np.abs(b)) if b.size else 1.0), (what, err)


# ----------------------------------------------------------------- mask pins

def pin_mask_ternary_closed_form(orc):
    """Full 3-ary trees: popcount(mask) = depth + 1, total set bits
    sum_l (l+1) 3^l, level sizes 1, 3, 9, 27."""
    for levels, total in ((2, 1 * 1 + 2 * 3 + 3 * 9), (3, 1 + 2 * 3 + 3 * 9 + 4 * 27)):
        n = wl.full_kary_nodes(levels)
        mask, depth = orc.mask_build(wl.kary_tree_parent(n))
        pops = [bin(int(m)).count("1") for m in mask]
        assert all(p == dd + 1 for p, dd in zip(pops, depth))
        assert sum(pops) == total, (sum(pops), total)
        hist = np.bincount(depth)
        assert list(hist) == [3 ** lv for lv in range(levels + 1)]
    assert total == 142


def pin_mask_chain(orc):
    """A single chain gives the causal (lower-triangular) pattern."""
    for T in (1, 2, 5, 63, 64):
        mask, depth = orc.mask_build(wl.chain_parent(T))
        for i in range(T):
            assert int(mask[i]) == (1 << (i + 1)) - 1
            assert depth[i] == i


def pin_mask_random_closure(orc):
    """Random trees vs the reflexive-transitive closure of the parent relation
    computed by Warshall's algorithm (a different method from walking)."""
    for seed in range(20):
        T = 1 + seed * 3 % 64
        parent = wl.random_tree_parent(T, seed)
        reach = np.eye(T, dtype=bool)
        for i in range(1, T):
            reach[i, parent[i]] = True
        for m in range(T):
            reach |= reach[:, m:m + 1] & reach[m:m + 1, :]
        mask, depth = orc.mask_build(parent)
        for i in range(T):
            bits = sum(1 << j for j in range(T) if reach[i, j])
            assert int(mask[i]) == bits
            assert depth[i] == reach[i].sum() - 1


def pin_mask_golden_13(orc):
    """The hand-written 13-node fixture."""
    rows = []
    with open(os.path.join(GOLDEN, "ternary_tree_13.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    parent = np.array([r[1] for r in rows], dtype=np.int32)
    mask, depth = orc.mask_build(parent)
    for r in rows:
        node, _, dep, anc = r[0], r[1], r[2], r[3:]
        assert depth[node] == dep
        assert int(mask[node]) == sum(1 << a for a in anc)


def pin_mask_rejects_bad_trees(orc):
    for bad in ([0], [-1, 1], [-1, 0, 3], [-1, -1], [], list(range(-1, 64))):
        try:
            orc.mask_build(np.array(bad, dtype=np.int32))
        except ValueError:
            continue
        raise AssertionError("accepted bad tree %r" % (bad,))


# ------------------------------------------------------------ attention pins

CASES = [  # (T, Hq, Hkv, d, n_prefix, tree seed or "ternary"/"chain")
    (1, 1, 1, 4, 0, "chain"),
    (1, 2, 1, 8, 9, "chain"),
    (6, 4, 2, 8, 5, 7),
    (13, 4, 4, 16, 37, "ternary"),
    (13, 6, 2, 8, 0, "ternary"),
    (9, 3, 1, 5, 11, 3),
    (40, 4, 1, 4, 3, "ternary"),
]


def _parent_for(T, spec):
    if spec == "chain":
        return wl.chain_parent(T)
    if spec == "ternary":
        return wl.kary_tree_parent(T, 3)
    return wl.random_tree_parent(T, spec)


def pin_explicit_sequence_bruteforce(orc):
    """Each node's output equals attention of the last query of the explicit
    sequence prefix + root-to-node path (numpy, float64)."""
    for n, (T, Hq, Hkv, d, npre, spec) in enumerate(CASES):
        parent = _parent_for(T, spec)
        q = _rand((T, Hq, d), 10 + n)
        k = _rand((Hkv, npre + T + 2, d), 20 + n)
        v = _rand((Hkv, npre + T + 2, d), 30 + n)
        scale = 1.0 / math.sqrt(d)
        o, lse = orc.tree_attn(q, k, v, parent, npre, scale)
        ob, lb = _explicit_sequence_attention(q, k, v, parent, npre, scale)
        _close(o, ob, what="O case %d" % n)
        _close(lse, lb, what="LSE case %d" % n)


def pin_chain_equals_causal_sdpa(orc):
    """A single chain is ordinary causal attention: torch's
    scaled_dot_product_attention (float64, CPU) over prefix + chain."""
    for T, H, d, npre in ((4, 2, 8, 7), (16, 3, 16, 33), (1, 1, 4, 0)):
        parent = wl.chain_parent(T)
        q = _rand((T, H, d), 41)
        k = _rand((H, npre + T, d), 42)
        v = _rand((H, npre + T, d), 43)
        scale = 0.37
        o, _ = orc.tree_attn(q, k, v, parent, npre, scale)
        L = npre + T
        qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
        kt = torch.from_numpy(k.astype(np.float64)).unsqueeze(0)
        vt = torch.from_numpy(v.astype(np.float64)).unsqueeze(0)
        pos_q = torch.arange(npre, L).unsqueeze(1)
        pos_k = torch.arange(L).unsqueeze(0)
        allowed = pos_k <= pos_q
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed,
                                                               scale=scale)
        _close(o, ref[0].permute(1, 0, 2).numpy(), what="chain vs sdpa")


def _key_counts(parent, n_pre):
    T = len(parent)
    return np.array([n_pre + len(_path(parent, i)) for i in range(T)])


def pin_zero_keys_give_mean(orc):
    """K = 0: every visible key has equal weight, so O is the mean of the
    visible V rows and LSE = ln(number of visible keys)."""
    T, Hq, Hkv, d, npre = 13, 4, 2, 8, 21
    parent = wl.kary_tree_parent(T, 3)
    q = _rand((T, Hq, d), 51)
    k = np.zeros((Hkv, npre + T, d), dtype=np.float32)
    v = _rand((Hkv, npre + T, d), 52)
    o, lse = orc.tree_attn(q, k, v, parent, npre, 0.5)
    cnt = _key_counts(parent, npre)
    for i in range(T):
        rows = list(range(npre)) + [npre + j for j in _path(parent, i)]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            _close(o[i, h], v[g, rows].astype(np.float64).mean(0), what="mean")
            _close(lse[i, h], math.log(cnt[i]), what="ln count")


def pin_scale_zero_gives_mean(orc):
    """scale = 0: uniform attention, LSE = ln(count), for the partial variant."""
    T, Hq, Hkv, d, npre = 6, 2, 1, 4, 50
    parent = wl.random_tree_parent(T, 5)
    idx = np.array([0, 1, 2, 17, 31, 49], dtype=np.int32)
    q = _rand((T, Hq, d), 53)
    k = _rand((Hkv, npre + T, d), 54)
    v = _rand((Hkv, npre + T, d), 55)
    o, lse = orc.tree_attn(q, k, v, parent, npre, 0.0, idx=idx)
    for i in range(T):
        rows = list(idx) + [npre + j for j in _path(parent, i)]
        for h in range(Hq):
            _close(o[i, h], v[0, rows].astype(np.float64).mean(0), what="mean")
            _close(lse[i, h], math.log(len(rows)), what="ln count")


def pin_onehot_values_give_weights(orc):
    """V = one-hot of the cache position: O is the softmax row itself.  It
    sums to 1, is zero off the visible set, and its ratios are exp of score
    differences, tying O to LSE: O_p = exp(s_p - LSE)."""
    T, Hq, Hkv, npre = 13, 2, 1, 10
    cap = npre + T
    d = cap
    parent = wl.kary_tree_parent(T, 3)
    q = _rand((T, Hq, d), 61)
    k = _rand((Hkv, cap, d), 62)
    v = np.tile(np.eye(cap, dtype=np.float32)[None], (Hkv, 1, 1))
    scale = 0.3
    o, lse = orc.tree_attn(q, k, v, parent, npre, scale)
    for i in range(T):
        vis = set(range(npre)) | {npre + j for j in _path(parent, i)}
        for h in range(Hq):
            assert abs(o[i, h].sum() - 1.0) < 1e-12
            for p in range(cap):
                if p not in vis:
                    assert o[i, h, p] == 0.0
                else:
                    s = scale * float(np.dot(q[i, h].astype(np.float64), k[0, p].astype(np.float64)))
                    assert abs(o[i, h, p] - math.exp(s - lse[i, h])) < 1e-12


def pin_shift_invariance(orc):
    """Adding u to every key row leaves O unchanged and adds scale*q.u to LSE."""
    T, Hq, Hkv, d, npre = 9, 4, 2, 8, 19
    parent = wl.random_tree_parent(T, 11)
    q = _rand((T, Hq, d), 71)
    # dyadic K (multiples of 2^-10, |k| < 8) so that k + u is exact in float32
    k = (np.round(_rand((Hkv, npre + T, d), 72) * 1024) / 1024).astype(np.float32)
    v = _rand((Hkv, npre + T, d), 73)
    u = np.array([0.5, -0.25, 1.0, 0.0, 0.125, -1.0, 0.75, 0.5], dtype=np.float32)
    scale = 0.25
    o1, l1 = orc.tree_attn(q, k, v, parent, npre, scale)
    ku = k + u
    assert np.array_equal(ku.astype(np.float64), k.astype(np.float64) + u.astype(np.float64))
    o2, l2 = orc.tree_attn(q, ku, v, parent, npre, scale)
    _close(o1, o2, tol=1e-10, what="O shift")
    shift = scale * (q.astype(np.float64) @ u.astype(np.float64))
    _close(l2, l1 + shift, tol=1e-10, what="LSE shift")


def pin_prefix_permutation(orc):
    """Reordering the committed prefix rows (K and V together) changes nothing."""
    T, Hq, Hkv, d, npre = 13, 2, 2, 8, 30
    parent = wl.kary_tree_parent(T, 3)
    q = _rand((T, Hq, d), 81)
    k = _rand((Hkv, npre + T, d), 82)
    v = _rand((Hkv, npre + T, d), 83)
    perm = np.concatenate([np.random.default_rng(84).permutation(npre), np.arange(npre, npre + T)])
    o1, l1 = orc.tree_attn(q, k, v, parent, npre, 0.35)
    o2, l2 = orc.tree_attn(q, k[:, perm], v[:, perm], parent, npre, 0.35)
    _close(o1, o2, tol=1e-11, what="perm O")
    _close(l1, l2, tol=1e-11, what="perm LSE")


def pin_partial_all_equals_verify(orc):
    """An index list holding every prefix position reproduces full attention."""
    T, Hq, Hkv, d, npre = 13, 4, 2, 8, 40
    parent = wl.kary_tree_parent(T, 3)
    q = _rand((T, Hq, d), 91)
    k = _rand((Hkv, npre + T, d), 92)
    v = _rand((Hkv, npre + T, d), 93)
    o1, l1 = orc.tree_attn(q, k, v, parent, npre, 0.3)
    o2, l2 = orc.tree_attn(q, k, v, parent, npre, 0.3, idx=np.arange(npre, dtype=np.int32))
    _close(o1, o2, tol=0.0, what="partial=all O")
    _close(l1, l2, tol=0.0, what="partial=all LSE")


def pin_partial_equals_compacted_cache(orc):
    """Partial attention over idx equals full attention over a cache that holds
    only the idx rows followed by the tree rows; the initial positions are
    always in idx, as the retained-prefix policy requires."""
    T, Hq, Hkv, d, npre = 4, 4, 2, 16, 300
    parent = wl.chain_parent(T)
    idx = wl.retained_index_set(npre, 40, 8, 7)
    assert list(idx[:8]) == list(range(8))
    q = _rand((T, Hq, d), 101)
    k = _rand((Hkv, npre + T, d), 102)
    v = _rand((Hkv, npre + T, d), 103)
    o1, l1 = orc.tree_attn(q, k, v, parent, npre, 0.25, idx=idx)
    keep = np.concatenate([idx, np.arange(npre, npre + T)])
    o2, l2 = orc.tree_attn(q, k[:, keep], v[:, keep], parent, len(idx), 0.25)
    _close(o1, o2, tol=1e-13, what="compact O")
    _close(l1, l2, tol=1e-13, what="compact LSE")


def pin_single_node_is_decode(orc):
    """T = 1 is single-query decode attention over n_prefix + 1 keys."""
    Hq, Hkv, d, npre = 4, 2, 8, 25
    q = _rand((1, Hq, d), 111)
    k = _rand((Hkv, npre + 1, d), 112)
    v = _rand((Hkv, npre + 1, d), 113)
    o, lse = orc.tree_attn(q, k, v, np.array([-1], dtype=np.int32), npre, 0.4)
    for h in range(Hq):
        g = h // 2
        s = 0.4 * (k[g].astype(np.float64) @ q[0, h].astype(np.float64))
        w = np.exp(s - s.max())
        _close(o[0, h], (w / w.sum()) @ v[g].astype(np.float64), what="decode O")
        _close(lse[0, h], s.max() + math.log(w.sum()), what="decode LSE")


def pin_gqa_equals_repeated_mha(orc):
    """Grouped-query attention equals MHA with each kv head repeated for its
    G consecutive query heads."""
    T, Hq, Hkv, d, npre = 13, 6, 2, 8, 15
    parent = wl.kary_tree_parent(T, 3)
    q = _rand((T, Hq, d), 121)
    k = _rand((Hkv, npre + T, d), 122)
    v = _rand((Hkv, npre + T, d), 123)
    o1, l1 = orc.tree_attn(q, k, v, parent, npre, 0.3)
    G = Hq // Hkv
    kr = np.repeat(k, G, axis=0)
    vr = np.repeat(v, G, axis=0)
    o2, l2 = orc.tree_attn(q, kr, vr, parent, npre, 0.3)
    _close(o1, o2, tol=0.0, what="gqa O")
    _close(l1, l2, tol=0.0, what="gqa LSE")


def pin_bf16_bits_are_exact(orc):
    """bfloat16 inputs are widened exactly: same result as float32 inputs
    holding the same values (torch's bf16 -> f32 conversion)."""
    T, Hq, Hkv, d, npre = 6, 2, 1, 8, 12
    parent = wl.random_tree_parent(T, 2)
    tq = torch.randn(T, Hq, d, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    tk = torch.randn(Hkv, npre + T, d, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    tv = torch.randn(Hkv, npre + T, d, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    o1, l1 = orc.tree_attn(wl.oracle_view(tq), wl.oracle_view(tk), wl.oracle_view(tv),
                           parent, npre, 0.3)
    o2, l2 = orc.tree_attn(tq.float().numpy(), tk.float().numpy(), tv.float().numpy(),
                           parent, npre, 0.3)
    _close(o1, o2, tol=0.0, what="bf16 O")
    _close(l1, l2, tol=0.0, what="bf16 LSE")


def pin_merge_is_split_softmax(orc):
    """Merging softmax attention over disjoint key groups reproduces the full
    softmax (numpy brute force per group and over all keys); an empty group
    (LSE = -inf) contributes nothing."""
    rng = np.random.default_rng(131)
    R, d, n = 5, 6, 40
    s = rng.standard_normal((R, n)) * 3
    vv = rng.standard_normal((n, d))
    cuts = [0, 7, 7, 25, 40]           # third group empty
    po, pl = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if a == b:
            po.append(np.zeros((R, d)))
            pl.append(np.full(R, -np.inf))
            continue
        w = np.exp(s[:, a:b] - s[:, a:b].max(1, keepdims=True))
        po.append((w / w.sum(1, keepdims=True)) @ vv[a:b])
        pl.append(s[:, a:b].max(1) + np.log(w.sum(1)))
    o, lse = orc.lse_merge(np.stack(po), np.stack(pl))
    w = np.exp(s - s.max(1, keepdims=True))
    _close(o, (w / w.sum(1, keepdims=True)) @ vv, what="merge O")
    _close(lse, s.max(1) + np.log(w.sum(1)), what="merge LSE")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
