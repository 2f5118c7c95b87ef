"""Pins for the importance / selection oracle (oracle/select.py): closed
forms (K = 0), the probability-mass identity, an explicit per-head softmax,
GQA = repeated MHA, and selection checked by hand and by brute-force sorting.
Each pin takes the oracle module (or a mutated copy) and raises on failure.

Page facts used (page title, part): the initial KV positions are always kept
and the rest of the cache is kept by importance -- "TokenSwift - A framework
for accelerating ..." (aiboss88), technical principles, dynamic KV cache
update.
"""
import numpy as np
import torch

import oracle
from tree_verification_attention_tsw_amd import workloads as wl


def _case(T, Hq, Hkv, d, n_prefix, seed, zero_k=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, Hq, d)).astype(np.float32)
    k = rng.standard_normal((Hkv, n_prefix + T, d)).astype(np.float32)
    v = rng.standard_normal((Hkv, n_prefix + T, d)).astype(np.float32)
    if zero_k:
        k[:] = 0.0
    parent = wl.kary_tree_parent(T, 3)
    scale = 1.0 / np.sqrt(d)
    _, lse = oracle.tree_attn(q, k, v, parent, n_prefix, scale)
    return q, k, lse, scale


def pin_zero_k(sel):
    # all scores 0: the root spreads each head's unit mass evenly over
    # n_prefix + 1 positions (prefix plus itself)
    for Hq, Hkv, n in ((4, 4, 50), (8, 2, 129)):
        q, k, lse, scale = _case(5, Hq, Hkv, 16, n, 1, zero_k=True)
        imp = sel.importance(q, k, lse, n, scale)
        assert np.allclose(imp, Hq / (n + 1), rtol=0, atol=1e-12), imp[:4]


def pin_mass_identity(sel):
    # per head the root's weights over prefix + itself sum to 1
    q, k, lse, scale = _case(13, 8, 2, 32, 300, 2)
    imp = sel.importance(q, k, lse, 300, scale)
    G = 4
    self_w = sum(np.exp(scale * float(q[0, h].astype(np.float64) @ k[h // G, 300].astype(np.float64))
                        - lse[0, h]) for h in range(8))
    assert abs(imp.sum() - (8 - self_w)) < 1e-10, (imp.sum(), 8 - self_w)


def pin_explicit_softmax(sel):
    q, k, lse, scale = _case(4, 6, 3, 8, 37, 3)
    G = 2
    want = np.zeros(37)
    for h in range(6):
        keys = torch.from_numpy(np.concatenate([k[h // G, :37], k[h // G, 37:38]]).astype(np.float64))
        s = scale * (keys @ torch.from_numpy(q[0, h].astype(np.float64)))
        want += torch.softmax(s, dim=0).numpy()[:37]
    got = sel.importance(q, k, lse, 37, scale)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


def pin_gqa_is_repeated_mha(sel):
    q, k, lse, scale = _case(4, 8, 2, 16, 60, 4)
    krep = np.repeat(k, 4, axis=0)
    assert np.allclose(sel.importance(q, k, lse, 60, scale), sel.importance(q, krep, lse, 60, scale),
                       rtol=1e-13, atol=0)


def pin_select_by_hand(sel):
    imp = np.array([5, 1, 9, 9, 2, 7, 0, 3], dtype=np.float64)
    assert sel.select(imp, 8, 2, 5).tolist() == [0, 1, 2, 3, 5]
    # equal importance at the cut: the lower positions win
    imp = np.array([0, 0, 4, 1, 4, 4, 1, 4], dtype=np.float64)
    assert sel.select(imp, 8, 1, 3).tolist() == [0, 2, 4]
    assert sel.select(imp, 8, 3, 3).tolist() == [0, 1, 2]
    assert sel.select(imp, 8, 0, 8).tolist() == list(range(8))
    assert sel.select(imp, 8, 2, 20).tolist() == list(range(8))


def pin_select_brute(sel):
    rng = np.random.default_rng(5)
    for trial in range(40):
        n = int(rng.integers(1, 300))
        imp = rng.integers(0, 6, size=n).astype(np.float64)      # many ties
        n_keep = int(rng.integers(0, n + 1))
        n_idx = int(rng.integers(0, n + 5))
        got = sel.select(imp, n, n_keep, n_idx).tolist()
        keep = list(range(min(n_keep, n, n_idx)))
        rest = sorted(range(len(keep), n), key=lambda p: (-imp[p], p))[:max(0, n_idx - len(keep))]
        assert got == keep + sorted(rest), (trial, got[:10])


PINS = [pin_zero_k, pin_mass_identity, pin_explicit_softmax, pin_gqa_is_repeated_mha, pin_select_by_hand,
        pin_select_brute]
