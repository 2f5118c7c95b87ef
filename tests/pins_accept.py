"""Pins for the acceptance / compaction oracle (oracle/accept.py): a
hand-worked fixture, brute force over every root-to-node path with an
independent first-maximum routine, closed-form special cases and invariants.
Each pin takes the oracle module (or a mutated copy of it) and raises on
failure.

Page facts used (page title, part): the longest valid candidate is kept and
the result must agree with the target model's own predictions --
"TokenSwift - A framework for accelerating ..." (aiboss88), technical
principles, tree-based multi-candidate token verification; Tencent Cloud
article "90分钟生成10万Token ...", 技术原理 (parallel verification).
"""
import os

import numpy as np

from tree_verification_attention_tsw_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name="accept_tree_13.txt"):
    kv = {}
    logits = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, val = line.split(":", 1)
        nums = [int(x) for x in val.split()]
        if key.startswith("logits "):
            logits[int(key.split()[1])] = nums
        else:
            kv[key] = nums
    T = len(kv["parent"])
    kv["logits"] = np.array([logits[i] for i in range(T)], dtype=np.float32)
    return kv


def first_max(row):
    """Index of the first maximum, by an explicit scan."""
    best = 0
    for j in range(1, len(row)):
        if row[j] > row[best]:
            best = j
    return best


def brute_force(parent, logits, draft):
    """Every node whose whole root path agrees, then the deepest (lowest index)."""
    T = len(parent)
    x = np.asarray(logits, dtype=np.float64)
    best, best_len = 0, 1
    for node in range(T):
        path = [node]
        while path[-1] != 0:
            path.append(int(parent[path[-1]]))
        path.reverse()
        ok = all(int(draft[path[k]]) == first_max(x[path[k - 1]]) for k in range(1, len(path)))
        if ok and len(path) > best_len:
            best, best_len = node, len(path)
    path = [best]
    while path[-1] != 0:
        path.append(int(parent[path[-1]]))
    return path[::-1], first_max(x[best])


def pin_golden_13(acc):
    g = read_golden()
    path, bonus, target = acc.accept_greedy(g["parent"], g["logits"], g["draft"])
    assert list(target) == g["targets"], target
    assert list(path) == g["path"], path
    assert bonus == g["bonus"][0], bonus


def pin_golden_compact(acc):
    g = read_golden()
    n_prefix = g["compact_n_prefix"][0]
    rows = n_prefix + len(g["parent"])
    cache = np.stack([np.arange(rows), 100 + np.arange(rows)], axis=1).astype(np.float32)[None]
    out = acc.kv_compact(cache, n_prefix, g["path"])
    assert out[0, :, 0].astype(int).tolist() == g["compact_rows_after"]
    assert np.array_equal(out[0, :, 1], 100 + out[0, :, 0])


def _planted(T, V, seed, tree="random", p_match=0.7):
    rng = np.random.default_rng(seed)
    parent = wl.random_tree_parent(T, seed) if tree == "random" else (
        wl.kary_tree_parent(T, 3) if tree == "ternary" else wl.chain_parent(T))
    logits = rng.integers(-4, 5, size=(T, V)).astype(np.float32)   # small ints: many ties
    draft = rng.integers(0, V, size=T)
    for i in range(1, T):
        if rng.random() < p_match:
            draft[i] = first_max(logits[int(parent[i])])
    return parent, logits, draft


def pin_brute_force(acc):
    for seed in range(60):
        T = 1 + seed % 23
        parent, logits, draft = _planted(T, 7, seed, tree=("random", "ternary", "chain")[seed % 3])
        path, bonus, _ = acc.accept_greedy(parent, logits, draft)
        bp, bb = brute_force(parent, logits, draft)
        assert list(path) == bp and bonus == bb, (seed, path, bp, bonus, bb)


def pin_no_match(acc):
    parent, logits, _ = _planted(13, 5, 3, tree="ternary")
    logits[:, 4] = -100.0            # token 4 is never the most likely
    draft = np.full(13, 4)
    path, bonus, _ = acc.accept_greedy(parent, logits, draft)
    assert list(path) == [0] and bonus == first_max(logits[0])


def pin_chain_all_match(acc):
    T = 17
    parent = wl.chain_parent(T)
    logits = np.random.default_rng(4).standard_normal((T, 50)).astype(np.float32)
    draft = [0] + [first_max(logits[i - 1]) for i in range(1, T)]
    path, bonus, _ = acc.accept_greedy(parent, logits, draft)
    assert list(path) == list(range(T)) and bonus == first_max(logits[T - 1])


def pin_longer_path_beats_lower_index(acc):
    # siblings 1 and 2 both carry the root's most likely token; only node 2's
    # child (node 4) agrees further down
    parent = np.array([-1, 0, 0, 1, 2], dtype=np.int32)
    logits = np.zeros((5, 4), dtype=np.float32)
    logits[0, 3] = 1.0               # target after root: 3
    logits[1, 0] = 1.0               # after node 1: 0
    logits[2, 2] = 1.0               # after node 2: 2
    logits[4, 1] = 1.0
    draft = [0, 3, 3, 1, 2]          # node 3 (child of 1) disagrees, node 4 agrees
    path, bonus, _ = acc.accept_greedy(parent, logits, draft)
    assert list(path) == [0, 2, 4] and bonus == 1, (path, bonus)
    # equal depth: the lower index wins
    draft = [0, 3, 3, 1, 1]
    path, _, _ = acc.accept_greedy(parent, logits, draft)
    assert list(path) == [0, 1], path


def pin_bf16_logits(acc):
    # bfloat16 bit patterns decide exactly as their float32 values; two values
    # that round to the same bfloat16 tie, and the first index wins
    x = np.array([[1.0, 3.0, 3.015625, 2.0]], dtype=np.float32)    # all bf16-exact
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert acc.target_tokens(bits) == [2]
    y = np.array([[1.0, 3.0, 3.0, 2.0]], dtype=np.float32)
    assert acc.target_tokens((y.view(np.uint32) >> 16).astype(np.uint16)) == [1]
    parent, logits, draft = _planted(20, 9, 11, tree="ternary")
    lb = (logits.view(np.uint32) >> 16).astype(np.uint16)          # small ints: exact in bf16
    assert acc.accept_greedy(parent, lb, draft)[:2] == acc.accept_greedy(parent, logits, draft)[:2]


def pin_compact_overlap(acc):
    # path [0, 2, 5]: row n+2 is both a source (node 2) and a destination
    n = 3
    rows = n + 8
    cache = np.random.default_rng(2).standard_normal((2, rows, 4)).astype(np.float32)
    out = acc.kv_compact(cache, n, [0, 2, 5])
    assert np.array_equal(out[:, n + 1], cache[:, n + 2])
    assert np.array_equal(out[:, n + 2], cache[:, n + 5])
    keep = [r for r in range(rows) if r not in (n + 1, n + 2)]
    assert np.array_equal(out[:, keep], cache[:, keep])


def pin_compact_identity(acc):
    cache = np.random.default_rng(3).standard_normal((3, 20, 5)).astype(np.float32)
    assert np.array_equal(acc.kv_compact(cache, 7, [0, 1, 2, 3]), cache)


PINS = [pin_golden_13, pin_golden_compact, pin_brute_force, pin_no_match, pin_chain_all_match,
        pin_longer_path_beats_lower_index, pin_bf16_logits, pin_compact_overlap,
        pin_compact_identity]
