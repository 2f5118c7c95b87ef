"""Greedy acceptance of a verified draft tree and compaction of the accepted
path's K/V rows -- TEST INFRASTRUCTURE (plain numpy / Python reference).

What it follows (page title, part):
 * "TokenSwift - A framework for accelerating the generation of ultra-long
   text" (aiboss88), technical principles, tree-based multi-candidate token
   verification: the candidate combinations in the tree are verified in
   parallel and the longest valid n-gram becomes the output, so that the
   result stays consistent with the target model's own predictions.
 * Tencent Cloud article "90分钟生成10万Token，新框架实现3倍无损加速超长文本生成",
   技术原理 (parallel verification figure text): the candidates are checked
   by the model with the full KV cache and the longest valid sequence is kept.

Readings (where the pages leave a step open):
 * "valid" = greedy agreement: node i (i > 0) is accepted when its parent is
   accepted and its draft token equals the target model's most likely next
   token at the parent (argmax of the parent's logits; the first index among
   equal maxima).  The root (node 0) is the already-committed token and is
   always accepted.
 * among accepted nodes of the greatest depth the lowest node index wins (one
   page picks randomly among equally long candidates, the other just takes
   the longest; with distinct sibling tokens there is never a tie).
 * the "bonus" token is the target's argmax at the last accepted node: the
   token the target model itself emits after the accepted path.
 * compaction: the tree's K/V rows sit at cache positions n_prefix + node;
   the accepted path's rows move to n_prefix, n_prefix + 1, ... in path
   order, and the committed length becomes n_prefix + len(path).
"""
import numpy as np


def widen_logits(logits):
    """float64 copy of float32 logits or of bfloat16 bit patterns (uint16); exact."""
    x = np.asarray(logits)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def target_tokens(logits):
    """Most likely next token at every node (first index among equal maxima)."""
    x = widen_logits(logits)
    return [int(np.argmax(x[i])) for i in range(x.shape[0])]


def accepted_nodes(parent, draft, target):
    """Accepted flag per node, in node order (parents come before children)."""
    T = len(parent)
    acc = [False] * T
    acc[0] = True
    for i in range(1, T):
        p = int(parent[i])
        acc[i] = acc[p] and int(draft[i]) == target[p]
    return acc


def depths(parent):
    d = [0] * len(parent)
    for i in range(1, len(parent)):
        d[i] = d[int(parent[i])] + 1
    return d


def root_path(parent, node):
    path = [node]
    while path[-1] != 0:
        path.append(int(parent[path[-1]]))
    return path[::-1]


def accept_greedy(parent, logits, draft):
    """(path, bonus token, per-node target tokens)."""
    target = target_tokens(logits)
    acc = accepted_nodes(parent, draft, target)
    dep = depths(parent)
    best = 0
    for i in range(len(parent)):
        if acc[i] and dep[i] > dep[best]:
            best = i
    path = root_path(parent, best)
    return path, target[best], target


def kv_compact(cache, n_prefix, path):
    """Cache [..., rows, d] (any leading dims): a copy with the accepted path's
    rows moved to n_prefix + 0, 1, ...; every other row unchanged."""
    out = np.array(cache, copy=True)
    for k, node in enumerate(path):
        out[..., n_prefix + k, :] = cache[..., n_prefix + node, :]
    return out
