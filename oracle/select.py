"""Importance of committed KV positions and selection of the partial cache
for the draft pass -- TEST INFRASTRUCTURE (plain numpy reference).

What it follows (page title, part):
 * "TokenSwift - A framework for accelerating the generation of ultra-long
   text" (aiboss88), technical principles, dynamic KV cache update: the
   initial part of the KV cache is kept and the rest of the cache is ordered
   by importance, the most important entries being kept.
 * Tencent Cloud article "90分钟生成10万Token，新框架实现3倍无损加速超长文本生成",
   无损的输出质量 / 技术原理: the draft model is the target model running on a
   partial KV cache.

Readings (the pages name importance but do not define it):
 * importance of committed position p = the attention mass the tree root's
   query heads (node 0, the last committed token, as seen in the
   verification pass) put on p: sum over query heads h of
   exp(scale * q[0][h] . k[g(h)][p] - LSE[0][h]), with LSE the root row's
   log-sum-exp from the verification pass (prefix plus the root itself).
 * selection: positions 0 .. n_keep-1 always; then the n_idx - n_keep most
   important of the remaining positions (equal importance: the lower
   position first); the list is sorted ascending.
"""
import numpy as np


def _widen(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def importance(q, k, lse, n_prefix, scale):
    """q [T][Hq][d], k [Hkv][rows][d] (float32 or bf16 bits), lse [T][Hq]
    (natural log, the verification pass's); returns float64 [n_prefix]."""
    q, k = _widen(q), _widen(k)
    lse = np.asarray(lse, dtype=np.float64)
    Hq, Hkv = q.shape[1], k.shape[0]
    G = Hq // Hkv
    imp = np.zeros(n_prefix, dtype=np.float64)
    for h in range(Hq):
        s = scale * (k[h // G, :n_prefix] @ q[0, h])
        imp += np.exp(s - lse[0, h])
    return imp


def select(imp, n_prefix, n_keep, n_idx):
    """Sorted int32 index list: [0, n_keep) plus the most important others."""
    n_keep = min(n_keep, n_prefix, n_idx)
    rest = n_idx - n_keep
    cand = np.arange(n_keep, n_prefix)
    if rest >= len(cand):
        chosen = cand
    else:
        order = np.lexsort((cand, -np.asarray(imp, dtype=np.float64)[n_keep:n_prefix]))
        chosen = np.sort(cand[order[:rest]])
    return np.concatenate([np.arange(n_keep), chosen]).astype(np.int32)
