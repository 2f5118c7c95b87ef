"""Contextual penalty on the target model's logits at every node of a draft
tree -- TEST INFRASTRUCTURE (plain numpy / Python reference).

What it follows (page title, part):
 * "TokenSwift - A framework for accelerating the generation of ultra-long
   text" (aiboss88), technical principles, contextual penalty strategy: a
   penalty is applied to recently generated tokens so that the next-token
   choice favours more diverse output.
 * Tencent Cloud article "90分钟生成10万Token，新框架实现3倍无损加速超长文本生成",
   上下文惩罚: the generation probabilities are adjusted to suppress repeated
   content.

Readings (the pages give neither the form nor the window):
 * the penalty is the usual repetition penalty with factor theta >= 1: for
   every distinct token v among the last `window` generated tokens, a
   positive logit l[v] becomes l[v] / theta and any other becomes
   l[v] * theta (applied once per token, however often it repeats);
 * "recently generated" for tree node t is what sequential generation would
   have seen before predicting the token after t: the committed tokens (the
   last of them is the tree root, node 0) followed by the draft tokens on
   the path from the root down to t (depth 1 .. depth(t)), of which the last
   `window` count;
 * the arithmetic is that of the logits' type: float32 logits in float32
   (IEEE division and product), bfloat16 logits widened to float32 and the
   result rounded back to bfloat16 (nearest even);
 * token ids outside [0, vocab) are ignored.
"""
import numpy as np


def node_window(parent, draft, recent, t, window):
    """The tokens that count for node t, oldest first."""
    path = []
    x = int(t)
    while x != 0:
        path.append(int(draft[x]))
        x = int(parent[x])
    seq = [int(v) for v in recent] + path[::-1]
    return seq[len(seq) - window:] if 0 < window < len(seq) else (seq if window > 0 else [])


def _bf16_round(x32):
    """float32 -> bfloat16 bit patterns, round to nearest even."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _bf16_widen(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def penalize(logits, parent, draft, recent, window, theta):
    """Penalised copy of logits [T][vocab] (float32, or bfloat16 as uint16 bit
    patterns); the input is not modified."""
    x = np.array(logits, copy=True)
    T, V = x.shape
    th = np.float32(theta)
    for t in range(T):
        for v in set(node_window(parent, draft, recent, t, window)):
            if not 0 <= v < V:
                continue
            if x.dtype == np.uint16:
                l = _bf16_widen(logits[t][v])
                x[t][v] = _bf16_round(l / th if l > 0 else l * th)
            else:
                l = np.float32(logits[t][v])
                x[t][v] = l / th if l > 0 else l * th
    return x
