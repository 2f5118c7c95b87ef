"""Seeded synthetic inputs for tree-verification attention.

This module only produces inputs: tree topologies, Q/K/V tensors and index
lists.  It holds none of the attention arithmetic, so both the GPU path and
the float64 oracle can be fed from it.

Shapes follow the workloads the TokenSwift pages talk about: 1.5B-14B models
with MHA and GQA layouts, caches of about 100K tokens, a 3-ary candidate tree
("From Hours to Minutes ..." arxivlens summary, Technical Contribution), and a
draft pass that sees only a partial KV cache which always keeps the initial
positions ("TokenSwift - A framework for accelerating ..." aiboss88 page,
technical principles, dynamic KV cache update).  No dataset is involved: all
values are N(0, 1) draws from torch generators with fixed seeds.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"

# Four fixed head-dim channels of K are scaled by 8 in the long-context GQA
# workload, standing in for the outlier channels real K caches show.  Scaling
# by a power of two is exact in bfloat16.
OUTLIER_CHANNELS = (0, 32, 64, 96)
OUTLIER_SCALE = 8.0


def kary_tree_parent(n_nodes: int, arity: int = 3) -> np.ndarray:
    """Full k-ary tree numbered breadth-first: parent[i] = (i - 1) // k."""
    p = np.empty(n_nodes, dtype=np.int32)
    p[0] = -1
    for i in range(1, n_nodes):
        p[i] = (i - 1) // arity
    return p


def full_kary_nodes(depth: int, arity: int = 3) -> int:
    """Node count of a full k-ary tree with `depth` levels below the root."""
    return sum(arity ** lv for lv in range(depth + 1))


def chain_parent(n_nodes: int) -> np.ndarray:
    """A single path: node i's parent is i - 1."""
    p = np.arange(-1, n_nodes - 1, dtype=np.int32)
    return p


def random_tree_parent(n_nodes: int, seed: int) -> np.ndarray:
    """A random valid tree: root 0, every later node picks an earlier parent."""
    rng = np.random.default_rng(seed)
    p = np.empty(n_nodes, dtype=np.int32)
    p[0] = -1
    for i in range(1, n_nodes):
        p[i] = rng.integers(0, i)
    return p


def retained_index_set(n_prefix: int, n_idx: int, n_keep: int, seed: int) -> np.ndarray:
    """Sorted distinct positions: 0..n_keep-1 always, plus n_idx - n_keep drawn
    uniformly without replacement from [n_keep, n_prefix)."""
    n_keep = min(n_keep, n_idx, n_prefix)
    rest = n_idx - n_keep
    rng = np.random.default_rng(seed)
    if rest > 0:
        picks = rng.choice(np.arange(n_keep, n_prefix, dtype=np.int64), size=rest, replace=False)
    else:
        picks = np.zeros(0, dtype=np.int64)
    idx = np.concatenate([np.arange(n_keep, dtype=np.int64), np.sort(picks)])
    return idx.astype(np.int32)


@dataclass
class Workload:
    """One attention call's shape and input recipe."""
    name: str
    Hq: int
    Hkv: int
    d: int
    n_prefix: int
    n_nodes: int
    dtype: str
    seed: int
    tree: str = "ternary"          # "ternary" | "chain"
    outliers: bool = False
    n_idx: Optional[int] = None    # partial-KV variant when set
    n_keep: int = 128
    layers: int = 1
    notes: str = field(default="")

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def parent(self) -> np.ndarray:
        if self.tree == "chain":
            return chain_parent(self.n_nodes)
        return kary_tree_parent(self.n_nodes, 3)

    @property
    def cap(self) -> int:
        return self.n_prefix + self.n_nodes

    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def kv_bytes(self) -> int:
        """K+V bytes one layer-call must read (prefix or index set, plus tree rows)."""
        esz = 4 if self.dtype == F32 else 2
        keys = (self.n_idx if self.n_idx is not None else self.n_prefix) + self.n_nodes
        return 2 * self.Hkv * keys * self.d * esz


WORKLOADS = {
    "tiny_mha_f32": Workload("tiny_mha_f32", Hq=4, Hkv=4, d=64, n_prefix=512,
                             n_nodes=full_kary_nodes(2), dtype=F32, seed=1000),
    "gqa8b_8k": Workload("gqa8b_8k", Hq=32, Hkv=8, d=128, n_prefix=8192,
                         n_nodes=full_kary_nodes(3), dtype=BF16, seed=2000),
    "gqa8b_100k": Workload("gqa8b_100k", Hq=32, Hkv=8, d=128, n_prefix=102400,
                           n_nodes=full_kary_nodes(3), dtype=BF16, seed=3000, outliers=True),
    "mha7b_100k": Workload("mha7b_100k", Hq=32, Hkv=32, d=128, n_prefix=102400,
                           n_nodes=full_kary_nodes(3), dtype=BF16, seed=4000),
    "gqa14b_100k": Workload("gqa14b_100k", Hq=40, Hkv=8, d=128, n_prefix=102400,
                            n_nodes=full_kary_nodes(3), dtype=BF16, seed=5000),
    "partial32_gqa8b_100k": Workload("partial32_gqa8b_100k", Hq=32, Hkv=8, d=128,
                                     n_prefix=102400, n_nodes=4, dtype=BF16, seed=6000,
                                     tree="chain", n_idx=4096, n_keep=128, layers=32),
}


@dataclass
class AcceptWorkload:
    """Acceptance of one verified tree and compaction of every layer's cache."""
    name: str
    n_nodes: int
    vocab: int
    logits_dtype: str
    layers: int
    Hkv: int
    d: int
    n_prefix: int
    seed: int
    p_match: float = 0.8
    penalty_window: int = 0      # contextual penalty before the argmax when > 0
    theta: float = 1.0
    n_recent: int = 4096         # committed tokens handed to the penalty

    def parent(self) -> np.ndarray:
        return kary_tree_parent(self.n_nodes, 3)

    def logits_bytes(self) -> int:
        return self.n_nodes * self.vocab * (4 if self.logits_dtype == F32 else 2)


ACCEPT_WORKLOADS = {
    # LLaMA3.1-8B: 128256-token vocabulary, 32 layers, 8 kv heads of 128
    "accept_llama8b": AcceptWorkload("accept_llama8b", n_nodes=full_kary_nodes(3), vocab=128256,
                                     logits_dtype=F32, layers=32, Hkv=8, d=128, n_prefix=102400,
                                     seed=7000),
    # the same step with the contextual penalty first (window and factor
    # assumed: the pages give neither)
    "accept_penalty_llama8b": AcceptWorkload("accept_penalty_llama8b", n_nodes=full_kary_nodes(3), vocab=128256,
                                             logits_dtype=F32, layers=32, Hkv=8, d=128, n_prefix=102400,
                                             seed=7000, penalty_window=1024, theta=1.2),
}


@dataclass
class PagedWorkload:
    """A batch of sequences sharing one tree shape, K/V in pages of a pool.
    With n_idx set it is the draft pass: sequence b reads an index list of
    min(n_idx, length) positions (the first n_keep always among them)."""
    name: str
    lengths: tuple
    Hq: int
    Hkv: int
    d: int
    n_nodes: int
    page_rows: int
    seed: int
    n_idx: Optional[int] = None
    n_keep: int = 128
    tree: str = "kary"

    def parent(self) -> np.ndarray:
        if self.tree == "chain":
            return chain_parent(self.n_nodes)
        return kary_tree_parent(self.n_nodes, 3)

    def pages_needed(self):
        return [-(-(n + self.n_nodes) // self.page_rows) for n in self.lengths]

    def index_lengths(self):
        return [min(self.n_idx, n) for n in self.lengths] if self.n_idx is not None else None

    def kv_bytes(self) -> int:
        """K+V bytes one call reads: every sequence's prefix (or index list)
        plus its tree rows."""
        keys = self.index_lengths() or list(self.lengths)
        return sum(2 * self.Hkv * (n + self.n_nodes) * self.d * 2 for n in keys)


PAGED_WORKLOADS = {
    # eight GQA-8B sequences of different lengths, 102400 committed tokens in
    # all (the headline's KV volume), 16-row pages shuffled in the pool
    "paged_gqa8b_b8": PagedWorkload("paged_gqa8b_b8", lengths=(25600, 19200, 16000, 12800, 9600, 8000,
                                                               6400, 4800),
                                    Hq=32, Hkv=8, d=128, n_nodes=full_kary_nodes(3), page_rows=16,
                                    seed=8000),
    # the draft pass over the same batch: 4096-position partial caches (the
    # first 128 positions kept), four drafted tokens in a chain
    "paged_partial_gqa8b_b8": PagedWorkload("paged_partial_gqa8b_b8",
                                            lengths=(25600, 19200, 16000, 12800, 9600, 8000, 6400, 4800),
                                            Hq=32, Hkv=8, d=128, n_nodes=4, page_rows=16, seed=8100,
                                            n_idx=4096, n_keep=128, tree="chain"),
}


def make_paged_index_lists(w: PagedWorkload, device, seed_offset: int = 0):
    """The draft pass's index lists as one int32 tensor [B, max n_idx], row b
    holding sequence b's sorted list (entries past its length are -1)."""
    lens = w.index_lengths()
    out = np.full((len(lens), max(max(lens), 1)), -1, dtype=np.int32)
    for b, (n, k) in enumerate(zip(w.lengths, lens)):
        out[b, :k] = retained_index_set(n, k, w.n_keep, w.seed + seed_offset + 7919 * (b + 1))
    return torch.from_numpy(out).to(device)


def make_paged_inputs(w: PagedWorkload, device, seed_offset: int = 0):
    """q [B, T, Hq, d], K/V page pools [n_pages, Hkv, page_rows, d] (bf16,
    N(0, 1)), a block table [B, max_pages] over a random permutation of the
    pages; returns (q, k_pages, v_pages, table)."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed + seed_offset)
    need = w.pages_needed()
    n_pages = sum(need)
    shape = (n_pages, w.Hkv, w.page_rows, w.d)
    kp = torch.randn(shape, generator=g, device=device).to(torch.bfloat16)
    vp = torch.randn(shape, generator=g, device=device).to(torch.bfloat16)
    q = torch.randn((len(w.lengths), w.n_nodes, w.Hq, w.d), generator=g, device=device).to(torch.bfloat16)
    perm = np.random.default_rng(w.seed + seed_offset).permutation(n_pages).astype(np.int32)
    table = np.zeros((len(w.lengths), max(need)), dtype=np.int32)
    at = 0
    for b, k in enumerate(need):
        table[b, :k] = perm[at:at + k]
        at += k
    return q, kp, vp, torch.from_numpy(table).to(device)


@dataclass
class SelectWorkload:
    """Importance of every committed position and the draft pass's index list."""
    name: str
    attn: str          # the verification workload whose q, k, lse feed it
    n_keep: int
    n_idx: int
    with_verify: bool = False   # timed together with the verification that feeds it


SELECT_WORKLOADS = {
    "select_gqa8b_100k": SelectWorkload("select_gqa8b_100k", attn="gqa8b_100k", n_keep=128, n_idx=4096),
    "verify_select_gqa8b_100k": SelectWorkload("verify_select_gqa8b_100k", attn="gqa8b_100k", n_keep=128,
                                               n_idx=4096, with_verify=True),
}


def make_accept_inputs(w: AcceptWorkload, device, seed_offset: int = 0):
    """Logits ~ N(0, 1) and draft tokens that repeat the most likely token at
    the parent with probability p_match (else a uniform token)."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed + seed_offset)
    logits = torch.randn((w.n_nodes, w.vocab), generator=g, device=device, dtype=torch.float32)
    if w.logits_dtype == BF16:
        logits = logits.to(torch.bfloat16)
    best = logits.float().argmax(dim=1).cpu().numpy()
    rng = np.random.default_rng(w.seed + seed_offset)
    parent = w.parent()
    draft = rng.integers(0, w.vocab, size=w.n_nodes).astype(np.int32)
    for i in range(1, w.n_nodes):
        if rng.random() < w.p_match:
            draft[i] = best[parent[i]]
    return logits, torch.from_numpy(draft).to(device)


def torch_dtype(dtype: str):
    return torch.float32 if dtype == F32 else torch.bfloat16


def make_qkv(w: Workload, layer: int = 0, device="cpu", seed_offset: int = 0
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Q [T, Hq, d] and K, V [Hkv, n_prefix + T, d] for one layer.

    Values are N(0, 1) float32 draws from a torch generator on `device`
    seeded with seed + 7919 * layer + seed_offset, then rounded to bfloat16
    (round-to-nearest-even) for bf16 workloads.  The same seed on a different
    device gives different (but equally valid) values, so callers must hand
    the oracle the exact tensors they used.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(int(w.seed + 7919 * layer + seed_offset))
    dt = torch_dtype(w.dtype)
    q = torch.randn((w.n_nodes, w.Hq, w.d), generator=gen, device=device, dtype=torch.float32).to(dt)
    k = torch.randn((w.Hkv, w.cap, w.d), generator=gen, device=device, dtype=torch.float32).to(dt)
    v = torch.randn((w.Hkv, w.cap, w.d), generator=gen, device=device, dtype=torch.float32).to(dt)
    if w.outliers:
        for ch in OUTLIER_CHANNELS:
            k[:, :, ch] *= OUTLIER_SCALE
    return q, k, v


def make_index_set(w: Workload, layer: int = 0) -> Optional[np.ndarray]:
    if w.n_idx is None:
        return None
    return retained_index_set(w.n_prefix, w.n_idx, w.n_keep, w.seed + 104729 * (layer + 1))


def oracle_view(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of an input tensor in the form the oracle takes:
    float32 as is, bfloat16 as its raw uint16 bit patterns."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)
