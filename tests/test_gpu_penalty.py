"""GPU parity of the contextual penalty (through the C ABI) against the numpy
oracle: the penalised logits bit-exact (float32 and bfloat16, float32
arithmetic in both), every other logit untouched, and greedy acceptance on
the penalised logits equal to the oracle's."""
import sys

import numpy as np
import pytest
import torch

import oracle.accept as acc
import oracle.penalty as pen
import pins_penalty as P
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


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).cuda()


def run(parent, logits_np, draft, recent, window, theta, dtype):
    """Penalise on the GPU and in the oracle; returns (GPU logits as oracle input
    type, oracle logits, the GPU tensor)."""
    lt = torch.from_numpy(np.ascontiguousarray(logits_np, dtype=np.float32)).cuda()
    if dtype == "bf16":
        lt = lt.to(torch.bfloat16)
        ref_in = lt.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        ref_in = np.asarray(logits_np, dtype=np.float32)
    tsw.context_penalty(parent, lt, i32(draft), i32(recent), window, theta)
    torch.cuda.synchronize()
    got = lt.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else lt.cpu().numpy()
    want = pen.penalize(ref_in, parent, draft, recent, window, theta)
    return got, want, lt


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_golden_fixture(dtype):
    kv, rows = P.read_golden()
    parent = [int(x) for x in kv["parent"]]
    draft = [int(x) for x in kv["draft"]]
    recent = [int(x) for x in kv["recent"]]
    logits = P._table(rows, "logits")
    got, want, lt = run(parent, logits, draft, recent, int(kv["window"][0]), kv["theta"][0], dtype)
    assert np.array_equal(got, want)
    res = tsw.accept_greedy(parent, lt, i32(draft)).cpu().numpy()
    assert res[0] == len(kv["path"]) and res[1] == int(kv["bonus"][0])
    assert list(res[2:2 + int(res[0])]) == [int(x) for x in kv["path"]]


@pytest.mark.parametrize("T,vocab,n_recent,window,theta,dtype", [
    (40, 128256, 5000, 1024, 1.2, "f32"),
    (40, 128256, 5000, 1024, 1.2, "bf16"),
    (40, 151936, 300, 8192, 1.7, "f32"),      # window longer than what exists
    (13, 32000, 64, 1, 3.0, "bf16"),          # only the newest token
    (64, 5000, 10000, 700, 1.05, "f32"),      # dense repeats in a small vocabulary
    (1, 128256, 2048, 2048, 1.3, "f32"),      # plain decode
])
def test_penalty_matches_oracle(T, vocab, n_recent, window, theta, dtype):
    rng = np.random.default_rng(T + vocab + window)
    parent = wl.kary_tree_parent(T, 3)
    draft = rng.integers(0, vocab, T)
    recent = rng.integers(0, vocab, n_recent)
    logits = rng.standard_normal((T, vocab)).astype(np.float32) * 4
    logits[:, :2] = 0.0
    got, want, _ = run(parent, logits, draft, recent, window, theta, dtype)
    say("penalty T=%d vocab=%d n_recent=%d window=%d theta=%g %s" % (T, vocab, n_recent, window, theta, dtype))
    assert np.array_equal(got, want)


def test_out_of_range_and_repeats():
    parent = wl.kary_tree_parent(13, 3)
    vocab = 1000
    draft = [5] * 13
    draft[4] = -3
    draft[7] = 1000
    recent = [5, 5, 2000, -1, 9, 5]
    logits = np.random.default_rng(4).standard_normal((13, vocab)).astype(np.float32)
    got, want, _ = run(parent, logits, draft, recent, 6, 2.0, "f32")
    assert np.array_equal(got, want)


def test_penalty_then_accept_matches_oracle():
    w = wl.ACCEPT_WORKLOADS["accept_llama8b"]
    T, vocab = w.n_nodes, w.vocab
    rng = np.random.default_rng(9)
    parent = w.parent()
    logits = rng.standard_normal((T, vocab)).astype(np.float32)
    # draft tokens that follow the unpenalised argmax, some of them recent, so
    # the penalty changes which nodes are accepted
    best = logits.argmax(axis=1)
    draft = np.array([best[parent[i]] if i else 0 for i in range(T)])
    recent = np.concatenate([rng.integers(0, vocab, 500), best[:6]])
    got, want, lt = run(parent, logits, draft, recent, 256, 1.5, "f32")
    assert np.array_equal(got, want)
    res = tsw.accept_greedy(parent, lt, i32(draft)).cpu().numpy()
    path, bonus, target = acc.accept_greedy(parent, want, draft)
    say("penalty+accept: path %s bonus %d" % (path, bonus))
    assert res[0] == len(path) and res[1] == bonus and list(res[2:2 + len(path)]) == list(path)
    assert list(res[2 + T:2 + 2 * T]) == list(target)


@pytest.mark.parametrize("T,vocab,n_recent,window,theta,dtype", [
    (40, 128256, 5000, 1024, 1.2, "f32"),
    (40, 128256, 5000, 1024, 1.2, "bf16"),
    (40, 151936, 300, 8192, 1.7, "f32"),
    (13, 5001, 64, 40, 3.0, "f32"),           # unaligned rows: the scalar scan
    (13, 5001, 64, 40, 3.0, "bf16"),
    (64, 2000, 10000, 700, 1.05, "bf16"),     # dense repeats, small vocabulary
    (1, 128256, 2048, 2048, 1.3, "f32"),
])
def test_penalized_acceptance_matches_oracle(T, vocab, n_recent, window, theta, dtype):
    """Acceptance with the penalty folded into the argmax: the oracle's
    acceptance on the oracle's penalised logits, the logits left unchanged,
    and the same result as the in-place penalty followed by acceptance."""
    rng = np.random.default_rng(T * 7 + vocab + window)
    parent = wl.kary_tree_parent(T, 3)
    logits = rng.standard_normal((T, vocab)).astype(np.float32) * 3
    best = logits.argmax(axis=1)
    draft = np.array([best[parent[i]] if i else 0 for i in range(T)])
    recent = np.concatenate([rng.integers(0, vocab, n_recent - 8), best[:8] if T >= 8 else rng.integers(0, vocab, 8)])
    recent[::97] = -5                                  # ignored ids
    lt = torch.from_numpy(logits).cuda()
    if dtype == "bf16":
        lt = lt.to(torch.bfloat16)
        ref_in = lt.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        ref_in = logits
    before = lt.clone()
    res = tsw.accept_greedy_penalized(parent, lt, i32(draft), i32(recent), window, theta).cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(lt.view(torch.int16) if dtype == "bf16" else lt,
                       before.view(torch.int16) if dtype == "bf16" else before)
    want_logits = pen.penalize(ref_in, parent, draft, recent, window, theta)
    path, bonus, target = acc.accept_greedy(parent, want_logits, draft)
    say("penalized accept T=%d vocab=%d window=%d %s: path %s bonus %d" % (T, vocab, window, dtype, path, bonus))
    assert res[0] == len(path) and res[1] == bonus and list(res[2:2 + len(path)]) == list(path)
    assert list(res[2 + T:2 + 2 * T]) == list(target)
    tsw.context_penalty(parent, lt, i32(draft), i32(recent), window, theta)
    res2 = tsw.accept_greedy(parent, lt, i32(draft)).cpu().numpy()
    assert np.array_equal(res, res2)


@pytest.mark.parametrize("case", range(16))
def test_penalty_random_shapes(case):
    """Seeded random shapes: tree (random, chain, 3-ary), vocabulary size
    (odd sizes included), window 0 .. 8192, theta (1 included), recent
    tokens (none included), ids out of range; the in-place penalty
    bit-exact, and the penalised acceptance equal to the oracle's acceptance
    on the oracle's penalised logits, with the logits left unchanged."""
    rng = np.random.default_rng(9500 + case)
    T = int(rng.choice([1, 2, 13, 40, 64]) if rng.random() < 0.4 else rng.integers(1, 65))
    kind = rng.integers(3)
    parent = (wl.random_tree_parent(T, 9500 + case) if kind == 0 else
              wl.chain_parent(T) if kind == 1 else wl.kary_tree_parent(T, 3))
    vocab = int(rng.choice([2, 7, 1000, 5001, 32000, 128256, 151936]) if rng.random() < 0.5
                else rng.integers(2, 200001))
    window = int(rng.choice([0, 1, 40, 8192]) if rng.random() < 0.3 else rng.integers(0, 8193))
    theta = float(1.0 if rng.random() < 0.15 else np.float32(rng.uniform(1.0, 3.0)))
    n_recent = int(rng.choice([0, 1, 8]) if rng.random() < 0.2 else rng.integers(0, 10001))
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    logits = (rng.standard_normal((T, vocab)) * 3).astype(np.float32)
    best = logits.argmax(axis=1)
    draft = rng.integers(0, vocab, T)
    for i in range(1, T):
        if rng.random() < 0.7:
            draft[i] = best[parent[i]]
    recent = rng.integers(0, vocab, n_recent)
    if n_recent:
        recent[-min(n_recent, 8):] = best[:min(n_recent, 8)] if T >= 8 else recent[-min(n_recent, 8):]
        recent[rng.random(n_recent) < 0.01] = -3
        recent[rng.random(n_recent) < 0.01] = vocab + 5
    if T > 1 and rng.random() < 0.3:
        draft[rng.integers(1, T)] = vocab
    say("penalty random case %d: T=%d vocab=%d window=%d theta=%.4f n_recent=%d %s" % (
        case, T, vocab, window, theta, n_recent, dtype))
    got, want, _ = run(parent, logits, draft, recent, window, theta, dtype)
    assert np.array_equal(got, want)
    lt = torch.from_numpy(logits).cuda()
    if dtype == "bf16":
        lt = lt.to(torch.bfloat16)
        ref_in = lt.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        ref_in = logits
    before = lt.clone()
    res = tsw.accept_greedy_penalized(parent, lt, i32(draft), i32(recent), window, theta).cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(lt.view(torch.int16) if dtype == "bf16" else lt,
                       before.view(torch.int16) if dtype == "bf16" else before)
    path, bonus, target = acc.accept_greedy(parent, pen.penalize(ref_in, parent, draft, recent, window, theta),
                                            draft)
    say("  path %s bonus %d" % (list(path), bonus))
    assert res[0] == len(path) and res[1] == bonus and list(res[2:2 + len(path)]) == list(path)
    assert list(res[2 + T:2 + 2 * T]) == list(target)
