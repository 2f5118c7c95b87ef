"""Pins for the contextual-penalty oracle (oracle/penalty.py): a hand-worked
fixture (with the acceptance that follows), closed forms (theta = 1, empty
window, the sign rule), an independent per-node window built top-down in
node order, once-per-token application, bf16 rounding against torch, and
range handling.  Each pin takes the oracle module (or a mutated copy of it)
and raises on failure.

Page facts used (page title, part): a penalty is applied to recently
generated tokens so that the next token is chosen more diversely --
"TokenSwift - A framework for accelerating ..." (aiboss88), technical
principles, contextual penalty strategy; Tencent Cloud article
"90分钟生成10万Token ...", 上下文惩罚.
"""
import os

import numpy as np
import torch

import oracle.accept as acc
from tree_verification_attention_tsw_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name="penalty_tree_4.txt"):
    kv, rows = {}, {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, val = line.split(":", 1)
        parts = key.split()
        nums = [float(x) for x in val.split()]
        if len(parts) == 2:
            rows.setdefault(parts[0], {})[int(parts[1])] = nums
        else:
            kv[key] = nums
    return kv, rows


def _table(rows, key):
    return np.array([rows[key][i] for i in sorted(rows[key])], dtype=np.float32)


def pin_golden_fixture(pen):
    kv, rows = read_golden()
    parent = [int(x) for x in kv["parent"]]
    draft = [int(x) for x in kv["draft"]]
    recent = [int(x) for x in kv["recent"]]
    W, theta = int(kv["window"][0]), kv["theta"][0]
    logits = _table(rows, "logits")
    for t in range(len(parent)):
        assert pen.node_window(parent, draft, recent, t, W) == [int(x) for x in rows["window"][t]], t
    got = pen.penalize(logits, parent, draft, recent, W, theta)
    assert np.array_equal(got, _table(rows, "penalized")), got
    path, bonus, _ = acc.accept_greedy(parent, got, draft)
    assert path == [int(x) for x in kv["path"]] and bonus == int(kv["bonus"][0]), (path, bonus)
    path, bonus, _ = acc.accept_greedy(parent, logits, draft)
    assert path == [int(x) for x in kv["path_unpenalized"]] and bonus == int(kv["bonus_unpenalized"][0])


def _random_case(T, V, n_recent, seed, dtype=np.float32):
    rng = np.random.default_rng(seed)
    parent = wl.kary_tree_parent(T, 3)
    draft = rng.integers(0, V, T)
    recent = rng.integers(0, V, n_recent)
    logits = rng.standard_normal((T, V)).astype(np.float32)
    logits[:, :3] = [0.0, 1.0, -1.0]                     # exact zero and signs in every row
    return parent, draft, recent, logits


def pin_identity_cases(pen):
    parent, draft, recent, logits = _random_case(13, 50, 20, 1)
    assert np.array_equal(pen.penalize(logits, parent, draft, recent, 8, 1.0), logits)
    assert np.array_equal(pen.penalize(logits, parent, draft, recent, 0, 3.0), logits)
    assert pen.node_window(parent, draft, recent, 5, 0) == []


def pin_sign_rule_and_untouched(pen):
    parent, draft, recent, logits = _random_case(13, 40, 30, 2)
    theta = 1.5
    got = pen.penalize(logits, parent, draft, recent, 6, theta)
    for t in range(13):
        win = set(pen.node_window(parent, draft, recent, t, 6))
        for v in range(40):
            l = np.float32(logits[t][v])
            if v in win:
                want = l / np.float32(theta) if l > 0 else l * np.float32(theta)
            else:
                want = l
            assert got[t][v] == want, (t, v)
        assert np.all(got[t] <= logits[t])                # theta >= 1 never raises a logit


def pin_windows_top_down(pen):
    # sequences built in node order from the parent's (children come after
    # parents): seq[0] = committed tokens, seq[t] = seq[parent[t]] + [draft[t]]
    for T, n_recent, W in ((40, 100, 7), (40, 2, 7), (13, 0, 5), (40, 30, 1), (13, 4, 50)):
        rng = np.random.default_rng(T + n_recent + W)
        parent = wl.kary_tree_parent(T, 3)
        draft = rng.integers(0, 1000, T).tolist()
        recent = rng.integers(0, 1000, n_recent).tolist()
        seqs = [list(recent)]
        for t in range(1, T):
            seqs.append(seqs[parent[t]] + [draft[t]])
        for t in range(T):
            want = seqs[t][-W:] if len(seqs[t]) > W else seqs[t]
            assert pen.node_window(parent, draft, recent, t, W) == want, (T, t)


def pin_once_per_token(pen):
    # a token repeated in the window is penalised once
    parent = [-1, 0]
    logits = np.array([[0, 8, 0, 0], [0, 8, -2, 0]], dtype=np.float32)
    got = pen.penalize(logits, parent, [1, 1], [1, 1, 1, 2], 4, 2.0)
    assert got[0][1] == 4 and got[1][1] == 4 and got[1][2] == -4 and got[0][2] == 0, got


def pin_bf16_rounding(pen):
    # bf16 logits: widened, penalised in float32, rounded to nearest even
    parent, draft, recent, logits = _random_case(13, 64, 40, 3)
    bits = (torch.from_numpy(logits).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    got = pen.penalize(bits, parent, draft, recent, 9, 1.3)
    wide = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    for t in range(13):
        for v in set(pen.node_window(parent, draft, recent, t, 9)):
            x = wide[t][v]
            wide[t][v] = x / 1.3 if x > 0 else x * torch.tensor(1.3, dtype=torch.float32)
    want = wide.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def pin_out_of_range_ignored(pen):
    parent = [-1, 0, 0]
    logits = np.ones((3, 5), dtype=np.float32)
    got = pen.penalize(logits, parent, [0, 7, -1], [9, 2], 3, 2.0)
    # every row's window holds token 2 once among ids 9, 7 and -1 (ignored)
    for t in range(3):
        assert got[t][2] == 0.5 and np.count_nonzero(got[t] != 1) == 1, (t, got[t])


PINS = [pin_golden_fixture, pin_identity_cases, pin_sign_rule_and_untouched, pin_windows_top_down,
        pin_once_per_token, pin_bf16_rounding, pin_out_of_range_ignored]
