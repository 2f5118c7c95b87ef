"""The contextual-penalty oracle against its pins, and mutated copies of it
(plausible mistakes) that must each fail at least one pin."""
import importlib.util
import os

import pytest

import oracle.penalty as pen
import pins_penalty as P

SRC = pen.__file__


@pytest.mark.parametrize("pin", P.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(pen)


MUTANTS = {
    "window_off_by_one": ("return seq[len(seq) - window:]", "return seq[len(seq) - window + 1:]"),
    "own_token_left_out": ("    x = int(t)\n    while x != 0:", "    x = int(parent[t]) if t else 0\n    while x != 0:"),
    "path_reversed": ("seq = [int(v) for v in recent] + path[::-1]", "seq = [int(v) for v in recent] + path"),
    "committed_ignored": ("seq = [int(v) for v in recent] + path[::-1]", "seq = path[::-1]"),
    "positive_multiplied": ("x[t][v] = l / th if l > 0 else l * th", "x[t][v] = l * th if l > 0 else l / th"),
    "compounds_repeats": ("for v in set(node_window(parent, draft, recent, t, window)):",
                          "for v in node_window(parent, draft, recent, t, window):\n            logits = x"),
    "bf16_truncated": ("r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16", "r = u >> 16"),
    "negative_ids_wrap": ("if not 0 <= v < V:", "if v >= V:"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path = os.path.join(str(tmp_path), "penalty_%s.py" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("penalty_" + name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = False
    for pin in P.PINS:
        try:
            pin(mod)
        except Exception:
            failed = True
            break
    assert failed, "mutant %s passed every pin" % name
