"""The acceptance / compaction oracle against its pins, and mutated copies of
it (plausible mistakes) that must each fail at least one pin."""
import importlib.util
import os
import sys

import pytest

import oracle.accept as acc
import pins_accept as P

SRC = acc.__file__


@pytest.mark.parametrize("pin", P.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(acc)


MUTANTS = {
    "compares_own_logits": ("acc[i] = acc[p] and int(draft[i]) == target[p]",
                            "acc[i] = acc[p] and int(draft[i]) == target[i]"),
    "ignores_parent": ("acc[i] = acc[p] and int(draft[i]) == target[p]",
                       "acc[i] = int(draft[i]) == target[p]"),
    "last_max_wins": ("return [int(np.argmax(x[i])) for i in range(x.shape[0])]",
                      "return [int(x.shape[1] - 1 - np.argmax(x[i][::-1])) for i in range(x.shape[0])]"),
    "highest_index_wins": ("if acc[i] and dep[i] > dep[best]:", "if acc[i] and dep[i] >= dep[best]:"),
    "bonus_from_parent": ("return path, target[best], target",
                          "return path, target[int(parent[best])] if best else target[0], target"),
    "compact_reverse_in_place": ("    for k, node in enumerate(path):\n        out[..., n_prefix + k, :] = cache[..., n_prefix + node, :]",
                                 "    for k, node in reversed(list(enumerate(path))):\n        out[..., n_prefix + k, :] = out[..., n_prefix + node, :]"),
    "compact_no_offset": ("out[..., n_prefix + k, :] = cache[..., n_prefix + node, :]",
                          "out[..., k, :] = cache[..., n_prefix + node, :]"),
    "bf16_wrong_shift": ("(x.astype(np.uint32) << 16)", "(x.astype(np.uint32) << 15)"),
}


def _load_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path = os.path.join(str(tmp_path), "accept_%s.py" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("accept_" + name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    mod = _load_mutant(name, *MUTANTS[name], tmp_path)
    failed = []
    for pin in P.PINS:
        try:
            pin(mod)
        except Exception:
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
