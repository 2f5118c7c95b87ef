"""The importance / selection oracle against its pins, and mutated copies of
it that must each fail at least one pin."""
import importlib.util
import os

import pytest

import oracle.select as sel
import pins_select as P

SRC = sel.__file__


@pytest.mark.parametrize("pin", P.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(sel)


MUTANTS = {
    "kv_head_by_modulo": ("s = scale * (k[h // G, :n_prefix] @ q[0, h])",
                          "s = scale * (k[h % Hkv, :n_prefix] @ q[0, h])"),
    "no_lse": ("imp += np.exp(s - lse[0, h])", "imp += np.exp(s)"),
    "unscaled": ("s = scale * (k[h // G, :n_prefix] @ q[0, h])", "s = (k[h // G, :n_prefix] @ q[0, h])"),
    "last_node_query": ("@ q[0, h])", "@ q[-1, h])"),
    "ties_high_position": ("order = np.lexsort((cand, -np.asarray(imp, dtype=np.float64)[n_keep:n_prefix]))",
                           "order = np.lexsort((-cand, -np.asarray(imp, dtype=np.float64)[n_keep:n_prefix]))"),
    "unsorted": ("chosen = np.sort(cand[order[:rest]])", "chosen = cand[order[:rest]]"),
    "keep_ignored": ("n_keep = min(n_keep, n_prefix, n_idx)", "n_keep = 0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path = os.path.join(str(tmp_path), "select_%s.py" % name)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("select_" + name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in P.PINS:
        try:
            pin(mod)
        except Exception:
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
