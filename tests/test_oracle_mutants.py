"""Each plausible mistake planted in a copy of the oracle source must make at
least one pin fail.  The mistakes are planted only in temporary CPU builds of
the oracle; the real oracle is untouched."""
import os

import pytest

import oracle
import pins

# (name, text in tsw_oracle.c, replacement)
MUTANTS = [
    ("self_not_attended", "for (int32_t a = i; a != -1; a = parent[a])",
     "for (int32_t a = parent[i]; a != -1; a = parent[a])"),
    ("gqa_head_modulo", "const int32_t g = h / G;", "const int32_t g = h % (Hq / G);"),
    ("scale_dropped", "s[j] = scale * acc;", "s[j] = acc;"),
    ("lse_without_max", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("lse_log2", "*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    ("tail_rows_own_node", "keys[n++] = n_prefix + anc[a];", "keys[n++] = n_prefix + i;"),
    ("q_layout_head_major", "const int64_t q_off = ((int64_t)i * Hq + h) * d;",
     "const int64_t q_off = ((int64_t)h * (T_) + i) * d;"),
    ("values_from_keys", "o_row[c] += s[j] * load_elem(v, dtype, vr + c);",
     "o_row[c] += s[j] * load_elem(k, dtype, vr + c);"),
    ("index_list_ignored", "keys[n++] = idx ? (int64_t)idx[j] : j;", "keys[n++] = j;"),
    ("mask_bits_by_depth", "m |= (uint64_t)1 << anc[a];", "m |= (uint64_t)1 << a;"),
    ("depth_off_by_one", "if (depth) depth[i] = n - 1;", "if (depth) depth[i] = n;"),
    ("merge_weight_unnormalised", "const double w = exp(ls - L);", "const double w = exp(ls - m);"),
    ("bf16_shift_wrong", "<< 16;", "<< 15;"),
    ("no_normalisation", "o_row[c] /= l;", "o_row[c] /= 1.0;"),
    ("max_nodes_63", "if (T < 1 || T > 64 || !parent || !mask) return ORACLE_EINVAL;",
     "if (T < 1 || T > 63 || !parent || !mask) return ORACLE_EINVAL;"),
]


def _mutant_source(src, old, new):
    assert src.count(old) >= 1, old
    out = src.replace(old, new)
    if "T_" in new:
        # head-major Q needs T inside attend_row: pass it through a global
        out = out.replace("static void attend_row(", "static int32_t T_;\nstatic void attend_row(")
        out = out.replace("const int32_t G = Hq / Hkv;", "const int32_t G = Hq / Hkv;\n    T_ = T;")
    return out


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    with open(oracle.SRC) as f:
        src = f.read()
    msrc = tmp_path / ("mutant_%s.c" % name)
    msrc.write_text(_mutant_source(src, old, new))
    lib = oracle.compile_oracle(str(msrc), str(tmp_path / ("libmutant_%s.so" % name)))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except Exception:  # noqa: BLE001 -- any failure counts as caught
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
