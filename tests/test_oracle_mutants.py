"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle.c with one plausible error (a wrong mask
alignment, an index off by one, a dropped term, a swapped operand...), built
on the CPU into a temporary directory.  The test asserts that at least one
quick pin fails for every mutant, so the pins are strong enough to trust the
oracle they pin.
"""
from pathlib import Path

import pytest

import oracle
import oracle_pins as P

SRC = Path(oracle.__file__).resolve().parent / "oracle.c"

MUTANTS = {
    "top_left_causal": ("const int32_t n_vis = (lk - lq) + i + 1;",
                        "const int32_t n_vis = i + 1;"),
    "visible_off_by_one": ("const int32_t n_vis = (lk - lq) + i + 1;",
                           "const int32_t n_vis = (lk - lq) + i + (i == 0 ? 1 : 0);"),
    "visibility_count_wrong": ("for (int32_t i = 0; i < lq; ++i) n_vis[cu[b] + i] = (lk - lq) + i + 1;",
                               "for (int32_t i = 0; i < lq; ++i) n_vis[cu[b] + i] = (lk - lq) + i;"),
    "page_offset_swapped": ("size_t page = (size_t)row[pos / page_size];",
                            "size_t page = (size_t)row[(pos % page_size) % ((pos / page_size) + 1)];"),
    "offset_dropped": ("size_t off = (size_t)(pos % page_size);", "size_t off = 0;"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "k_read_from_v": ("dot += load_elem(q, q0 + d, dtype) * load_elem(k_cache, kidx, dtype);",
                      "dot += load_elem(q, q0 + d, dtype) * load_elem(v_cache, kidx, dtype);"),
    "gqa_head_map": ("const int32_t kvh = h / group;", "const int32_t kvh = h % num_kv_heads;"),
    "normalise_by_count": ("for (int32_t d = 0; d < head_dim; ++d) out[q0 + d] = acc[d] / l;",
                           "for (int32_t d = 0; d < head_dim; ++d) out[q0 + d] = acc[d] / n_vis;"),
    "exp_base_two": ("double wgt = exp(s[j] - m);", "double wgt = exp2(s[j] - m);"),
    "weights_not_exponentiated": ("double wgt = exp(s[j] - m);", "double wgt = 1.0 + (s[j] - m);"),
    "q_row_transposed": ("const size_t q0 = ((size_t)r * num_heads + h) * head_dim;",
                         "const size_t q0 = ((size_t)h * total + r) * head_dim;"),
    "append_neighbour_slot": ("size_t dst = (size_t)s * row_elems + e;",
                              "size_t dst = (size_t)(s ^ 1) * row_elems + e;"),
    "append_value_into_k": ("memcpy((char*)k_cache + dst * es, (const char*)key + src * es, es);",
                            "memcpy((char*)k_cache + dst * es, (const char*)value + src * es, es);"),
    "slot_position_unshifted": ("int32_t pos = (lk - lq) + i;", "int32_t pos = i;"),
    "last_key_dropped": ("for (int32_t j = 0; j < n_vis; ++j) {\n        double wgt",
                         "for (int32_t j = 0; j + 1 < n_vis || j == 0; ++j) {\n        double wgt"),
}


@pytest.fixture(scope="module")
def source():
    return SRC.read_text()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutant anchor for {name} no longer matches oracle.c"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(source.replace(old, new))
    lib = oracle.build(src=mutated, out=tmp_path / "liboracle_mutant.so")
    orc = oracle.Oracle(lib)
    failures = []
    for pin in P.QUICK_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:  # a pin caught the planted mistake
            failures.append((getattr(pin, "__name__", "pin"), str(e)[:80]))
    assert failures, f"no pin catches the planted mistake '{name}'"
