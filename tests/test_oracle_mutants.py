"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/oracle.c`` to a temporary directory, replaces one
exact fragment with a plausible mistake (a dropped term, a wrong sign, index or
bound, a swapped operand), builds it, and runs the pin battery of
``oracle_pins.py`` against it.  At least one pin must fail for every mistake;
if none does, the pins do not constrain that part of the oracle.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = {
    "head_map_modulo": ("int g = h / G;\n    int n = c->seqlens",
                        "int g = h % c->H_kv;\n    int n = c->seqlens"),
    "prefill_head_map_modulo": ("int g = h / G;\n    const uint16_t *qrow",
                                "int g = h % c->H_kv;\n    const uint16_t *qrow"),
    "scale_dropped": ("s[j] = tau * dot;", "s[j] = dot;"),
    "no_normalisation": ("double p = exp(s[j] - m) / l;", "double p = exp(s[j] - m);"),
    "lse_without_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "scores_from_v": ("const uint16_t *kj = k + (size_t)j * kv_stride;",
                      "const uint16_t *kj = v + (size_t)j * kv_stride;"),
    "causal_excludes_diagonal": ("i + 1, c->d, c->tau", "i, c->d, c->tau"),
    "causal_one_extra_key": ("i + 1, c->d, c->tau", "(i + 2 < c->S ? i + 2 : c->S), c->d, c->tau"),
    "kv_row_stride_wrong": ("attend_row(c->q + (size_t)r * c->d, k0, v0, (size_t)c->H_kv * c->d",
                            "attend_row(c->q + (size_t)r * c->d, k0, v0, (size_t)c->d"),
    "max_pass_min": ("        if (s[j] > m) m = s[j];\n    /* pass 2",
                     "        if (s[j] < m || m == -INFINITY) m = s[j];\n    /* pass 2"),
    "merge_alpha_sign": ("double a = exp(mr[p] - M);", "double a = exp(M - mr[p]);"),
    "merge_no_divide": ("for (int x = 0; x < d; ++x) out[x] /= L;", ""),
    "merge_lse_drops_max": ("lse_out[r] = M + log(L);", "lse_out[r] = log(L);"),
    "partial_l_not_shifted": ("double e = exp(s[j] - m);\n        l += e;",
                              "double e = exp(s[j] - m);\n        l += exp(s[j]);"),
    "partial_wrong_start": ("(((size_t)b * c->S_max + c->j0) * c->H_kv + g) * c->d;\n    const uint16_t *v0",
                            "(((size_t)b * c->S_max) * c->H_kv + g) * c->d;\n    const uint16_t *v0"),
    "q_widening_offset": ("for (int c = 0; c < d; ++c) qd[c] = bf16_to_double(q[c]);",
                          "for (int c = 0; c < d; ++c) qd[c] = bf16_to_double(q[(c + 1) % d]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(oracle.SOURCE).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"anchor for {name} must occur exactly once"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(str(path), str(tmp_path / "liboracle_mutant.so")))
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects the planted mistake {name}"
