"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/oracle.c`` to a temporary directory, replaces one
exact fragment with a plausible mistake (a dropped term, a wrong sign, index or
bound, a swapped operand), builds it, and runs the pin battery of
``oracle_pins.py`` against it.  At least one pin must fail for every mistake;
if none does, the pins do not constrain that part of the oracle.
"""
import os

import numpy as np
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
    "causal_excludes_diagonal": ("pos + 1, c->d, c->tau", "pos, c->d, c->tau"),
    "causal_one_extra_key": ("pos + 1, c->d, c->tau",
                             "(pos + 2 < c->S_kv ? pos + 2 : c->S_kv), c->d, c->tau"),
    "chunk_start_ignored": ("int pos = c->q_start + i;", "int pos = i;"),
    "chunk_aligned_to_cache_end": ("int pos = c->q_start + i;", "int pos = c->S_kv - c->T + i;"),
    "chunk_q_stride_from_keys": ("(((size_t)b * c->T + i) * c->H_q + h)",
                                 "(((size_t)b * c->S_kv + i) * c->H_q + h)"),
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
    "bwd_D_dropped": ("double ds = s[j] * (dp[j] - D);", "double ds = s[j] * dp[j];"),
    "bwd_dq_without_scale": ("for (int x = 0; x < d; ++x) dq[x] *= c->tau;", ""),
    "bwd_dp_from_k": ("dpj += dod[x] * bf16_to_double(vj[x]);",
                      "dpj += dod[x] * bf16_to_double(kj[x]);"),
    "bwd_rows_exclude_diagonal": ("int n = i + 1;                  /* keys 0 .. i */",
                                  "int n = i;"),
    "bwd_dk_from_k": ("dk[x] += c->tau * ds * bf16_to_double(c->q[qoff + x]);",
                      "dk[x] += c->tau * ds * kd[x];"),
    "bwd_dv_weighted_by_ds": ("dv[x] += pij * bf16_to_double(c->dout[qoff + x]);",
                              "dv[x] += ds * bf16_to_double(c->dout[qoff + x]);"),
    "bwd_keys_head_map_modulo": ("for (int h = g * G; h < (g + 1) * G; ++h) {",
                                 "for (int h = g; h < c->H_q; h += c->H_kv) {"),
    "bwd_keys_skip_diagonal_row": ("for (int i = j; i < c->S; ++i) {", "for (int i = j + 1; i < c->S; ++i) {"),
    "bwd_keys_lse_of_key_row": ("double pij = exp(c->tau * dot - lse[i]);",
                                "double pij = exp(c->tau * dot - lse[j]);"),
    "bwd_keys_D_of_key_row": ("double ds = pij * (dpij - D[i]);", "double ds = pij * (dpij - D[j]);"),
    "bwd_stored_D_ignored": ("    if (c->D_in) D = c->D_in[r];", ""),
    "fp8_ties_to_odd": ("((lo & 1) == 0 ? lo : hi)", "((lo & 1) == 1 ? lo : hi)"),
    "fp8_subnormal_step": ("ldexp((double)man, -9)", "ldexp((double)man, -10)"),
    "fp8_exponent_bias_8": ("ldexp(1.0 + man / 8.0, ex - 7)", "ldexp(1.0 + man / 8.0, ex - 8)"),
    "fp8_encode_drops_sign": ("    return sign | c;\n}", "    return c;\n}"),
    "fp8_scale_not_minimal": ("while (e < 127 && amax > ldexp(448.0, e)) ++e;",
                              "while (e < 127 && amax >= ldexp(448.0, e)) ++e;"),
    "fp8_scale_one_binade_low": ("while (e < 127 && amax > ldexp(448.0, e)) ++e;",
                                 "while (e < 127 && amax > ldexp(896.0, e)) ++e;"),
    "fp8_quantise_without_scale": ("oracle_e4m3_encode(ldexp(bf16_to_double(row[i]), -e))",
                                   "oracle_e4m3_encode(bf16_to_double(row[i]))"),
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


# Planted mistakes in the paged-cache gather (Python): the token-to-page map of
# V07 section 16 with a swapped or shifted index must also fail a pin.
def _gather_variant(kind):
    def gather(pool, block_table, seqlens, page_size):
        B, max_blocks = block_table.shape
        out = np.zeros((B, max_blocks * page_size) + pool.shape[2:], dtype=pool.dtype)
        for b in range(B):
            t = np.arange(int(seqlens[b]))
            if kind == "swapped":
                blk, row = t % page_size % max_blocks, t // page_size % page_size
            elif kind == "row_shift":
                blk, row = t // page_size, (t + 1) % page_size
            else:   # "table_of_first_sequence"
                blk, row = t // page_size, t % page_size
                out[b, :t.size] = pool[np.maximum(block_table[0, blk], 0), row]
                continue
            out[b, :t.size] = pool[np.maximum(block_table[b, blk], 0), row]
        return out
    return gather


@pytest.mark.parametrize("kind", ["swapped", "row_shift", "table_of_first_sequence"])
def test_planted_gather_mistake_is_caught(kind, monkeypatch, oracle_lib):
    monkeypatch.setattr(oracle, "gather_pages", _gather_variant(kind))
    caught = []
    for pin in PINS:
        try:
            pin(oracle_lib)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects the gather mistake {kind}"


# Planted mistakes in the FP8 page layout (Python): V07 section 17.7 appends a page's
# per-token scales after its rows; scales written first, or rows at the wrong stride, must
# fail a pin.
def _pages_variant(kind):
    real = oracle.quantize_to_pages

    def quantize_to_pages(x, seqlens, block_table, page_size, num_pages, fill=0, lib=None):
        pool = real(x, seqlens, block_table, page_size, num_pages, fill=fill, lib=lib)
        B, S_max, H_kv, d = x.shape
        data = page_size * H_kv * d
        if kind == "scales_first":
            return np.concatenate([pool[:, data:], pool[:, :data]], axis=1)
        rows = pool[:, :data].reshape(num_pages, page_size, H_kv * d)
        return np.concatenate([np.roll(rows, 1, axis=1).reshape(num_pages, data), pool[:, data:]],
                              axis=1)
    return quantize_to_pages


@pytest.mark.parametrize("kind", ["scales_first", "row_stride"])
def test_planted_fp8_page_mistake_is_caught(kind, monkeypatch, oracle_lib):
    monkeypatch.setattr(oracle, "quantize_to_pages", _pages_variant(kind))
    caught = []
    for pin in PINS:
        try:
            pin(oracle_lib)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects the FP8 page mistake {kind}"


# Planted mistakes in the stored-output D (Python; V07 section 6.2: D_i = dO_i . O_i): the
# rows in token-major order instead of (b, h, i), or the output dotted with itself, must fail
# a pin.
def _stored_D_variant(kind):
    def stored_output_D(o, do):
        o64 = oracle._f32_of_bits(o).astype(np.float64)
        do64 = oracle._f32_of_bits(do).astype(np.float64)
        if kind == "token_major_rows":
            return np.einsum("bshd,bshd->bsh", o64, do64)
        return np.einsum("bshd,bshd->bhs", o64, o64)
    return stored_output_D


@pytest.mark.parametrize("kind", ["token_major_rows", "o_for_both_factors"])
def test_planted_stored_D_mistake_is_caught(kind, monkeypatch, oracle_lib):
    monkeypatch.setattr(oracle, "stored_output_D", _stored_D_variant(kind))
    caught = []
    for pin in PINS:
        try:
            pin(oracle_lib)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects the stored-D mistake {kind}"
