"""Pins for the fp64 oracle: checks against what the definitions and the pages fix.

Each pin is a function ``pin_*(lib)`` that raises AssertionError when the
oracle library ``lib`` disagrees with a closed form, an invariant, a special
case, or a brute-force evaluation built on library routines (scipy's softmax
and logsumexp, ``math.fsum``).  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on copies of ``oracle.c`` with a
planted mistake and requires that some pin fails for every such mistake.
"""
import json
import math
import os

import numpy as np
from scipy.special import logsumexp, softmax

import oracle
from gqa_workloads.generate import bf16_bits_from_f32, chunk_inputs, decode_inputs, \
    f32_from_bf16_bits, paged_decode_inputs, prefill_bwd_inputs, prefill_inputs

BF16_ONE = 0x3F80


def _f64(bits):
    return f32_from_bf16_bits(bits).astype(np.float64)


def _fsum_dot(a, b):
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


def _brute_row(qrow, K, V, tau):
    """Library-routine evaluation of one attention row (exact dot products via fsum)."""
    s = np.array([tau * _fsum_dot(qrow, K[j]) for j in range(K.shape[0])])
    p = softmax(s)
    o = np.array([math.fsum(p[j] * V[j, c] for j in range(K.shape[0])) for c in range(V.shape[1])])
    return o, float(logsumexp(s))


def _rel_close(a, b, rtol, atol=0.0):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.isfinite(a) == np.isfinite(b)), "finiteness differs"
    fin = np.isfinite(b)
    err = np.abs(a[fin] - b[fin])
    bound = atol + rtol * np.maximum(np.abs(b[fin]), 1e-300)
    assert np.all(err <= bound), f"max err {err.max() if err.size else 0} (rtol {rtol})"
    assert np.array_equal(a[~fin], b[~fin]), "non-finite values differ"


# ---------------------------------------------------------------------------
# Softmax normalisation (V07 section 2, safe softmax): with V = identity rows the
# output row IS the probability vector, so it must be non-negative and sum to 1.

def pin_softmax_rows_sum_to_one(lib):
    rng = np.random.default_rng(7)
    B, H_q, H_kv, d, S = 2, 4, 2, 32, 20
    q = bf16_bits_from_f32(rng.standard_normal((B, H_q, d)).astype(np.float32) * 2)
    k = bf16_bits_from_f32(rng.standard_normal((B, S, H_kv, d)).astype(np.float32))
    v = np.zeros((B, S, H_kv, d), dtype=np.uint16)
    for j in range(S):
        v[:, j, :, j] = BF16_ONE
    o, _ = oracle.decode(q, k, v, lib=lib)
    assert np.all(o >= 0.0)
    assert np.all(o[..., S:] == 0.0)
    assert np.max(np.abs(o.sum(axis=-1) - 1.0)) <= 1e-12
    # the probabilities must also be the softmax of the score row (brute force)
    for b in range(B):
        for h in range(H_q):
            g = h // (H_q // H_kv)
            s = np.array([_fsum_dot(_f64(q[b, h]), _f64(k[b, j, g])) for j in range(S)])
            p = softmax(s / math.sqrt(d))
            _rel_close(o[b, h, :S], p, 1e-12, 1e-15)


# ---------------------------------------------------------------------------
# Brute force on tiny inputs, decode and causal prefill.

def pin_brute_force_decode(lib):
    inp = decode_inputs(2, 4, 2, 8, ragged=(1, 13), seed=11)
    q, k, v, sl = inp["q"], inp["k"], inp["v"], inp["seqlens"]
    o, lse = oracle.decode(q, k, v, sl, lib=lib)
    tau = 1.0 / math.sqrt(8)
    for b in range(2):
        for h in range(4):
            g = h // 2
            n = int(sl[b])
            ob, lb = _brute_row(_f64(q[b, h]), _f64(k[b, :n, g]), _f64(v[b, :n, g]), tau)
            _rel_close(o[b, h], ob, 1e-12, 1e-14)
            assert abs(lse[b, h] - lb) <= 1e-13 * max(1.0, abs(lb))


def pin_brute_force_prefill(lib):
    B, S, H_q, H_kv, d = 1, 9, 4, 2, 16
    inp = prefill_inputs(B, S, H_q, H_kv, d, seed=12)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o, lse = oracle.prefill_causal(q, k, v, lib=lib)
    tau = 1.0 / math.sqrt(d)
    for h in range(H_q):
        g = h // (H_q // H_kv)
        for i in range(S):
            ob, lb = _brute_row(_f64(q[0, i, h]), _f64(k[0, :i + 1, g]), _f64(v[0, :i + 1, g]), tau)
            _rel_close(o[0, i, h], ob, 1e-12, 1e-14)
            assert abs(lse[0, h, i] - lb) <= 1e-13 * max(1.0, abs(lb))


# ---------------------------------------------------------------------------
# Merge associativity (V07 section 3): the merged states of ANY partition of the
# keys -- uneven, singleton and empty chunks included -- equal the unsplit result.

def pin_split_merge_equals_unsplit(lib):
    inp = decode_inputs(1, 8, 2, 32, S_max=96, seed=13)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o_full, lse_full = oracle.decode(q, k, v, lib=lib)
    rng = np.random.default_rng(5)
    for trial in range(6):
        ncut = rng.integers(1, 9)
        cuts = np.sort(rng.integers(0, 97, size=ncut))
        bounds = [0, *cuts.tolist(), 96]
        if trial == 0:
            bounds = [0, 0, 1, 1, 50, 96, 96]          # empty, singleton, empty, ..., empty
        parts = [oracle.decode_partial(q, k, v, a, b, lib=lib) for a, b in zip(bounds, bounds[1:])]
        m = np.stack([p[0].reshape(-1) for p in parts], axis=1)
        l = np.stack([p[1].reshape(-1) for p in parts], axis=1)
        ob = np.stack([p[2].reshape(-1, 32) for p in parts], axis=1)
        if trial % 2:
            perm = rng.permutation(m.shape[1])        # commutativity: any order of partials
            m, l, ob = m[:, perm], l[:, perm], ob[:, perm]
        o_m, lse_m = oracle.merge_states(m, l, ob, lib=lib)
        _rel_close(o_m, o_full.reshape(-1, 32), 1e-12, 1e-14)
        _rel_close(lse_m, lse_full.reshape(-1), 1e-13)


def pin_merge_identity_and_empty(lib):
    inp = decode_inputs(1, 4, 1, 16, S_max=10, seed=14)
    q, k, v = inp["q"], inp["k"], inp["v"]
    m, l, o = oracle.decode_partial(q, k, v, 0, 10, lib=lib)
    me, le, oe = oracle.decode_partial(q, k, v, 4, 4, lib=lib)
    assert np.all(me == -np.inf) and np.all(le == 0.0) and np.all(oe == 0.0)
    # merging with the identity state (-inf, 0, 0) leaves the result unchanged, exactly
    o1, lse1 = oracle.merge_states(m.reshape(-1, 1), l.reshape(-1, 1), o.reshape(-1, 1, 16), lib=lib)
    o2, lse2 = oracle.merge_states(np.stack([m.reshape(-1), me.reshape(-1)], 1),
                                   np.stack([l.reshape(-1), le.reshape(-1)], 1),
                                   np.stack([o.reshape(-1, 16), oe.reshape(-1, 16)], 1), lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(lse1, lse2)
    # a single state normalises to O/l and lse = m + ln l
    _rel_close(o1, (o / l[..., None]).reshape(-1, 16), 1e-15, 1e-300)
    _rel_close(lse1, (m + np.log(l)).reshape(-1), 1e-15)
    # all partials empty -> O = 0, lse = -inf
    o3, lse3 = oracle.merge_states(np.full((2, 3), -np.inf), np.zeros((2, 3)),
                                   np.zeros((2, 3, 16)), lib=lib)
    assert np.all(o3 == 0.0) and np.all(lse3 == -np.inf)
    # decode with the full state equals the normalised partial
    o_full, lse_full = oracle.decode(q, k, v, lib=lib)
    _rel_close(o1, o_full.reshape(-1, 16), 1e-13, 1e-15)
    _rel_close(lse1, lse_full.reshape(-1), 1e-14)


# ---------------------------------------------------------------------------
# GQA head map (V07 section 14): query head h reads KV head floor(h / G).  G = 1
# is plain multi-head attention, so GQA must equal MHA on K/V repeated G times
# per head (the materialised broadcast of ADR-0061, rejected for the kernels
# but a valid definition to test against).

def pin_gqa_equals_mha_on_repeated_kv(lib):
    inp = decode_inputs(2, 8, 2, 16, S_max=24, seed=15)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o_g, lse_g = oracle.decode(q, k, v, lib=lib)
    k_rep = np.repeat(k, 4, axis=2)
    v_rep = np.repeat(v, 4, axis=2)
    o_m, lse_m = oracle.decode(q, k_rep, v_rep, lib=lib)
    assert np.array_equal(o_g, o_m) and np.array_equal(lse_g, lse_m)
    # the modulo map (h mod H_kv) is a different function on these inputs
    o_t, _ = oracle.decode(q, np.tile(k, (1, 1, 4, 1)), np.tile(v, (1, 1, 4, 1)), lib=lib)
    assert not np.allclose(o_t, o_g)
    # same for causal prefill
    pin = prefill_inputs(1, 12, 8, 2, 16, seed=16)
    o_pg, l_pg = oracle.prefill_causal(pin["q"], pin["k"], pin["v"], lib=lib)
    o_pm, l_pm = oracle.prefill_causal(pin["q"], np.repeat(pin["k"], 4, axis=2),
                                       np.repeat(pin["v"], 4, axis=2), lib=lib)
    assert np.array_equal(o_pg, o_pm) and np.array_equal(l_pg, l_pm)


# ---------------------------------------------------------------------------
# Closed forms derived from the definition.

def pin_identical_keys_give_mean_of_v(lib):
    rng = np.random.default_rng(17)
    B, H_q, H_kv, d, S = 1, 4, 2, 32, 37
    q = bf16_bits_from_f32(rng.standard_normal((B, H_q, d)).astype(np.float32))
    krow = bf16_bits_from_f32(rng.standard_normal((H_kv, d)).astype(np.float32))
    k = np.broadcast_to(krow, (B, S, H_kv, d)).copy()
    v = bf16_bits_from_f32(rng.standard_normal((B, S, H_kv, d)).astype(np.float32))
    o, lse = oracle.decode(q, k, v, lib=lib)
    for h in range(H_q):
        g = h // 2
        mean = np.array([math.fsum(_f64(v[0, :, g, c])) / S for c in range(d)])
        _rel_close(o[0, h], mean, 1e-13, 1e-15)
        s = _fsum_dot(_f64(q[0, h]), _f64(krow[g])) / math.sqrt(d)
        assert abs(lse[0, h] - (s + math.log(S))) <= 1e-13 * max(1.0, abs(s) + math.log(S))


def pin_zero_scale_gives_mean_and_log_n(lib):
    inp = decode_inputs(1, 4, 2, 16, S_max=29, seed=18)
    o, lse = oracle.decode(inp["q"], inp["k"], inp["v"], tau=0.0, lib=lib)
    v = _f64(inp["v"])
    for h in range(4):
        mean = v[0, :, h // 2].mean(axis=0)
        _rel_close(o[0, h], mean, 1e-13, 1e-15)
        assert abs(lse[0, h] - math.log(29)) <= 1e-14


def pin_single_key(lib):
    inp = decode_inputs(1, 4, 2, 32, S_max=5, seed=19)
    sl = np.array([1], dtype=np.int32)
    o, lse = oracle.decode(inp["q"], inp["k"], inp["v"], sl, lib=lib)
    for h in range(4):
        g = h // 2
        assert np.array_equal(o[0, h], _f64(inp["v"][0, 0, g]))
        s = _fsum_dot(_f64(inp["q"][0, h]), _f64(inp["k"][0, 0, g])) / math.sqrt(32)
        assert abs(lse[0, h] - s) <= 1e-14 * max(1.0, abs(s))


def pin_two_keys_sigmoid(lib):
    inp = decode_inputs(1, 2, 1, 16, S_max=2, seed=20)
    o, lse = oracle.decode(inp["q"], inp["k"], inp["v"], lib=lib)
    q, k, v = _f64(inp["q"]), _f64(inp["k"]), _f64(inp["v"])
    for h in range(2):
        s0 = _fsum_dot(q[0, h], k[0, 0, 0]) / 4.0
        s1 = _fsum_dot(q[0, h], k[0, 1, 0]) / 4.0
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        _rel_close(o[0, h], w0 * v[0, 0, 0] + w1 * v[0, 1, 0], 1e-13, 1e-15)
        assert abs(lse[0, h] - np.logaddexp(s0, s1)) <= 1e-14 * max(1.0, abs(lse[0, h]))


def pin_safe_softmax_survives_huge_logits(lib):
    """V07 section 2: the unshifted exponential overflows (fp32 beyond x > 88, fp64
    beyond ~709); the max-shifted form stays finite.  With logits thousands apart the
    softmax is one-hot on the largest score, so O is that key's V row exactly and
    LSE is that score."""
    d, S = 32, 6
    q = bf16_bits_from_f32(np.full((1, 1, d), 64.0, dtype=np.float32))
    levels = np.array([1.0, -2.0, 4.0, 3.0, -4.0, 0.5], dtype=np.float32)
    k = bf16_bits_from_f32(np.broadcast_to(levels[:, None], (S, d)).reshape(1, S, 1, d).copy())
    v = bf16_bits_from_f32(
        np.random.default_rng(26).standard_normal((1, S, 1, d)).astype(np.float32))
    o, lse = oracle.decode(q, k, v, lib=lib)
    s = 64.0 * levels.astype(np.float64) * d / math.sqrt(d)      # exact: spread > 1000
    j = int(np.argmax(s))
    assert np.array_equal(o[0, 0], _f64(v[0, j, 0]))
    assert abs(lse[0, 0] - s[j]) <= 1e-12 * abs(s[j])


def pin_empty_sequence(lib):
    inp = decode_inputs(2, 4, 2, 16, S_max=6, seed=21)
    sl = np.array([0, 6], dtype=np.int32)
    o, lse = oracle.decode(inp["q"], inp["k"], inp["v"], sl, lib=lib)
    assert np.all(o[0] == 0.0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(o[1])) and np.all(np.isfinite(lse[1]))


def pin_ragged_tail_never_read(lib):
    inp = decode_inputs(3, 4, 2, 16, ragged=(3, 17), seed=22, nan_fill=True)
    o, lse = oracle.decode(inp["q"], inp["k"], inp["v"], inp["seqlens"], lib=lib)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    # truncating each sequence's cache to its own length gives the same rows
    for b in range(3):
        n = int(inp["seqlens"][b])
        ob, lb = oracle.decode(inp["q"][b:b + 1], inp["k"][b:b + 1, :n].copy(),
                               inp["v"][b:b + 1, :n].copy(), lib=lib)
        assert np.array_equal(ob[0], o[b]) and np.array_equal(lb[0], lse[b])


def pin_key_permutation_invariance(lib):
    inp = decode_inputs(1, 4, 2, 32, S_max=40, seed=23)
    o, lse = oracle.decode(inp["q"], inp["k"], inp["v"], lib=lib)
    perm = np.random.default_rng(3).permutation(40)
    o_p, lse_p = oracle.decode(inp["q"], inp["k"][:, perm].copy(), inp["v"][:, perm].copy(),
                               lib=lib)
    _rel_close(o_p, o, 1e-13, 1e-15)
    _rel_close(lse_p, lse, 1e-14)
    # but permuting only V changes the result (K and V must stay paired)
    o_v, _ = oracle.decode(inp["q"], inp["k"], inp["v"][:, perm].copy(), lib=lib)
    assert not np.allclose(o_v, o)


# ---------------------------------------------------------------------------
# Causal prefill (V07 section 12): row i sees keys 0..i, the diagonal included.

def pin_causal_row0_and_bounds(lib):
    B, S, H_q, H_kv, d = 1, 16, 4, 2, 32
    inp = prefill_inputs(B, S, H_q, H_kv, d, seed=24)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o, lse = oracle.prefill_causal(q, k, v, lib=lib)
    for h in range(H_q):
        g = h // 2
        assert np.array_equal(o[0, 0, h], _f64(v[0, 0, g]))          # row 0: O = v_0 exactly
        s00 = _fsum_dot(_f64(q[0, 0, h]), _f64(k[0, 0, g])) / math.sqrt(d)
        assert abs(lse[0, h, 0] - s00) <= 1e-14 * max(1.0, abs(s00))
    # the future never matters: change keys/values after row 7, rows 0..7 unchanged
    k2, v2 = k.copy(), v.copy()
    k2[:, 8:] = bf16_bits_from_f32(np.full(k2[:, 8:].shape, 3.0, dtype=np.float32))
    v2[:, 8:] = bf16_bits_from_f32(np.full(v2[:, 8:].shape, -5.0, dtype=np.float32))
    o2, lse2 = oracle.prefill_causal(q, k2, v2, lib=lib)
    assert np.array_equal(o2[:, :8], o[:, :8]) and np.array_equal(lse2[..., :8], lse[..., :8])
    # ...but the diagonal key does: row 8 changes
    assert not np.allclose(o2[:, 8], o[:, 8])


def pin_prefill_row_equals_decode(lib):
    B, S, H_q, H_kv, d = 1, 13, 4, 2, 16
    inp = prefill_inputs(B, S, H_q, H_kv, d, seed=25)
    q, k, v = inp["q"], inp["k"], inp["v"]
    rows = np.array([[0, h, i] for h in range(H_q) for i in (0, 5, 12)], dtype=np.int32)
    o, lse = oracle.prefill_causal_rows(q, k, v, rows, lib=lib)
    for r, (_, h, i) in enumerate(rows):
        od, ld = oracle.decode(q[:, i].copy(), k, v, np.array([i + 1], dtype=np.int32), lib=lib)
        assert np.array_equal(o[r], od[0, h]) and lse[r] == ld[0, h]


# ---------------------------------------------------------------------------
# Chunked causal prefill (ADR-0060 sections 0.5.2 and 5.4: a query block of T_q
# rows starting at q_start against the cached keys; V07 section 12: causal).

def pin_chunk_whole_prompt_is_causal_prefill(lib):
    inp = prefill_inputs(2, 11, 4, 2, 16, seed=27)
    o, lse = oracle.prefill_causal(inp["q"], inp["k"], inp["v"], lib=lib)
    oc, lc = oracle.prefill_chunk(inp["q"], inp["k"], inp["v"], q_start=0, lib=lib)
    assert np.array_equal(o, oc) and np.array_equal(lse, lc)


def pin_chunk_rows_are_rows_of_full_prefill(lib):
    """Running a prompt's rows [q_start, q_start + T) as one chunk against the whole
    cache gives exactly those rows of the whole-prompt causal prefill, wherever the
    chunk sits; cache rows past the chunk's last token are never visible."""
    B, S, H_q, H_kv, d = 2, 23, 4, 2, 16
    inp = prefill_inputs(B, S, H_q, H_kv, d, seed=28)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o, lse = oracle.prefill_causal(q, k, v, lib=lib)
    for q_start, T in ((0, 5), (7, 9), (15, 8), (22, 1)):
        qc = q[:, q_start:q_start + T].copy()
        # the cache past the chunk's end holds NaN: a read of it would show
        kc, vc = k.copy(), v.copy()
        kc[:, q_start + T:] = 0x7FC0
        vc[:, q_start + T:] = 0x7FC0
        oc, lc = oracle.prefill_chunk(qc, kc, vc, q_start=q_start, lib=lib)
        assert np.array_equal(oc, o[:, q_start:q_start + T])
        assert np.array_equal(lc, lse[..., q_start:q_start + T])
        # the default alignment is bottom-right: the chunk is the cache's last T tokens
        ob, lb = oracle.prefill_chunk(qc, k[:, :q_start + T].copy(), v[:, :q_start + T].copy(),
                                      lib=lib)
        assert np.array_equal(ob, oc) and np.array_equal(lb, lc)


def pin_chunk_single_row_is_decode(lib):
    B, S, H_q, H_kv, d = 2, 19, 8, 2, 32
    inp = prefill_inputs(B, S, H_q, H_kv, d, seed=29)
    q1 = inp["q"][:, -1:].copy()
    oc, lc = oracle.prefill_chunk(q1, inp["k"], inp["v"], lib=lib)
    od, ld = oracle.decode(q1[:, 0].copy(), inp["k"], inp["v"], lib=lib)
    assert np.array_equal(oc[:, 0], od) and np.array_equal(lc[..., 0], ld)


def pin_brute_force_chunk(lib):
    B, T, S_kv, H_q, H_kv, d = 1, 4, 10, 4, 2, 8
    inp = chunk_inputs(B, T, S_kv, H_q, H_kv, d, seed=30)
    q, k, v = inp["q"], inp["k"], inp["v"]
    for q_start in (6, 3):
        o, lse = oracle.prefill_chunk(q, k, v, q_start=q_start, lib=lib)
        for h in range(H_q):
            g = h // 2
            for i in range(T):
                n = q_start + i + 1
                ob, lb = _brute_row(_f64(q[0, i, h]), _f64(k[0, :n, g]), _f64(v[0, :n, g]),
                                    1.0 / math.sqrt(d))
                _rel_close(o[0, i, h], ob, 1e-12, 1e-14)
                assert abs(lse[0, h, i] - lb) <= 1e-13 * max(1.0, abs(lb))


# ---------------------------------------------------------------------------
# Paged KV cache (V07 section 16: token t of a request is row t mod B_p of page
# block_table[req][t div B_p]; section 17: the decode kernel reads through it).

def pin_paged_equals_contiguous(lib):
    """A paged cache holding the same token rows, in randomly permuted pages with
    NaN in every unused slot and -1 past each table's last block, gives exactly the
    contiguous result, for page sizes that do and do not divide the lengths."""
    for page in (16, 32, 48):
        a = decode_inputs(3, 8, 2, 32, ragged=(1, 90), seed=31)
        p = paged_decode_inputs(3, 8, 2, 32, page, ragged=(1, 90), seed=31)
        o, lse = oracle.decode(a["q"], a["k"], a["v"], a["seqlens"], lib=lib)
        op, lp = oracle.decode_paged(p["q"], p["k_pool"], p["v_pool"], p["block_table"],
                                     p["seqlens"], page, lib=lib)
        assert np.array_equal(o, op) and np.array_equal(lse, lp)


def pin_paged_identity_table(lib):
    """Pages laid out in order (table[b][i] = b * blocks + i) are the contiguous cache."""
    B, S, H_kv, d, page = 2, 64, 2, 16, 16
    inp = decode_inputs(B, 4, H_kv, d, S_max=S, seed=32)
    nb = S // page
    pool_k = inp["k"].reshape(B * nb, page, H_kv, d)
    pool_v = inp["v"].reshape(B * nb, page, H_kv, d)
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    sl = np.array([S, 37], dtype=np.int32)
    o, lse = oracle.decode(inp["q"], inp["k"], inp["v"], sl, lib=lib)
    op, lp = oracle.decode_paged(inp["q"], pool_k, pool_v, table, sl, page, lib=lib)
    assert np.array_equal(o, op) and np.array_equal(lse, lp)


def pin_paged_worked_example(lib):
    """The block tables the pages draw: requests A and B share their first two pages,
    so over those pages (and equal queries) they attend to the same keys; one token
    further, A reads p5 and B reads p2.  Each request's keys are also its pages' rows
    concatenated in table order."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "paged_block_table_example.json")))
    page, H_kv, d = 4, 1, 16
    rng = np.random.default_rng(33)
    pool_k = bf16_bits_from_f32(rng.standard_normal((g["pool_pages"], page, H_kv, d),
                                                    dtype=np.float32))
    pool_v = bf16_bits_from_f32(rng.standard_normal((g["pool_pages"], page, H_kv, d),
                                                    dtype=np.float32))
    names = sorted(g["tables"])
    width = max(len(t) for t in g["tables"].values())
    table = np.full((len(names), width), -1, dtype=np.int32)
    for r, n in enumerate(names):
        table[r, :len(g["tables"][n])] = g["tables"][n]
    q1 = bf16_bits_from_f32(rng.standard_normal((1, 2, d), dtype=np.float32))
    q = np.repeat(q1, len(names), axis=0)
    shared = g["shared_prefix_pages"] * page
    a, b = names.index("A"), names.index("B")
    sl = np.array([len(g["tables"][n]) * page for n in names], dtype=np.int32)
    sl[a] = sl[b] = shared
    o, lse = oracle.decode_paged(q, pool_k, pool_v, table, sl, page, lib=lib)
    assert np.array_equal(o[a], o[b]) and np.array_equal(lse[a], lse[b])
    sl[a] = sl[b] = shared + 1
    o, lse = oracle.decode_paged(q, pool_k, pool_v, table, sl, page, lib=lib)
    assert not np.allclose(o[a], o[b])
    sl = np.array([len(g["tables"][n]) * page for n in names], dtype=np.int32)
    o, lse = oracle.decode_paged(q, pool_k, pool_v, table, sl, page, lib=lib)
    for r, n in enumerate(names):
        kc = np.concatenate([pool_k[p] for p in g["tables"][n]])[None]
        vc = np.concatenate([pool_v[p] for p in g["tables"][n]])[None]
        oc, lc = oracle.decode(q[r:r + 1], kc, vc, lib=lib)
        assert np.array_equal(oc[0], o[r]) and np.array_equal(lc[0], lse[r])


# ---------------------------------------------------------------------------
# Decode of T tokens per sequence (the M-fold of G*T rows, ADR-0060 section 5.2).

def pin_decode_tokens_reduces_to_decode_and_chunks(lib):
    """T = 1 is the one-token decode; for T > 1 each sequence's tokens are the rows of its
    whole-prompt causal prefill at the last T positions; a token with a negative position
    (length below T) sees nothing."""
    inp = decode_inputs(3, 8, 2, 16, ragged=(5, 40), seed=34)
    q1 = inp["q"][:, None].copy()
    o, lse = oracle.decode_tokens(q1, inp["k"], inp["v"], inp["seqlens"], lib=lib)
    od, ld = oracle.decode(inp["q"], inp["k"], inp["v"], inp["seqlens"], lib=lib)
    assert np.array_equal(o[:, 0], od) and np.array_equal(lse[..., 0], ld)
    T = 4
    pin = prefill_inputs(3, 40, 8, 2, 16, seed=35)
    lens = np.array([40, 17, 4], dtype=np.int32)
    qs = np.stack([pin["q"][b, lens[b] - T:lens[b]] for b in range(3)])
    o, lse = oracle.decode_tokens(qs, pin["k"], pin["v"], lens, lib=lib)
    for b in range(3):
        n = int(lens[b])
        of, lf = oracle.prefill_causal(pin["q"][b:b + 1, :n].copy(), pin["k"][b:b + 1, :n].copy(),
                                       pin["v"][b:b + 1, :n].copy(), lib=lib)
        assert np.array_equal(o[b], of[0, n - T:]) and np.array_equal(lse[b], lf[0, :, n - T:])
    short = np.array([40, 2, 0], dtype=np.int32)
    o, lse = oracle.decode_tokens(qs, pin["k"], pin["v"], short, lib=lib)
    assert np.all(o[1, :2] == 0) and np.all(lse[1, :, :2] == -np.inf)
    assert np.all(np.isfinite(lse[1, :, 2:]))
    assert np.all(o[2] == 0) and np.all(lse[2] == -np.inf)


# ---------------------------------------------------------------------------
# Backward of causal prefill (V07 section 6.1, gradient formulas; section 6.4, recompute of
# P from the row's LSE).  The gradient of the scalar L = sum(O * dO) with respect to q, k
# and v is exactly what the backward returns for output gradient dO, so central
# differences of a library-routine forward pin every formula, index and scale in it.

def _np_causal_forward(q, k, v, tau):
    """Causal GQA attention on float64 arrays with scipy's softmax (head h reads KV head
    floor(h / G)): q [B, S, H_q, d]; k, v [B, S, H_kv, d] -> o [B, S, H_q, d]."""
    B, S, H_q, _ = q.shape
    G = H_q // k.shape[2]
    above = np.triu(np.ones((S, S), dtype=bool), 1)
    o = np.zeros_like(q)
    for b in range(B):
        for h in range(H_q):
            s = tau * (q[b, :, h] @ k[b, :, h // G].T)
            s[above] = -np.inf
            o[b, :, h] = softmax(s, axis=1) @ v[b, :, h // G]
    return o


def pin_bwd_finite_differences(lib):
    """Every coordinate of dq, dk, dv of a tiny case (two query heads per KV head, a scale
    that is not 1/sqrt(d)) against central differences of sum(O * dO)."""
    p = prefill_bwd_inputs(1, 5, 4, 2, 6, seed=71)
    q, k, v, do = (_f64(p[x]) for x in ("q", "k", "v", "do"))
    tau = 0.37
    dq, dk, dv, _, _ = oracle.prefill_causal_bwd(p["q"], p["k"], p["v"], p["do"], tau=tau,
                                                 nthreads=2, lib=lib)
    h = 1e-6
    for arr, grad, name in ((q, dq, "dq"), (k, dk, "dk"), (v, dv, "dv")):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            x0 = arr[idx]
            arr[idx] = x0 + h
            lp = float(np.sum(_np_causal_forward(q, k, v, tau) * do))
            arr[idx] = x0 - h
            lm = float(np.sum(_np_causal_forward(q, k, v, tau) * do))
            arr[idx] = x0
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(grad - fd).max()
        assert err <= 1e-7 + 1e-6 * np.abs(fd).max(), (name, err)


def pin_bwd_torch_autograd(lib):
    """A larger case (B = 2, ragged-looking S = 23, three query heads per KV head) against
    torch's fp64 autograd of the plain definition on the CPU."""
    import torch
    p = prefill_bwd_inputs(2, 23, 6, 2, 16, seed=72)
    tau = 0.21
    q, k, v = (torch.from_numpy(_f64(p[x])).requires_grad_(True) for x in ("q", "k", "v"))
    do = torch.from_numpy(_f64(p["do"]))
    G = 3
    kr = k.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)      # [B, H_q, S, d]
    vr = v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    s = tau * torch.matmul(q.permute(0, 2, 1, 3), kr.transpose(-1, -2).contiguous())
    s = s.masked_fill(torch.triu(torch.ones(23, 23, dtype=torch.bool), 1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vr).permute(0, 2, 1, 3)
    (o * do).sum().backward()
    dq, dk, dv, _, _ = oracle.prefill_causal_bwd(p["q"], p["k"], p["v"], p["do"], tau=tau,
                                                 nthreads=4, lib=lib)
    for mine, ref in ((dq, q.grad), (dk, k.grad), (dv, v.grad)):
        ref = ref.numpy()
        assert np.abs(mine - ref).max() <= 1e-10 * (1 + np.abs(ref).max())


def pin_bwd_invariants(lib):
    """Rows of P sum to one, so the dV rows of a KV head add up to the dO rows of its query
    heads; rows of dS sum to zero (sum_j P_ij (dP_ij - D_i) = D_i - D_i), so the dK rows of
    a KV head add up to zero."""
    p = prefill_bwd_inputs(2, 40, 8, 2, 16, seed=73)
    dq, dk, dv, _, _ = oracle.prefill_causal_bwd(p["q"], p["k"], p["v"], p["do"], nthreads=4,
                                                 lib=lib)
    do = _f64(p["do"])
    for b in range(2):
        for g in range(2):
            want = do[b][:, 4 * g:4 * g + 4].sum(axis=(0, 1))
            _rel_close(dv[b, :, g].sum(axis=0), want, rtol=1e-12, atol=1e-12)
            assert np.abs(dk[b, :, g].sum(axis=0)).max() <= 1e-12 * np.abs(dk[b, :, g]).sum()


def pin_bwd_single_token_and_gqa(lib):
    """S = 1: P = [1] and dS = 0, so dq = dk = 0 and dv sums the group's dO.  Grouped heads
    equal MHA on K/V repeated per query head, with dk, dv summed over each group."""
    p = prefill_bwd_inputs(1, 1, 4, 2, 8, seed=74)
    dq, dk, dv, lse, D = oracle.prefill_causal_bwd(p["q"], p["k"], p["v"], p["do"], lib=lib)
    assert np.all(dq == 0) and np.all(dk == 0)
    do = _f64(p["do"])
    _rel_close(dv[0, 0], do[0, 0].reshape(2, 2, 8).sum(axis=1), rtol=1e-15, atol=0)
    p = prefill_bwd_inputs(1, 19, 6, 2, 8, seed=75)
    kr, vr = (np.repeat(p[x], 3, axis=2) for x in ("k", "v"))
    g = oracle.prefill_causal_bwd(p["q"], p["k"], p["v"], p["do"], nthreads=4, lib=lib)
    m = oracle.prefill_causal_bwd(p["q"], kr, vr, p["do"], nthreads=4, lib=lib)
    _rel_close(g[0], m[0], rtol=1e-13, atol=1e-15)
    for t in (1, 2):
        _rel_close(g[t], m[t].reshape(1, 19, 2, 3, 8).sum(axis=3), rtol=1e-12, atol=1e-14)


def pin_bwd_row_and_key_subsets(lib):
    """The row and key functions on a subset give the rows of the whole backward, and the
    LSE the backward keeps is the forward's."""
    p = prefill_bwd_inputs(2, 21, 4, 1, 8, seed=76)
    dq, dk, dv, lse, D = oracle.prefill_causal_bwd(p["q"], p["k"], p["v"], p["do"], nthreads=3,
                                                   lib=lib)
    rows = np.array([[1, 3, 20], [0, 0, 0], [1, 2, 7]], dtype=np.int32)
    dqr, lser, Dr = oracle.prefill_causal_bwd_rows(p["q"], p["k"], p["v"], p["do"], rows,
                                                   lib=lib)
    for n, (b, h, i) in enumerate(rows):
        assert np.array_equal(dqr[n], dq[b, i, h]) and lser[n] == lse[b, h, i] and Dr[n] == D[b, h, i]
    keys = np.array([[0, 0, 20], [1, 0, 0], [1, 0, 9]], dtype=np.int32)
    dkr, dvr = oracle.prefill_causal_bwd_keys(p["q"], p["k"], p["v"], p["do"], lse, D, keys,
                                              lib=lib)
    for n, (b, g, j) in enumerate(keys):
        assert np.array_equal(dkr[n], dk[b, j, g]) and np.array_equal(dvr[n], dv[b, j, g])
    _, lse_f = oracle.prefill_causal(p["q"], p["k"], p["v"], lib=lib)
    _rel_close(lse, lse_f, rtol=1e-14, atol=1e-14)


def pin_bwd_stored_output_D(lib):
    """D taken from the caller: the exact D reproduces the exact gradient, and D shifted by
    delta_i moves dQ_i by -tau delta_i sum_j P_ij k_j -- attention with K as the values --
    while dK and dV follow the same formula (dV does not depend on D)."""
    p = prefill_bwd_inputs(1, 30, 4, 2, 16, seed=77)
    B, S, H_q, d = p["q"].shape
    tau = 0.3
    rows = np.stack(np.meshgrid([0], np.arange(H_q), np.arange(S), indexing="ij"),
                    axis=-1).reshape(-1, 3).astype(np.int32)
    dq0, lse, D0 = oracle.prefill_causal_bwd_rows(p["q"], p["k"], p["v"], p["do"], rows, tau=tau,
                                                  nthreads=2, lib=lib)
    dq1, _, D1 = oracle.prefill_causal_bwd_rows(p["q"], p["k"], p["v"], p["do"], rows, D=D0,
                                                tau=tau, nthreads=2, lib=lib)
    assert np.array_equal(D1, D0)
    _rel_close(dq1, dq0, rtol=1e-14, atol=1e-15)
    delta = np.linspace(-1.5, 2.0, rows.shape[0])
    dq2, _, D2 = oracle.prefill_causal_bwd_rows(p["q"], p["k"], p["v"], p["do"], rows,
                                                D=D0 + delta, tau=tau, nthreads=2, lib=lib)
    assert np.array_equal(D2, D0 + delta)
    ok, _ = oracle.prefill_causal(p["q"], p["k"], p["k"], tau=tau, lib=lib)   # sum_j P_ij k_j
    ok = ok[0].transpose(1, 0, 2).reshape(-1, d)                              # rows (h, i)
    _rel_close(dq2 - dq0, -tau * delta[:, None] * ok, rtol=1e-9, atol=1e-12)


def pin_bwd_stored_output_D_rows(lib):
    """D of a stored output (V07 section 6.2: D_i is the row-wise dot of dO_i and O_i),
    checked element by element against an explicit loop over (b, h, i) with exact sums, in
    the [B, H_q, S] order the backward's rows use; B = 2 and S != H_q so that a transposed or
    batch-mixed order cannot pass.  The D that ``prefill_causal_bwd(..., o=...)`` returns is
    the same array, and its dQ is that of the row-level call fed the loop's D.  With O the
    forward's own output, D also equals the sum over keys of P_ij dP_ij (the identity that
    section 6.2 uses to replace that sum), up to the bf16 rounding of the stored O."""
    B, S, H_q, H_kv, d = 2, 9, 4, 2, 16
    p = prefill_bwd_inputs(B, S, H_q, H_kv, d, seed=303)
    q, k, v, do = p["q"], p["k"], p["v"], p["do"]
    tau = 0.25
    o64, _ = oracle.prefill_causal(q, k, v, tau=tau, lib=lib)          # [B, S, H_q, d]
    o = bf16_bits_from_f32(o64.astype(np.float32))
    D = oracle.stored_output_D(o, do)
    assert D.shape == (B, H_q, S), D.shape
    of, dof = _f64(o), _f64(do)
    ref = np.empty((B, H_q, S))
    for b in range(B):
        for h in range(H_q):
            for i in range(S):
                ref[b, h, i] = math.fsum(float(of[b, i, h, c]) * float(dof[b, i, h, c])
                                         for c in range(d))
    _rel_close(D, ref, rtol=1e-15, atol=1e-300)
    dq, dk, dv, lse, D_ret = oracle.prefill_causal_bwd(q, k, v, do, o=o, tau=tau, nthreads=2,
                                                       lib=lib)
    _rel_close(D_ret, ref, rtol=1e-15, atol=1e-300)
    rows = np.stack(np.meshgrid(np.arange(B), np.arange(H_q), np.arange(S), indexing="ij"),
                    axis=-1).reshape(-1, 3).astype(np.int32)
    dq_r, _, _ = oracle.prefill_causal_bwd_rows(q, k, v, do, rows, D=ref.reshape(-1), tau=tau,
                                                nthreads=2, lib=lib)
    _rel_close(dq, dq_r.reshape(B, H_q, S, d).transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-15)
    # the exact D (sum_j P_ij dP_ij, the oracle's own) against the stored-output D: they
    # differ only through O's rounding to bf16, at most 2^-8 |O_i| per element (RNE)
    _, _, D_exact = oracle.prefill_causal_bwd_rows(q, k, v, do, rows, tau=tau, nthreads=2,
                                                   lib=lib)
    # (fp64 -> fp32 -> bf16 rounds twice: 2^-24 more at most)
    bound = (2.0 ** -8 + 2.0 ** -24) * np.einsum("bshc,bshc->bhs", np.abs(o64),
                                                np.abs(dof)).reshape(-1)
    err = np.abs(D_exact - ref.reshape(-1))
    assert np.all(err <= bound + 1e-13), f"max excess {np.max(err - bound)}"


# ---------------------------------------------------------------------------
# FP8 KV cache (V07 section 17.7; E4M3 as the OCP 8-bit floating-point specification
# defines it).

def pin_fp8_e4m3_values(lib):
    """Values the E4M3 definition fixes: zero, the subnormals m * 2^-9, the smallest normal
    2^-6, one, the largest finite 448, NaN at 0x7F and 0xFF; ascending codes give ascending
    values (no gap, no repeat), the sign bit mirrors them, and within a binade consecutive
    values are 2^(e-3) apart."""
    t = oracle.e4m3_table(lib)
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
            0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x40: 2.0, 0x7D: 416.0, 0x7E: 448.0,
            0x81: -(2.0 ** -9), 0xB8: -1.0, 0xFE: -448.0}
    for c, v in want.items():
        assert t[c] == v, (hex(c), t[c], v)
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isfinite(t[:0x7F]).all()
    assert np.all(np.diff(t[:0x7F]) > 0)
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F]) and np.signbit(t[0x80])
    for ex in range(1, 16):
        vals = t[8 * ex:min(8 * ex + 8, 0x7F)]
        assert np.allclose(np.diff(vals), 2.0 ** (ex - 7 - 3))


def pin_fp8_encode_nearest_even(lib):
    """Every finite value encodes to its own code; the midpoint of two neighbours goes to
    the one with the even mantissa, and a value one step off the midpoint to the nearer;
    beyond 448 saturates; NaN gives 0x7F."""
    t = oracle.e4m3_table(lib)[:0x7F]
    enc = lib.oracle_e4m3_encode
    for c in range(0x7F):
        assert enc(float(t[c])) == c and enc(float(-t[c])) == (0x80 | c), hex(c)
    for c in range(0x7E):
        mid = (t[c] + t[c + 1]) / 2
        assert enc(float(mid)) == (c if c % 2 == 0 else c + 1), hex(c)
        assert enc(float(np.nextafter(mid, 0.0))) == c and enc(float(np.nextafter(mid, 1e9))) == c + 1
    assert enc(1e6) == 0x7E and enc(-1e6) == 0xFE and enc(float("nan")) == 0x7F
    assert enc(2.0 ** -11) == 0 and enc(-(2.0 ** -11)) == 0x80


def pin_fp8_quantize_rows(lib):
    """Per-token quantisation: the scale is the smallest power of two 2^e with
    max|x| <= 448 * 2^e; every value dequantises to within half an E4M3 step of x (relative
    2^-4 in the normal range, 2^-10 * 2^e below it), exactly as a bfloat16; an all-zero
    row takes 2^-126 and zero codes."""
    rng = np.random.default_rng(81)
    rows = rng.standard_normal((40, 96)).astype(np.float32)
    rows *= np.exp2(rng.integers(-30, 30, size=(40, 1))).astype(np.float32)
    rows[3] = 0.0
    rows[4] = 0.0
    rows[4, 17] = 3.0e5
    x = bf16_bits_from_f32(rows)
    codes, scales = oracle.quantize_fp8_rows(x, lib)
    xv = _f64(x)
    t = oracle.e4m3_table(lib)
    for r in range(40):
        e = np.log2(float(scales[r]))
        assert e == int(e)
        amax = np.abs(xv[r]).max()
        if amax == 0:
            assert e == -126 and np.all(codes[r] == 0)
            continue
        assert amax <= 448 * 2.0 ** e and amax > 448 * 2.0 ** (e - 1)
        deq = t[codes[r]] * 2.0 ** e
        y = np.abs(xv[r]) * 2.0 ** -e
        half_step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 4),
                             2.0 ** -10) * 2.0 ** e
        assert np.all(np.abs(deq - xv[r]) <= half_step * (1 + 1e-12))
        assert np.array_equal(_f64(bf16_bits_from_f32(deq.astype(np.float32))), deq)


def pin_fp8_page_layout(lib):
    """V07 section 17.7's page: B_p token rows of codes, then the B_p per-token scales
    appended.  A worked example, byte by byte: two sequences of 20 and 5 tokens, pages of
    16 rows of one KV head of d = 8, tables [[2, 0], [1, -1]]; and the dequantised pool,
    gathered in token order, equals the dequantised rows."""
    rng = np.random.default_rng(82)
    x = bf16_bits_from_f32(rng.standard_normal((2, 20, 1, 8)).astype(np.float32))
    table = np.array([[2, 0], [1, -1]], dtype=np.int32)
    lens = np.array([20, 5], dtype=np.int32)
    pool = oracle.quantize_to_pages(x, lens, table, 16, 3, fill=0xAB, lib=lib)
    assert pool.shape == (3, 16 * 8 + 64)
    codes, scales = oracle.quantize_fp8_rows(x.reshape(2, 20, 8), lib)
    for b, n in ((0, 20), (1, 5)):
        for tok in range(n):
            pg, r = table[b, tok // 16], tok % 16
            assert np.array_equal(pool[pg, 8 * r:8 * r + 8], codes[b, tok])
            assert pool[pg, 128 + 4 * r:132 + 4 * r].view(np.float32)[0] == scales[b, tok]
    assert np.all(pool[0, 8 * 4:128] == 0xAB) and np.all(pool[1, 8 * 5:128] == 0xAB)
    deq = oracle.dequantize_pages(np.where(pool == 0xAB, 0, pool).astype(np.uint8), 16, 1, 8, lib)
    got = oracle.gather_pages(deq, table, lens, 16)
    want = oracle.e4m3_table(lib)[codes] * scales[..., None].astype(np.float64)
    assert np.array_equal(_f64(got[0, :20]).reshape(20, 8), want[0])
    assert np.array_equal(_f64(got[1, :5]).reshape(5, 8), want[1, :5])


def pin_fp8_decode_lossless_cache(lib):
    """A cache whose rows are already E4M3 values times a power of two (with 448 * 2^e in
    each row, so the quantiser picks that exponent) quantises losslessly: the decode over its
    FP8 pages equals the decode over the bf16 cache, bit for bit."""
    rng = np.random.default_rng(83)
    B, S, H_kv, d, page = 2, 48, 2, 16, 16
    t = oracle.e4m3_table(lib)
    def cache():
        c = rng.integers(0, 0x7F, size=(B, S, H_kv * d))
        c |= rng.integers(0, 2, size=c.shape) << 7
        c[:, :, 5] = 0x7E
        e = rng.integers(-12, 4, size=(B, S, 1))
        return bf16_bits_from_f32((t[c] * 2.0 ** e).astype(np.float32)).reshape(B, S, H_kv, d)
    k, v = cache(), cache()
    q = bf16_bits_from_f32(rng.standard_normal((B, 8, d)).astype(np.float32))
    lens = np.array([48, 21], dtype=np.int32)
    table = np.array([[4, 1, 0], [2, 3, -1]], dtype=np.int32)
    kp = oracle.quantize_to_pages(k, lens, table, page, 5, lib=lib)
    vp = oracle.quantize_to_pages(v, lens, table, page, 5, lib=lib)
    o8, l8 = oracle.decode_paged_fp8(q, kp, vp, table, lens, page, nthreads=2, lib=lib)
    o, l = oracle.decode(q, k, v, lens, nthreads=2, lib=lib)
    assert np.array_equal(o8, o) and np.array_equal(l8, l)


PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
