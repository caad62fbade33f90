"""Causal prefill against the fp64 oracle on the GPU."""
import numpy as np
import pytest
import torch

import gqa_attention_amd as g
import oracle
from gpu_util import bf16_bits, say, to_gpu_bf16
from gqa_workloads import LLAMA_LONG_PREFILL, LLAMA_PREFILL
from gqa_workloads.generate import for_config, prefill_inputs
from parity import check, to_f64

pytestmark = pytest.mark.gpu


def run_prefill(inp, scale=None):
    q, k, v = (to_gpu_bf16(inp[x]) for x in ("q", "k", "v"))
    o, lse = g.prefill_causal(q, k, v, softmax_scale=scale)
    torch.cuda.synchronize()
    return q, k, v, o, lse


SMALL = [
    # (B, S, H_q, H_kv)
    (1, 256, 8, 2),       # two q-blocks, diagonal and off-diagonal tiles
    (2, 200, 8, 2),       # ragged last q-block and key tile
    (1, 1, 8, 2),         # a single token
    (1, 63, 4, 4),        # G = 1 (MHA), shorter than one key tile
    (1, 384, 8, 1),       # MQA, three q-blocks
    (1, 520, 16, 2),      # G = 8 with the XCD remap active, ragged tail
    (2, 700, 16, 2),      # three 256-row q-blocks per head, ragged, B = 2 (remap active)
    (1, 1000, 8, 8),      # MHA at four q-blocks with a ragged last key tile
    (1, 333, 4, 2),       # G = 2
    (1, 300, 6, 2),       # G = 3 (no remap: 2 q-blocks x 2 KV heads is not a multiple of 8)
    (1, 200, 32, 2),      # G = 16
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_prefill_small_full(case, gpu_available):
    B, S, H_q, H_kv = case
    inp = prefill_inputs(B, S, H_q, H_kv, 128, seed=200 + S + H_q)
    say(f"prefill small {case}")
    _, _, v, o, lse = run_prefill(inp)
    o_ref, lse_ref = oracle.prefill_causal(inp["q"], inp["k"], inp["v"])
    check(to_f64(o), to_f64(lse), o_ref, lse_ref, str(case))
    # row 0 attends to key 0 only: O is V_0 exactly, for every head
    G = H_q // H_kv
    o0 = bf16_bits(o[:, 0])                                    # [B, H_q, d]
    v0 = np.repeat(inp["v"][:, 0], G, axis=1)                  # [B, H_q, d]
    assert np.array_equal(o0, v0)


def sample_rows(S, H_q, B, rng, n_random, extra_rows=()):
    """A stratified set of (b, h, i): first and last rows, q-block edges, random rows."""
    rows = set()
    heads = sorted({0, H_q - 1, *rng.integers(0, H_q, size=6).tolist()})
    # q-block (256 rows), key-tile (64) and pipeline-step (32) edges near every 1024th row
    edges = [i for qb in range(0, S, 1024)
             for i in (qb - 1, qb, qb + 31, qb + 32, qb + 63, qb + 64, qb + 127, qb + 128,
                       qb + 255, qb + 256)
             if 0 <= i < S]
    fixed = list(range(0, 16)) + list(range(S - 16, S)) + edges + list(extra_rows)
    for b in range(B):
        for h in heads:
            for i in fixed:
                rows.add((b, h, int(i)))
    for _ in range(n_random):
        rows.add((int(rng.integers(0, B)), int(rng.integers(0, H_q)), int(rng.integers(0, S))))
    return np.array(sorted(rows), dtype=np.int32)


def check_sampled(inp, o, lse, rows, what):
    o_ref, lse_ref = oracle.prefill_causal_rows(inp["q"], inp["k"], inp["v"], rows)
    b, h, i = (torch.from_numpy(rows[:, c].astype(np.int64)).to(o.device) for c in range(3))
    o_all = o[b, i, h]                                         # o is [B, S, H_q, d]
    l_all = lse[b, h, i]                                       # lse is [B, H_q, S]
    return check(to_f64(o_all), to_f64(l_all), o_ref, lse_ref, what)


def test_prefill_llama_s8192_full(gpu_available):
    """The Llama S = 8192 causal prefill, every O and LSE element of all 64 heads against
    the oracle (about 1.1e12 fp64 operations on the host)."""
    cfg = LLAMA_PREFILL
    inp = for_config(cfg)
    say(f"prefill {cfg.name}: GPU, then the oracle on every row")
    q, k, v, o, lse = run_prefill(inp)
    o_ref, lse_ref = oracle.prefill_causal(inp["q"], inp["k"], inp["v"])
    stats = check(to_f64(o), to_f64(lse), o_ref, lse_ref, cfg.name)
    say(f"  every row of {cfg.H_q} heads: {stats}")
    # deterministic: a second run is bitwise identical
    o2, lse2 = g.prefill_causal(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.fixture(scope="module")
def long_prefill_run(gpu_available):
    """The S = 65536 outlier prefill, run once on the GPU for the sampled checks below."""
    cfg = LLAMA_LONG_PREFILL
    inp = for_config(cfg)
    say(f"prefill {cfg.name}")
    q, k, v, o, lse = run_prefill(inp)
    yield cfg, inp, q, k, v, o, lse
    del q, k, v, o, lse


def long_positions(cfg, inp, part, parts):
    """Query positions of the S = 65536 check, about 2048 in all, dealt round-robin into
    `parts` shares: the first and last 64 rows, the rows either side of every 8th q-block
    (256-row) boundary, the rows at and just after 256 outlier keys, and uniform rows."""
    S = cfg.S
    rng = np.random.default_rng(4242)
    pos = set(range(64)) | set(range(S - 64, S))
    for blk in range(256, S, 8 * 256):
        pos |= {blk - 1, blk}
    outl = np.flatnonzero(inp["outlier_mask"][0].any(axis=-1))
    for i in rng.choice(outl, size=min(256, outl.size), replace=False):
        pos |= {int(i), min(int(i) + 1, S - 1)}
    while len(pos) < 2048:
        pos.add(int(rng.integers(0, S)))
    return np.array(sorted(pos))[part::parts]


@pytest.mark.parametrize("part", range(4))
def test_prefill_long_outliers_all_heads(long_prefill_run, part):
    """A quarter of about 2048 query positions of the S = 65536 prefill with outlier keys,
    every one of the 64 heads, against the oracle row by row."""
    cfg, inp, q, k, v, o, lse = long_prefill_run
    pos = long_positions(cfg, inp, part, 4)
    b, h, i = np.meshgrid([0], np.arange(cfg.H_q), pos, indexing="ij")
    rows = np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int32)
    say(f"  long prefill share {part}: {pos.size} positions x {cfg.H_q} heads")
    stats = check_sampled(inp, o, lse, rows, f"{cfg.name} share {part}")
    say(f"  {len(rows)} rows: {stats}")


def test_prefill_long_outliers_properties(long_prefill_run):
    """Properties at full size: finite, and LSE_i >= s_ii (the diagonal term is one of the
    sum's terms)."""
    cfg, inp, q, k, v, o, lse = long_prefill_run
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    G = cfg.H_q // cfg.H_kv
    for h in (0, 17, 63):
        qi = q[0, :, h].float()
        ki = k[0, :, h // G].float()
        s_diag = (qi * ki).sum(-1) * (1.0 / np.sqrt(cfg.d))
        assert torch.all(lse[0, h] >= s_diag - 1e-3)


def test_prefill_custom_scale(gpu_available):
    inp = prefill_inputs(1, 300, 8, 2, 128, seed=5)
    for scale in (0.0, 0.05):
        say(f"prefill scale={scale}")
        _, _, _, o, lse = run_prefill(inp, scale=scale)
        o_ref, lse_ref = oracle.prefill_causal(inp["q"], inp["k"], inp["v"],
                                               tau=float(np.float32(scale)))
        check(to_f64(o), to_f64(lse), o_ref, lse_ref, f"scale {scale}")
