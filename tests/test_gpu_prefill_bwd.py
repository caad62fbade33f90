"""Backward of causal prefill on the GPU against the fp64 oracle.

The backward's inputs are the forward's q, k, v, its output O and LSE, and the output
gradient dO.  The method forms D_i = dO_i . O_i from the stored O ("Attention Kernel
lineage" (V07), section 6.2), so a rounded O moves D slightly away from its exact value.
The parity cases therefore give both sides the same stored O -- the oracle's own forward
output rounded to bf16 -- and the oracle takes D from it (``o=``); what remains between
them is the kernels' own arithmetic, under the gradient bar of ``parity.check_grad``.
A second check per case runs the GPU forward then the GPU backward, as a training step
does, against the exact gradient (D from the exact O) on the relative L2 error.
The workspace is filled with 0xFF (NaN in every fp32 slot) before each call, so a slot
read before it is written would show.
"""
import numpy as np
import pytest
import torch

import gqa_attention_amd as g
import oracle
from gpu_util import say, to_gpu_bf16
from gqa_workloads import LLAMA_LONG_PREFILL, LLAMA_PREFILL
from gqa_workloads.generate import bf16_bits_from_f32, prefill_bwd_inputs
from parity import GRAD_REL_L2, check_grad, to_f64

pytestmark = pytest.mark.gpu


def oracle_stored_output(p, tau=None, rows=None):
    """The oracle forward's O rounded to bf16 (the stored output) and its LSE in fp32."""
    o, lse = oracle.prefill_causal(p["q"], p["k"], p["v"], tau=tau)
    return bf16_bits_from_f32(o.astype(np.float32)), lse.astype(np.float32)


def gpu_bwd(q, k, v, o, lse, do, tau=None):
    B, S, H_q, d = q.shape
    ws = g.prefill_bwd_workspace(B, S, H_q, k.shape[2], d)
    ws.fill_(0xFF)
    out = g.prefill_causal_bwd(q, k, v, o, lse, do, softmax_scale=tau, workspace=ws)
    torch.cuda.synchronize()
    return out


def rel_l2(mine, ref):
    m = to_f64(mine)
    return float(np.linalg.norm(m - ref) / np.linalg.norm(ref))


CASES = [
    # (B, S, H_q, H_kv)
    (1, 64, 8, 2),      # one key tile, one query tile
    (1, 300, 8, 2),     # ragged: two key blocks, two query blocks, a partial last tile
    (2, 257, 16, 2),    # one row past a 256 block, B = 2
    (1, 520, 4, 4),     # G = 1 (MHA), three query blocks
    (1, 33, 8, 1),      # MQA, shorter than a tile
    (1, 1, 8, 2),       # a single token: dQ = dK = 0, dV = the group's dO
    (1, 1000, 16, 8),   # G = 2, four key blocks
    (1, 768, 64, 8),    # Llama3-70B heads, whole blocks
    (1, 200, 6, 2),     # G = 3: the dK/dV items step through 3 heads a query tile
    (1, 130, 32, 2),    # G = 16, a partial last key block
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_bwd_small_full(case, gpu_available):
    B, S, H_q, H_kv = case
    p = prefill_bwd_inputs(B, S, H_q, H_kv, 128, seed=900 + S + H_q)
    o_bits, lse = oracle_stored_output(p)
    q, k, v, do, o = (to_gpu_bf16(x) for x in (p["q"], p["k"], p["v"], p["do"], o_bits))
    say(f"prefill backward {case}")
    dq, dk, dv = gpu_bwd(q, k, v, o, torch.from_numpy(lse).cuda(), do)
    rq, rk, rv, _, _ = oracle.prefill_causal_bwd(p["q"], p["k"], p["v"], p["do"], o=o_bits)
    for name, mine, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        say(f"  {name} {check_grad(to_f64(mine), ref, f'{case} {name}')}")
    if S == 1:   # dS = dP - D = 0 up to fp32 rounding: dQ = dK = 0
        assert dq.abs().max().item() < 1e-5 and dk.abs().max().item() < 1e-5
    # training order: the GPU forward's O and LSE, against the exact gradient
    say(f"prefill forward + backward {case}")
    o2, lse2 = g.prefill_causal(q, k, v)
    dq2, dk2, dv2 = gpu_bwd(q, k, v, o2, lse2, do)
    eq, ek, ev, _, _ = oracle.prefill_causal_bwd(p["q"], p["k"], p["v"], p["do"])
    errs = [rel_l2(dq2, eq), rel_l2(dk2, ek), rel_l2(dv2, ev)] if S > 1 else [rel_l2(dv2, ev)]
    say(f"  end to end rel-L2 (dq, dk, dv; dv only when S = 1): {[f'{e:.2e}' for e in errs]}")
    assert max(errs) <= GRAD_REL_L2, errs


def test_bwd_scale_and_determinism(gpu_available):
    """A scale other than 1/sqrt(d); two calls give the same bits."""
    tau = 0.05
    p = prefill_bwd_inputs(1, 200, 8, 2, 128, seed=931)
    o_bits, lse = oracle_stored_output(p, tau=tau)
    q, k, v, do, o = (to_gpu_bf16(x) for x in (p["q"], p["k"], p["v"], p["do"], o_bits))
    lse = torch.from_numpy(lse).cuda()
    say("prefill backward, tau = 0.05, twice")
    a = gpu_bwd(q, k, v, o, lse, do, tau=tau)
    b = gpu_bwd(q, k, v, o, lse, do, tau=tau)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    rq, rk, rv, _, _ = oracle.prefill_causal_bwd(p["q"], p["k"], p["v"], p["do"], o=o_bits,
                                                 tau=tau)
    for name, mine, ref in (("dq", a[0], rq), ("dk", a[1], rk), ("dv", a[2], rv)):
        check_grad(to_f64(mine), ref, f"tau 0.05 {name}")


def test_bwd_llama_s8192_sampled(gpu_available):
    """The Llama3-70B prefill workload (S = 8192, 64 query heads, 8 KV heads).  The GPU
    forward gives O and LSE; the O of query heads 0..7 (KV head 0) is replaced by the
    oracle's stored output, so that for those heads both sides form D from the same O.
    Checked: sampled dQ rows of heads 0..7, and sampled dK, dV rows of KV head 0 (the
    oracle's key side needs LSE and D of every row of those 8 query heads)."""
    cfg = LLAMA_PREFILL
    S, H_q, G = cfg.S, cfg.H_q, cfg.H_q // cfg.H_kv
    p = prefill_bwd_inputs(cfg.B, S, H_q, cfg.H_kv, cfg.d, seed=cfg.seed)
    q, k, v, do = (to_gpu_bf16(p[x]) for x in ("q", "k", "v", "do"))
    say(f"prefill forward {cfg.name}")
    o, lse = g.prefill_causal(q, k, v)
    torch.cuda.synchronize()
    say("  oracle forward of query heads 0..7")
    bb, hh, ii = np.meshgrid([0], np.arange(G), np.arange(S), indexing="ij")
    rows_g = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1).astype(np.int32)
    o_g, _ = oracle.prefill_causal_rows(p["q"], p["k"], p["v"], rows_g)
    o_g_bits = bf16_bits_from_f32(o_g.astype(np.float32)).reshape(G, S, cfg.d)
    o[0, :, :G] = to_gpu_bf16(np.ascontiguousarray(o_g_bits.transpose(1, 0, 2)))
    say(f"prefill backward {cfg.name}")
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, do)
    # D of every row of heads 0..7 from the stored O
    do_g = p["do"][0, :, :G].transpose(1, 0, 2)                       # [G, S, d]
    D_g = oracle.stored_output_D(o_g_bits[None].transpose(0, 2, 1, 3),
                                 do_g[None].transpose(0, 2, 1, 3))[0].reshape(-1)
    say("  oracle backward rows of query heads 0..7")
    dq_g, lse_g, D_chk = oracle.prefill_causal_bwd_rows(p["q"], p["k"], p["v"], p["do"], rows_g,
                                                        D=D_g)
    rng = np.random.default_rng(932)
    edges = [0, 1, 31, 32, 63, 64, 255, 256, 257, S - 257, S - 256, S - 1]
    pick = sorted({h * S + i for h in range(G) for i in edges} |
                  set(rng.integers(0, G * S, size=160).tolist()))
    pick = np.array(pick)
    hsel = torch.from_numpy(rows_g[pick, 1].astype(np.int64)).to(dq.device)
    isel = torch.from_numpy(rows_g[pick, 2].astype(np.int64)).to(dq.device)
    say(f"  dq {check_grad(to_f64(dq[0, isel, hsel]), dq_g[pick], 'llama dq rows')}")
    lse_all = np.zeros((1, H_q, S))
    D_all = np.zeros((1, H_q, S))
    lse_all[0, :G] = lse_g.reshape(G, S)
    D_all[0, :G] = D_chk.reshape(G, S)
    keys = sorted({0, 1, 255, 256, 4095, S - 257, S - 1, *rng.integers(0, S, size=40).tolist()})
    keys = np.array([(0, 0, j) for j in keys], dtype=np.int32)
    rk, rv = oracle.prefill_causal_bwd_keys(p["q"], p["k"], p["v"], p["do"], lse_all, D_all, keys)
    j = torch.from_numpy(keys[:, 2].astype(np.int64)).to(dk.device)
    say(f"  dk {check_grad(to_f64(dk[0, j, 0]), rk, 'llama dk keys')}")
    say(f"  dv {check_grad(to_f64(dv[0, j, 0]), rv, 'llama dv keys')}")


def test_bwd_llama_long_s65536_outliers_sampled(gpu_available):
    """The long-context workload (S = 65536, 1 % of key rows scaled by 8), forward and
    backward on the GPU.  The oracle's forward gives the stored O of the checked rows of
    query heads 0..7 (KV head 0), which replaces the GPU's O there, so both sides form
    those rows' D from the same O.  Checked: dQ on sampled rows across the whole prompt,
    and dK, dV of KV head 0 on keys of the last 256 positions, which only the last 256
    rows of each query head see (so the oracle's key side needs LSE and D of those rows
    only)."""
    cfg = LLAMA_LONG_PREFILL
    S, H_q, G, d = cfg.S, cfg.H_q, cfg.H_q // cfg.H_kv, cfg.d
    p = prefill_bwd_inputs(cfg.B, S, H_q, cfg.H_kv, d, seed=cfg.seed,
                           outlier_frac=cfg.outlier_frac, outlier_scale=cfg.outlier_scale)
    q, k, v, do = (to_gpu_bf16(p[x]) for x in ("q", "k", "v", "do"))
    say(f"prefill forward {cfg.name}")
    o, lse = g.prefill_causal(q, k, v)
    torch.cuda.synchronize()
    tail = 256
    rng = np.random.default_rng(933)
    picked = {(h, i) for h in range(G) for i in range(S - tail, S)}
    picked |= {(h, i) for h in (0, G - 1) for i in (0, 1, 255, 256, 4095, 32767, 32768)}
    picked |= {(int(rng.integers(0, G)), int(rng.integers(0, S - tail))) for _ in range(96)}
    rows = np.array([(0, h, i) for h, i in sorted(picked)], dtype=np.int32)
    say(f"  oracle forward of {len(rows)} rows of query heads 0..7")
    o_r, _ = oracle.prefill_causal_rows(p["q"], p["k"], p["v"], rows)
    o_r_bits = bf16_bits_from_f32(o_r.astype(np.float32))                  # [n, d]
    hsel = torch.from_numpy(rows[:, 1].astype(np.int64)).to(o.device)
    isel = torch.from_numpy(rows[:, 2].astype(np.int64)).to(o.device)
    o[0, isel, hsel] = to_gpu_bf16(o_r_bits)
    say(f"prefill backward {cfg.name}")
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, do)
    do_r = p["do"][0, rows[:, 2], rows[:, 1]]                              # [n, d]
    D_r = oracle.stored_output_D(o_r_bits[None, :, None], do_r[None, :, None]).reshape(-1)
    say("  oracle backward rows")
    dq_r, lse_r, D_chk = oracle.prefill_causal_bwd_rows(p["q"], p["k"], p["v"], p["do"], rows,
                                                        D=D_r)
    say(f"  dq {check_grad(to_f64(dq[0, isel, hsel]), dq_r, 'long dq rows')}")
    lse_all = np.zeros((1, H_q, S))
    D_all = np.zeros((1, H_q, S))
    lse_all[0, rows[:, 1], rows[:, 2]] = lse_r
    D_all[0, rows[:, 1], rows[:, 2]] = D_chk
    keys = sorted({S - tail, S - tail + 1, S - 129, S - 128, S - 2, S - 1,
                   *rng.integers(S - tail, S, size=10).tolist()})
    keys = np.array([(0, 0, j) for j in keys], dtype=np.int32)
    rk, rv = oracle.prefill_causal_bwd_keys(p["q"], p["k"], p["v"], p["do"], lse_all, D_all, keys)
    j = torch.from_numpy(keys[:, 2].astype(np.int64)).to(dk.device)
    say(f"  dk {check_grad(to_f64(dk[0, j, 0]), rk, 'long dk keys')}")
    say(f"  dv {check_grad(to_f64(dv[0, j, 0]), rv, 'long dv keys')}")
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all()
