"""Tolerance checks of GPU outputs against the fp64 oracle (test infrastructure).

The bar, per output tensor of one workload:
  O (bf16):  every element |O_gpu - O_ref| <= max(1e-2, ulp_bf16(O_ref)),
             and ||O_gpu - O_ref||_2 / ||O_ref||_2 <= 5e-3;
  LSE (fp32): max |LSE_gpu - LSE_ref| <= 1e-3, and rows with no key (LSE_ref =
             -inf) must be -inf with O = 0 exactly.
The ulp term only binds where |O_ref| >= 2 (a bf16 ulp there is >= 2^-6): rounding
the output to bf16 alone can then move it by half an ulp, more than 1e-2 once
|O_ref| >= 4.  The checker reports how many elements needed it.
"""
import numpy as np

O_MAX_ABS = 1e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


def bf16_ulp(x):
    """Spacing of bfloat16 values at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(ax > 0, ax, 1.0))
    return np.where(ax > 0, np.ldexp(1.0, e - 8), 0.0)


def to_f64(t):
    """A torch tensor (any float dtype, any device) as float64 numpy, exactly."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    """Assert the bar above; returns a dict of error statistics."""
    o = np.asarray(o_gpu, dtype=np.float64)
    lse = np.asarray(lse_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    assert o.shape == o_ref.shape, (what, o.shape, o_ref.shape)
    assert lse.shape == lse_ref.shape, (what, lse.shape, lse_ref.shape)

    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty-row LSE pattern differs"
    assert np.all(np.isfinite(lse[~empty])), f"{what}: non-finite LSE"
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"

    err = np.abs(o - o_ref)
    bound = np.maximum(O_MAX_ABS, bf16_ulp(o_ref))
    bad = err > bound
    n_ulp = int(np.sum((err > O_MAX_ABS) & ~bad))
    denom = np.linalg.norm(o_ref)
    rel_l2 = float(np.linalg.norm(o - o_ref) / denom) if denom > 0 else float(np.linalg.norm(o))
    lse_err = float(np.max(np.abs(lse[~empty] - lse_ref[~empty]))) if np.any(~empty) else 0.0
    stats = {"max_abs": float(err.max()) if err.size else 0.0, "rel_l2": rel_l2,
             "lse_max_abs": lse_err, "n_ulp_bound": n_ulp, "n": int(err.size)}
    if np.any(bad):
        idx = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} O elements beyond max(1e-2, ulp); worst at "
                             f"{idx}: gpu {o[idx]!r} ref {o_ref[idx]!r}; stats {stats}")
    assert rel_l2 <= O_REL_L2, f"{what}: rel-L2 {rel_l2} > {O_REL_L2}; stats {stats}"
    assert lse_err <= LSE_MAX_ABS, f"{what}: LSE error {lse_err} > {LSE_MAX_ABS}; stats {stats}"
    return stats


# Gradients of the causal-prefill backward (bf16 outputs).  Each element is a sum of
# products in which one bf16 operand was rounded on the GPU (P or dS, relative error
# <= 2^-8 each), D comes from the bf16-rounded forward output, and the result is rounded
# to bf16 (<= 2^-8 relative).  The products have mixed signs (the rows of dS sum to zero),
# so an element's error scales with the magnitude of its row's terms, not with the element
# itself: a query row that sees few keys has large dS terms and a small, cancelled sum.
# The bar per tensor, with rows the last axis (one query or key vector):
#   every element |g - g_ref| <= GRAD_REL |g_ref| + GRAD_ROW rms(row of g_ref)
#                                + GRAD_TENSOR rms(g_ref),
#   ||g - g_ref||_2 / ||g_ref||_2 <= GRAD_REL_L2 (twice the forward's O bound: two
#   rounded operands in the chain instead of one).
# The tensor term and GRAD_ABS cover rows whose exact gradient is zero (dQ of query row 0:
# its only key gives dS = dP - D = 0, which the GPU forms as the difference of two fp32
# dot products of d = 128 terms summed in different orders; the residue, about
# 2^-24 |dO| |v| ~ 1e-6 before the factor tau |k|, stays far below 1e-5).
GRAD_REL = 2.0 ** -6
GRAD_ROW = 2.0 ** -4
GRAD_TENSOR = 2.0 ** -8
GRAD_ABS = 1e-5
GRAD_REL_L2 = 1e-2


def check_grad(g_gpu, g_ref, what=""):
    """Assert the gradient bar above; returns error statistics."""
    g = np.asarray(g_gpu, dtype=np.float64)
    ref = np.asarray(g_ref, dtype=np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    rms_row = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    err = np.abs(g - ref)
    bound = GRAD_REL * np.abs(ref) + GRAD_ROW * rms_row + GRAD_TENSOR * rms + GRAD_ABS
    denom = np.linalg.norm(ref)
    rel_l2 = float(np.linalg.norm(g - ref) / denom) if denom > 0 else 0.0
    stats = {"max_abs": float(err.max()) if err.size else 0.0, "rms_ref": rms,
             "max_err_over_bound": float((err / bound).max()) if err.size else 0.0,
             "rel_l2": rel_l2, "n": int(err.size)}
    bad = err > bound
    if np.any(bad):
        idx = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond the bound; worst at {idx}: "
                             f"gpu {g[idx]!r} ref {ref[idx]!r} row rms "
                             f"{float(rms_row[idx[:-1]][0])!r}; stats {stats}")
    assert rel_l2 <= GRAD_REL_L2, f"{what}: rel-L2 {rel_l2} > {GRAD_REL_L2}; stats {stats}"
    return stats
