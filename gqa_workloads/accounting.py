"""Byte and FLOP accounting for the attention workloads.

These are the algorithmic figures the measurements divide by; they count what
the method must touch, not what a kernel happens to move.

* KV cache bytes: 2 * N * H_kv * d * sizeof(dtype) -- the GQA/MQA page of
  "Attention Kernel lineage" (section 14, KV cache size).
* Attention FLOP: 4 * N^2 * d per head (two N x N x d products, 2 FLOP per
  multiply-add) -- same page, section 4 (FlashAttention keeps the FLOP of the
  naive form).  Under a causal mask half of the square is kept: 4*S^2*d*H_q/2.
* Backward FLOP: the gradient formulas (same page, section 6.1) need four N x N x d
  products (dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q) and P again, which is
  formed from Q K^T and the row's LSE (section 6.3): five products, 2.5x the forward.
* Causal tile keep ratio 1/2 + B_c/(2N) -- same page, section 12.
* Score-matrix storage N^2 * sizeof(dtype) per head -- same page, section 1.
"""


def kv_bytes(n_tokens: int, H_kv: int, d: int, elem_bytes: int = 2) -> int:
    """Bytes of K plus V for ``n_tokens`` cached tokens (one layer)."""
    return 2 * n_tokens * H_kv * d * elem_bytes


def decode_kv_bytes(seqlens, H_kv: int, d: int, elem_bytes: int = 2) -> int:
    """K+V bytes one decode launch must read: every cached token of every sequence."""
    return sum(kv_bytes(int(s), H_kv, d, elem_bytes) for s in seqlens)


def decode_kv_bytes_fp8(seqlens, H_kv: int, d: int) -> int:
    """Bytes one decode launch must read from FP8 pages (same page, section 17.7): per token
    and pool the H_kv * d one-byte E4M3 codes plus its 4-byte scale."""
    return sum(2 * int(s) * (H_kv * d + 4) for s in seqlens)


def decode_flop(seqlens, H_q: int, d: int) -> int:
    """Q.K^T plus P.V multiply-adds of one decode launch, 2 FLOP each."""
    return sum(4 * int(s) * H_q * d for s in seqlens)


def prefill_causal_flop(B: int, S: int, H_q: int, d: int) -> float:
    """Causal prefill FLOP as the workload metric counts it: 4*S^2*d*H_q/2 per sequence."""
    return B * 4.0 * S * S * d * H_q / 2.0


def prefill_causal_bwd_flop(B: int, S: int, H_q: int, d: int) -> float:
    """Backward of causal prefill: five S x S x d products per head under the causal mask,
    5*S^2*d*H_q per sequence (2.5x ``prefill_causal_flop``)."""
    return B * 5.0 * 2.0 * S * S * d * H_q / 2.0


def prefill_chunk_flop(B: int, T: int, q_start: int, H_q: int, d: int) -> float:
    """Chunked causal prefill FLOP on the same convention: the chunk's rows see the
    q_start keys before it in full and its own T x T block as a half square,
    4*d*H_q*(T*q_start + T^2/2) per sequence (q_start = 0 gives the whole-prompt figure)."""
    return B * 4.0 * d * H_q * (T * q_start + T * T / 2.0)


def prefill_causal_flop_exact(B: int, S: int, H_q: int, d: int) -> int:
    """FLOP over the kept (i, j <= i) pairs only: 4*d per pair, S(S+1)/2 pairs per head."""
    return B * H_q * 4 * d * (S * (S + 1) // 2)


def score_matrix_bytes(N: int, elem_bytes: int = 2) -> int:
    """Bytes of one head's N x N score matrix if it were materialised."""
    return N * N * elem_bytes


def causal_keep_ratio(N: int, B_c: int) -> float:
    """Fraction of KV tiles a causal block-skip loop touches, in the square-tile limit."""
    return 0.5 + B_c / (2.0 * N)


def causal_tiles_kept(S: int, B_r: int, B_c: int) -> int:
    """Exact number of (q-block, kv-block) pairs with at least one visible key (j <= i)."""
    n_q = -(-S // B_r)
    kept = 0
    for qb in range(n_q):
        last_row = min(S, (qb + 1) * B_r) - 1
        kept += last_row // B_c + 1
    return kept


def kv_bytes_per_context_token(H_kv: int, d: int, elem_bytes: int = 2) -> int:
    """K+V bytes per cached token per layer."""
    return kv_bytes(1, H_kv, d, elem_bytes)
