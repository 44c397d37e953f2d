"""Algorithmic work of the hot path: attended pairs, FLOPs and bytes.

Counting rules ("Attention Mechanism Optimization for Efficient LLM
Inference", "Why Decode is Memory-bound"): a score is a length-d dot product,
about 2d FLOPs, and so is each row of P V, so every attended (query, key) pair
costs 4d FLOPs; decode streams every cached key and value once.

The backward pass by recomputation (FlashAttention explainer, §4 재계산)
rebuilds S once and forms dV, dP, dQ and dK: five length-d products, 10d FLOPs
per attended pair. Its compulsory HBM traffic reads Q, K, V, O, dO and the LSE
once and writes dQ, dK and dV once.

Only pairs that are actually attended count (causal: the lower triangle;
block-sparse: live blocks only). Softmax work and the key-norm pre-pass are
excluded from the FLOP count.
"""

import numpy as np


def causal_pairs_per_row(nq, nk, rows=None):
    """Attended keys of each query row under the bottom-right causal rule
    (key j visible iff j <= i + nk - nq): clamp(i + nk - nq + 1, 0, nk)."""
    i = np.arange(nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    return np.clip(i + (nk - nq) + 1, 0, nk)


def attended_pairs(nq, nk, causal=False, block_mask=None, block_q=None, block_k=None):
    """Number of attended (query, key) pairs for one (batch, head)."""
    if block_mask is None:
        if not causal:
            return int(nq) * int(nk)
        return int(causal_pairs_per_row(nq, nk).sum())
    bm = np.asarray(block_mask) != 0
    if not causal:
        return int(bm.sum()) * int(block_q) * int(block_k)
    total = 0
    off = nk - nq
    for qb, kb in zip(*np.nonzero(bm)):
        i = np.arange(qb * block_q, (qb + 1) * block_q, dtype=np.int64)
        c0 = kb * block_k
        total += int(np.clip(i + off - c0 + 1, 0, block_k).sum())
    return total


def prefill_flops(B, Hq, d, pairs_per_head):
    """4 d FLOPs per attended pair (2d for Q K^T, 2d for P V), all heads."""
    return 4 * int(d) * int(pairs_per_head) * int(B) * int(Hq)


def decode_flops(seqlens, Hq, d):
    return 4 * int(d) * int(np.asarray(seqlens, dtype=np.int64).sum()) * int(Hq)


def decode_kv_bytes(seqlens, Hkv, d, elem_bytes=2):
    """K and V rows that must be read once: sum_b seqlen_b * Hkv * d * 2 * size."""
    return int(np.asarray(seqlens, dtype=np.int64).sum()) * int(Hkv) * int(d) * 2 * int(elem_bytes)


def prefill_io_bytes(B, Hq, Hkv, Nq, Nk, d, elem_bytes=2, lse=True):
    """Compulsory HBM bytes of a prefill call: read Q, K, V once, write O (+LSE)."""
    b = elem_bytes * d * (B * Nq * Hq * 2 + B * Nk * Hkv * 2)
    if lse:
        b += 4 * B * Hq * Nq
    return int(b)


def backward_flops(B, Hq, d, pairs_per_head):
    """10 d FLOPs per attended pair (S recomputed, dV, dP, dQ, dK), all heads."""
    return 10 * int(d) * int(pairs_per_head) * int(B) * int(Hq)


def backward_io_bytes(B, Hq, Hkv, Nq, Nk, d, elem_bytes=2):
    """Read Q, O, dO, K, V and the LSE once; write dQ, dK, dV once."""
    return int(elem_bytes * d * (B * Nq * Hq * 4 + B * Nk * Hkv * 4) + 4 * B * Hq * Nq)


def workload_work(w, block_mask=None, seqlens=None):
    """(flops, bytes) of one call of a named workload."""
    eb = 2 if w.dtype == "bf16" else 4
    if w.kind == "decode":
        # several new tokens share one read of the cache (their FLOPs: about 4 d
        # per token and cached row)
        return (decode_flops(seqlens, w.Hq, w.d) * w.n_new,
                decode_kv_bytes(seqlens, w.Hkv, w.d, eb))
    pairs = attended_pairs(w.Nq, w.Nk, causal=w.causal, block_mask=block_mask,
                           block_q=w.block or None, block_k=w.block or None)
    if w.kind == "backward":
        return (backward_flops(w.B, w.Hq, w.d, pairs),
                backward_io_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, eb))
    return (prefill_flops(w.B, w.Hq, w.d, pairs),
            prefill_io_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, eb))
