"""fp64 reference gradients of exact attention, written out from the definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module.

Pages cited (by title and section):

* "플래시어텐션: 메모리를 아끼는 정확한 어텐션" (FlashAttention explainer,
  base.kaita.kr): §4 재계산 -- the backward pass keeps only O and the row
  statistics from the forward pass and rebuilds S and P from Q, K, V; the
  algorithm flowchart ends in the same step; FAQ item 3 restates it.
* "Attention Mechanism Optimization for Efficient LLM Inference"
  (pyy0715.github.io): "Background: Scaled Dot-Product Attention" (the function
  being differentiated) and "Grouped-Query Attention (GQA)" (query heads of a
  group share one K/V head).

The pages give the recomputation principle but print no gradient formulas.
Reading taken here: the backward pass returns the exact gradient of
O = softmax(scale * Q K^T + mask) V with respect to Q, K and V, for an upstream
gradient dO, by the chain rule; nothing else is plausible for an exact method.
With GQA a K/V head's gradient is the sum over the query heads that read it.
Masked pairs have P = 0 and receive no gradient. Each gradient is a sum over
the allowed (row, key) pairs only, so a value at a pair the mask hides (an
Inf or NaN included) is no term of any gradient -- the forward oracle's
reading carried through the chain rule.
"""

import numpy as np

from .attention import _check_heads, element_mask

_ROW_CHUNK = 2048


def _pair_sum(W, X, allowed):
    """R[i] = sum over j with allowed[i, j] of W[i, j] * X[j], where W is 0 at
    the pairs that are not allowed. With X finite this is W @ X; an Inf or NaN
    entry X[j, c] is added only to the rows i allowed to pair with j (a zero
    weight times it would otherwise make every row NaN)."""
    fin = np.isfinite(X)
    if fin.all():
        return W @ X
    R = W @ np.where(fin, X, 0.0)
    for j, c in zip(*np.nonzero(~fin)):
        a = allowed[:, j]
        R[a, c] += W[a, j] * X[j, c]
    return R


def attention_backward(q, k, v, do, scale, *, causal=False, block_mask=None,
                       block_q=None, block_k=None):
    """Gradients (dQ, dK, dV) of exact attention, fp64.

    q, do: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d]. Returns dQ [B, Nq, Hq, d],
    dK and dV [B, Nk, Hkv, d], all float64.

    Per batch b and query head h (K/V head h // (Hq / Hkv)):
    1. S = scale * Q K^T with -inf at disallowed pairs; P = softmax(S) per row,
       the same safe softmax as the forward oracle. A row with no allowed key
       has P = 0 (its output is the constant 0).
    2. O = P V is linear in P and in V:  dV = P^T dO  and  dP = dO V^T.
    3. Softmax Jacobian per row: dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik).
    4. S is linear in Q and K:  dQ = scale * dS K  and  dK = scale * dS^T Q.
    5. GQA: dK and dV of a K/V head accumulate over its query heads.
    Every sum in 2-4 runs over the allowed pairs only: dP and dS are 0 at the
    other pairs, and the three products add a non-finite operand entry only
    through allowed pairs (_pair_sum).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape or do.shape != q.shape:
        raise ValueError("q/k/v/do shapes do not agree")
    group = _check_heads(Hq, Hkv)

    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            Kb = k[b, :, kvh, :]
            Vb = v[b, :, kvh, :]
            for r0 in range(0, Nq, _ROW_CHUNK):
                rr = np.arange(r0, min(Nq, r0 + _ROW_CHUNK))
                allowed = element_mask(Nq, Nk, causal=causal, block_mask=block_mask,
                                       block_q=block_q, block_k=block_k, rows=rr)
                S = np.where(allowed, scale * (q[b, rr, h, :] @ Kb.T), -np.inf)
                live = allowed.any(axis=1)
                m = np.where(live, S.max(axis=1), 0.0)
                P = np.where(allowed, np.exp(S - m[:, None]), 0.0)
                l = P.sum(axis=1)
                P = np.where(allowed, P / np.where(live, l, 1.0)[:, None], 0.0)
                dO = do[b, rr, h, :]
                dV[b, :, kvh, :] += _pair_sum(P.T, dO, allowed.T)
                dP = np.where(allowed, dO @ Vb.T, 0.0)
                dS = np.where(allowed, P * (dP - (P * dP).sum(axis=1, keepdims=True)), 0.0)
                dQ[b, rr, h, :] = scale * _pair_sum(dS, Kb, allowed)
                dK[b, :, kvh, :] += scale * _pair_sum(dS.T, q[b, rr, h, :], allowed.T)
    return dQ, dK, dV
