"""Pins for the fp64 gradient oracle (oracle.attention_backward).

None of these re-types the oracle's formulas. The gradients are checked against
central finite differences of the forward oracle (itself pinned in
test_oracle.py), against closed forms and invariants that follow from the
definition of attention, and against torch autograd in float64 on the CPU.
A planted mistake in a copy of the gradient (a dropped term, a wrong sign, a
transposed operand, a missing scale) must fail the finite-difference pin.
"""

import numpy as np
import pytest
import torch

import oracle

rng = np.random.default_rng(2024)


def _case(B, Nq, Nk, Hq, Hkv, d):
    q = rng.standard_normal((B, Nq, Hq, d))
    k = rng.standard_normal((B, Nk, Hkv, d))
    v = rng.standard_normal((B, Nk, Hkv, d))
    do = rng.standard_normal((B, Nq, Hq, d))
    return q, k, v, do


def _loss(q, k, v, do, scale, **mask):
    """L = sum(O * dO); its gradient with respect to q, k, v is what the
    backward pass returns for the upstream gradient dO."""
    o, _ = oracle.attention(q, k, v, scale, **mask)
    return float((o * do).sum())


def _fd_grad(x, f, h=1e-5):
    """Central differences of f at x, element by element (error O(h^2))."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def _fd_all(q, k, v, do, scale, **mask):
    f = lambda: _loss(q, k, v, do, scale, **mask)  # noqa: E731
    return _fd_grad(q, f), _fd_grad(k, f), _fd_grad(v, f)


MASKS = {
    "none": dict(),
    "causal": dict(causal=True),
    "block": dict(block_mask=np.array([[1, 0, 1], [0, 1, 1]]), block_q=3, block_k=2),
}


@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("shape", [(1, 5, 5, 1, 1, 3), (2, 4, 7, 4, 2, 3), (1, 6, 6, 2, 1, 4)])
def test_gradients_match_finite_differences(mask, shape):
    B, Nq, Nk, Hq, Hkv, d = shape
    m = MASKS[mask]
    if mask == "block":
        Nq, Nk = 6, 6  # the 2 x 3 block mask at blocks 3 x 2
    q, k, v, do = _case(B, Nq, Nk, Hq, Hkv, d)
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, **m)
    fq, fk, fv = _fd_all(q, k, v, do, scale, **m)
    for got, want in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-8)


def test_causal_rows_without_keys_get_no_gradient():
    # Nq > Nk with the causal rule aligned at the end: the first Nq - Nk rows
    # see no key; their output is the constant 0, so their dQ is 0 and they
    # add nothing to dK or dV.
    q, k, v, do = _case(1, 6, 3, 2, 1, 4)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, causal=True)
    assert np.all(dq[:, :3] == 0)
    fq, fk, fv = _fd_all(q, k, v, do, 0.5, causal=True)
    np.testing.assert_allclose(dq, fq, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dk, fk, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dv, fv, rtol=1e-6, atol=1e-8)


# ------------------------------------------------------- closed forms, invariants
def test_constant_values_give_no_score_gradient():
    # every v_j equal: O = v whatever the weights, so dQ = dK = 0 exactly up to
    # rounding, and dV_j = sum_i P_ij dO_i sums to sum_i dO_i
    q, k, _, do = _case(1, 8, 8, 2, 2, 4)
    v = np.broadcast_to(rng.standard_normal((1, 1, 2, 4)), k.shape).copy()
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.6, causal=True)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), rtol=1e-12, atol=1e-12)


def test_single_key():
    # one key: P = 1 for every row, O = v_0; dV_0 = sum of dO, dQ = dK = 0
    q, k, v, do = _case(2, 5, 1, 4, 2, 3)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 1.3)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    want = do.reshape(2, 5, 2, 2, 3).sum(axis=(1, 3))  # rows and the group's heads
    np.testing.assert_allclose(dv[:, 0], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mask", list(MASKS))
def test_key_shift_invariance(mask):
    # adding one vector c to every key moves each row's scores by a constant,
    # which softmax ignores: dL/dc = sum_j dK_j = 0 per batch and K/V head
    m = MASKS[mask]
    q, k, v, do = _case(2, 6, 6, 4, 2, 5)
    _, dk, _ = oracle.attention_backward(q, k, v, do, 0.8, **m)
    assert np.abs(dk.sum(axis=1)).max() < 1e-11 * max(1.0, np.abs(dk).max())


@pytest.mark.parametrize("mask", list(MASKS))
def test_value_gradient_sums_to_upstream(mask):
    # sum_j P_ij = 1 for a row with keys, 0 without: sum_j dV_j is the sum of
    # dO over the rows that have keys and over the group's query heads
    m = MASKS[mask]
    q, k, v, do = _case(1, 6, 6, 4, 2, 3)
    _, _, dv = oracle.attention_backward(q, k, v, do, 0.9, **m)
    allowed = oracle.element_mask(6, 6, **{kk: vv for kk, vv in m.items()})
    live = allowed.any(axis=1)
    want = (do * live[None, :, None, None]).reshape(1, 6, 2, 2, 3).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), want, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ library routine
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_float64(causal):
    B, Nq, Nk, Hq, Hkv, d = 2, 9, 13, 4, 2, 8
    q, k, v, do = _case(B, Nq, Nk, Hq, Hkv, d)
    scale = d ** -0.5
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal=causal)

    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    G = Hq // Hkv
    qq = tq.permute(0, 2, 1, 3)
    kk = tk.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vv = tv.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    mask = None
    if causal:
        mask = torch.tensor(oracle.element_mask(Nq, Nk, causal=True))
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
    o.permute(0, 2, 1, 3).backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


# ------------------------------------------------------- the pin catches mistakes
def _planted(q, k, v, do, scale, mistake):
    """A copy of the gradient with one plausible mistake, for one head, no mask."""
    Q, K, V, dO = q[0, :, 0], k[0, :, 0], v[0, :, 0], do[0, :, 0]
    S = scale * Q @ K.T
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    dP = dO @ V.T
    Dr = (P * dP).sum(axis=1, keepdims=True)
    dS = {"no_row_term": P * dP, "sign": P * (Dr - dP)}.get(mistake, P * (dP - Dr))
    dQ = dS @ K * (1.0 if mistake == "no_scale" else scale)
    dK = scale * (dS.T @ Q)
    dV = (dO.T @ P).T if mistake != "transposed" else P @ dO[: P.shape[1]]
    return dQ, dK, dV


@pytest.mark.parametrize("mistake", ["none", "no_row_term", "sign", "no_scale", "transposed"])
def test_finite_differences_reject_planted_mistakes(mistake):
    q, k, v, do = _case(1, 5, 5, 1, 1, 3)
    fq, fk, fv = _fd_all(q, k, v, do, 0.7)
    dq, dk, dv = _planted(q, k, v, do, 0.7, mistake)
    ok = all(np.allclose(g, f[0, :, 0], rtol=1e-6, atol=1e-8)
             for g, f in ((dq, fq), (dk, fk), (dv, fv)))
    assert ok == (mistake == "none")  # the unplanted copy is the control


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # NaN/Inf inputs on purpose
def test_values_at_hidden_pairs_are_no_term_of_any_gradient():
    """An Inf or NaN planted where the mask hides it from part of the rows
    leaves every gradient entry that has no allowed path to it exactly as with
    a finite value there; entries reached through an allowed pair propagate it
    (IEEE). Paths worked out by hand from the chain rule, causal with
    Nq != Nk (row q sees keys <= q + 3) and a 3 x 3 block mask."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 12, 2, 8))
    k = rng.standard_normal((1, 15, 1, 8))
    v = rng.standard_normal((1, 15, 1, 8))
    do = rng.standard_normal((1, 12, 2, 8))
    rows = np.arange(12)
    keys = np.arange(15)
    base = oracle.attention_backward(q, k, v, do, 0.3, causal=True)

    def run(**planted):
        t = {"q": q, "k": k, "v": v, "do": do}
        for name, (idx, val) in planted.items():
            t[name] = t[name].copy()
            t[name][idx] = val
        return oracle.attention_backward(t["q"], t["k"], t["v"], t["do"], 0.3, causal=True)

    for bad in (np.nan, np.inf):
        # V at key 9 (seen by rows >= 6): dV never involves V; rows < 6 never meet it
        dQ, dK, dV = run(v=((0, 9, 0, slice(None)), bad))
        assert np.array_equal(dV, base[2])
        assert np.array_equal(dQ[0, rows < 6], base[0][0, rows < 6])
        assert not np.isfinite(dQ[0, rows >= 6]).any()
        # dO at row 4 (sees keys <= 7)
        dQ, dK, dV = run(do=((0, 4, 0, slice(None)), bad))
        assert np.array_equal(dV[0, keys > 7], base[2][0, keys > 7])
        assert np.array_equal(dK[0, keys > 7], base[1][0, keys > 7])
        assert np.array_equal(dQ[0, rows != 4], base[0][0, rows != 4])
        assert np.array_equal(dQ[0, 4, 1], base[0][0, 4, 1])  # the other query head
        assert not np.isfinite(dQ[0, 4, 0]).any() and not np.isfinite(dV[0, keys <= 7]).any()
        # K at key 9: rows < 6 never meet it
        dQ, dK, dV = run(k=((0, 9, 0, slice(None)), bad))
        assert np.array_equal(dQ[0, rows < 6], base[0][0, rows < 6])
        assert not np.isfinite(dQ[0, rows >= 6]).any()
        # Q at row 4: keys > 7 never meet it
        dQ, dK, dV = run(q=((0, 4, 1, slice(None)), bad))
        assert np.array_equal(dK[0, keys > 7], base[1][0, keys > 7])
        assert np.array_equal(dV[0, keys > 7], base[2][0, keys > 7])
        assert np.array_equal(dQ[0, rows != 4], base[0][0, rows != 4])
        assert not np.isfinite(dK[0, keys <= 7]).any()

    # block mask: key block 1 (keys 5..9) is seen by block rows 1 and 2 (rows 4..11)
    bm = np.array([[1, 0, 1], [0, 1, 1], [1, 1, 0]], dtype=np.uint8)
    kw = dict(block_mask=bm, block_q=4, block_k=5)
    b0 = oracle.attention_backward(q, k, v, do, 0.5, **kw)
    vb = v.copy()
    vb[0, 7, 0, 2] = np.nan
    dQ, dK, dV = oracle.attention_backward(q, k, vb, do, 0.5, **kw)
    assert np.array_equal(dV, b0[2])
    assert np.array_equal(dQ[0, rows < 4], b0[0][0, rows < 4])
    assert not np.isfinite(dQ[0, rows >= 4]).any()
    dob = do.copy()
    dob[0, 1, 0, :] = np.inf  # block row 0 sees key blocks 0 and 2
    dQ, dK, dV = oracle.attention_backward(q, k, v, dob, 0.5, **kw)
    assert np.array_equal(dV[0, 5:10], b0[2][0, 5:10])
    assert np.array_equal(dK[0, 5:10], b0[1][0, 5:10])
    assert not np.isfinite(dV[0, :5]).any() and not np.isfinite(dV[0, 10:]).any()
