"""Pins for the fp64 oracle against what the pages and the mathematics fix.

Each test names the passage or property it rests on. None of them re-types the
oracle's formula: they use printed numbers, closed forms, invariants, library
routines (torch SDPA in float64 on the CPU, scipy logsumexp) or independent
constructions (frame gather, chunked prefill, split + merge).
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from exact_io_aware_attn_amd.inputs import frame_block_mask

from conftest import GOLDEN

rng = np.random.default_rng(12345)


def _randn(*shape):
    return rng.standard_normal(shape)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _row_as_attention(x):
    """Embed a score row x as attention: d = len(x), q = e0, k_j = x_j e0, v_j = e_j.
    Then S_j = x_j (scale 1) and O = P, so O and LSE expose the softmax itself."""
    n = len(x)
    q = np.zeros((1, 1, 1, n)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, n, 1, n)); k[0, :, 0, 0] = x
    v = np.eye(n)[None, :, None, :]
    return q, k, v


# ---------------------------------------------------------------- printed examples
def test_online_softmax_flash_explainer_example():
    ex = _golden("online_softmax_examples.json")["flash_explainer_tiling"]
    p, tol = ex["printed"], 0.5 * 10 ** -ex["decimals"] + 1e-12
    steps = oracle.online_softmax(ex["x"], ex["blocks"])
    (m1, l1), (m, l) = steps
    assert m1 == p["block1_m"] and abs(l1 - p["block1_l"]) <= tol
    assert m == p["merged_m"] and abs(l - p["merged_l"]) <= tol
    (m2, l2), = oracle.online_softmax(ex["x"][2:], [2])
    assert m2 == p["block2_m"] and abs(l2 - p["block2_l"]) <= tol
    # the rescaled first block and the direct sum printed on the page
    assert abs(l1 * math.exp(m1 - m) - p["block1_rescaled"]) <= tol
    assert abs(sum(p["direct_terms"]) - l) <= 4 * tol


def test_online_softmax_llm_inference_example():
    ex = _golden("online_softmax_examples.json")["llm_inference_online_softmax"]
    p, tol = ex["printed"], 0.5 * 10 ** -ex["decimals"] + 1e-12
    (m_old, d_old), (m_new, d_new) = oracle.online_softmax(ex["x"], ex["blocks"])
    assert m_old == p["block1_m"] and abs(d_old - p["block1_d"]) <= tol
    assert m_new == p["block2_m"] and abs(d_new - p["d_new"]) <= tol
    assert abs(math.exp(m_old - m_new) - p["rescale"]) <= tol
    assert abs(d_old * math.exp(m_old - m_new) - p["block1_rescaled"]) <= tol
    (_, d_b2), = oracle.online_softmax(ex["x"][2:], [2])
    assert abs(d_b2 - p["block2_d"]) <= tol


@pytest.mark.parametrize("key", ["flash_explainer_tiling", "llm_inference_online_softmax"])
def test_attention_reproduces_printed_softmax(key):
    """Exact attention on the printed score row gives the printed normaliser and
    (with V = I) the printed per-term exponentials divided by it."""
    ex = _golden("online_softmax_examples.json")[key]
    p, tol = ex["printed"], 0.5 * 10 ** -ex["decimals"]
    q, k, v = _row_as_attention(ex["x"])
    O, LSE = oracle.attention(q, k, v, 1.0)
    m = p.get("merged_m", p.get("m"))
    l_printed = p.get("merged_l", p.get("Z_prime"))
    assert abs(math.exp(LSE[0, 0, 0] - m) - l_printed) <= tol
    # both pages print the exponentials exp(x_j - m) in the order of x
    terms = p.get("direct_terms", p.get("terms"))
    for j in range(len(ex["x"])):
        assert abs(O[0, 0, 0, j] - terms[j] / l_printed) <= 2 * tol / l_printed


def test_merge_rule_on_printed_blocks():
    """Merging the two blocks' (O, LSE) with the block rule gives the printed
    merged normaliser and equals the undivided row (FlashAttention explainer §2)."""
    ex = _golden("online_softmax_examples.json")["flash_explainer_tiling"]
    p = ex["printed"]
    q, k, v = _row_as_attention(ex["x"])
    parts_o, parts_l = [], []
    for lo, hi in [(0, 2), (2, 4)]:
        o, lse = oracle.attention(q, k[:, lo:hi], v[:, lo:hi], 1.0)
        parts_o.append(o[0, 0, 0]); parts_l.append(lse[0, 0, 0])
    assert abs(math.exp(parts_l[0] - p["block1_m"]) - p["block1_l"]) <= 5e-4
    assert abs(math.exp(parts_l[1] - p["block2_m"]) - p["block2_l"]) <= 5e-4
    o, lse = oracle.merge_partials(parts_o, parts_l)
    assert abs(math.exp(lse - p["merged_m"]) - p["merged_l"]) <= 5e-4
    O, LSE = oracle.attention(q, k, v, 1.0)
    np.testing.assert_allclose(o, O[0, 0, 0], atol=1e-15)
    assert abs(lse - LSE[0, 0, 0]) <= 1e-14


# ---------------------------------------------------------------- closed forms
def test_rows_of_p_sum_to_one():
    n = 37
    q = _randn(2, 19, 3, n)
    k = _randn(2, n, 3, n)
    v = np.broadcast_to(np.eye(n)[None, :, None, :], (2, n, 3, n)).copy()
    O, _ = oracle.attention(q, k, v, 0.3, causal=True)
    P = O  # with V = I the output rows are the probability rows
    assert (P >= 0).all()
    np.testing.assert_allclose(P.sum(axis=-1), 1.0, atol=1e-12)


def test_single_key_returns_its_value_row():
    q = _randn(1, 5, 2, 8)
    k = _randn(1, 1, 2, 8)
    v = _randn(1, 1, 2, 8)
    O, LSE = oracle.attention(q, k, v, 0.7)
    for h in range(2):
        assert np.array_equal(O[0, :, h, :], np.broadcast_to(v[0, 0, h], (5, 8)))
        np.testing.assert_allclose(LSE[0, h], 0.7 * (q[0, :, h] @ k[0, 0, h]), atol=1e-14)


def test_identical_keys_return_mean_value():
    n = 29
    q = _randn(1, 7, 1, 16)
    k = np.broadcast_to(_randn(1, 1, 1, 16), (1, n, 1, 16)).copy()
    v = _randn(1, n, 1, 16)
    O, LSE = oracle.attention(q, k, v, 0.25)
    np.testing.assert_allclose(O[0, :, 0], np.broadcast_to(v[0, :, 0].mean(axis=0), (7, 16)), atol=1e-13)
    np.testing.assert_allclose(LSE[0, 0], 0.25 * (q[0, :, 0] @ k[0, 0, 0]) + math.log(n), atol=1e-12)


def test_causal_first_row_is_first_value():
    q, k, v = _randn(2, 9, 2, 8), _randn(2, 9, 2, 8), _randn(2, 9, 2, 8)
    O, _ = oracle.attention(q, k, v, 0.5, causal=True)
    assert np.array_equal(O[:, 0], v[:, 0])


def test_empty_row_is_zero_with_minus_inf_lse():
    bm = np.ones((2, 2), dtype=np.uint8); bm[1, :] = 0
    q, k, v = _randn(1, 32, 1, 8), _randn(1, 32, 1, 8), _randn(1, 32, 1, 8)
    O, LSE = oracle.attention(q, k, v, 1.0, block_mask=bm, block_q=16, block_k=16)
    assert (O[0, 16:] == 0).all() and np.isneginf(LSE[0, 0, 16:]).all()
    assert np.isfinite(LSE[0, 0, :16]).all()


# ---------------------------------------------------------------- invariants
def test_joint_permutation_invariance():
    q, k, v = _randn(2, 11, 4, 16), _randn(2, 23, 2, 16), _randn(2, 23, 2, 16)
    perm = rng.permutation(23)
    O1, L1 = oracle.attention(q, k, v, 0.25)
    O2, L2 = oracle.attention(q, k[:, perm], v[:, perm], 0.25)
    np.testing.assert_allclose(O1, O2, atol=1e-12)
    np.testing.assert_allclose(L1, L2, atol=1e-12)


def test_split_then_merge_equals_whole():
    """Attention over two disjoint key ranges, combined by the block rule, is the
    attention over all keys (the split-K decode relies on this)."""
    q, k, v = _randn(3, 1, 4, 32), _randn(3, 100, 2, 32), _randn(3, 100, 2, 32)
    O, L = oracle.attention(q, k, v, 0.2)
    parts = [oracle.attention(q, k[:, a:b], v[:, a:b], 0.2) for a, b in [(0, 37), (37, 64), (64, 100)]]
    # LSE is [B, H, Nq]; lay it out like O's leading dims [B, Nq, H] for the merge
    o, l = oracle.merge_partials([p[0] for p in parts], [p[1].transpose(0, 2, 1) for p in parts])
    np.testing.assert_allclose(o, O, atol=1e-12)
    np.testing.assert_allclose(l, L.transpose(0, 2, 1), atol=1e-12)


def test_merge_ignores_empty_parts():
    o = np.array([[1.0, 2.0], [5.0, 7.0]])
    lse = np.array([0.3, -np.inf])
    mo, ml = oracle.merge_partials(o, lse)
    np.testing.assert_array_equal(mo, o[0]); assert ml == 0.3
    mo, ml = oracle.merge_partials(o, np.array([-np.inf, -np.inf]))
    assert (mo == 0).all() and np.isneginf(ml)


# ---------------------------------------------------------------- library routines
def _sdpa(q, k, v, scale, causal=False, mask=None):
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=am, is_causal=causal, scale=scale,
        enable_gqa=tq.shape[1] != tk.shape[1])
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_fp64(Hq, Hkv, causal):
    q, k, v = _randn(2, 45, Hq, 24), _randn(2, 45, Hkv, 24), _randn(2, 45, Hkv, 24)
    O, _ = oracle.attention(q, k, v, 0.37, causal=causal)
    np.testing.assert_allclose(O, _sdpa(q, k, v, 0.37, causal=causal), atol=1e-12)


def test_block_mask_against_sdpa_with_dense_mask():
    bm = (rng.random((3, 4)) < 0.6).astype(np.uint8)
    bm[:, 0] = 1  # every row keeps a live block
    q, k, v = _randn(1, 48, 2, 8), _randn(1, 64, 2, 8), _randn(1, 64, 2, 8)
    O, _ = oracle.attention(q, k, v, 0.5, block_mask=bm, block_q=16, block_k=16)
    dense = np.kron(bm, np.ones((16, 16))).astype(bool)
    np.testing.assert_allclose(O, _sdpa(q, k, v, 0.5, mask=dense), atol=1e-12)


def test_lse_is_logsumexp_of_scaled_scores():
    q, k, v = _randn(2, 13, 3, 16), _randn(2, 40, 3, 16), _randn(2, 40, 3, 16)
    _, L = oracle.attention(q, k, v, 0.125)
    S = 0.125 * np.einsum("bihd,bjhd->bhij", q, k)
    np.testing.assert_allclose(L, logsumexp(S, axis=-1), atol=1e-12)


# ---------------------------------------------------------------- head groups
@pytest.mark.parametrize("pattern,Hkv", [("MHA_G8", 8), ("GQA_G2", 2), ("MQA_G1", 1)])
def test_gqa_head_groups_follow_the_diagram(pattern, Hkv):
    table = _golden("gqa_head_groups.json")[pattern]
    q, k, v = _randn(1, 9, 8, 16), _randn(1, 21, Hkv, 16), _randn(1, 21, Hkv, 16)
    O, L = oracle.attention(q, k, v, 0.25)
    for h in range(8):
        kv = table[h] - 1
        o1, l1 = oracle.attention(q[:, :, h:h + 1], k[:, :, kv:kv + 1], v[:, :, kv:kv + 1], 0.25)
        np.testing.assert_allclose(O[:, :, h], o1[:, :, 0], atol=1e-14)
        np.testing.assert_allclose(L[:, h], l1[:, 0], atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_heads():
    q, k, v = _randn(2, 17, 8, 16), _randn(2, 17, 2, 16), _randn(2, 17, 2, 16)
    O, _ = oracle.attention(q, k, v, 0.3, causal=True)
    O2, _ = oracle.attention(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 0.3, causal=True)
    np.testing.assert_allclose(O, O2, atol=1e-14)


# ---------------------------------------------------------------- causal alignment, decode
def test_causal_chunked_prefill_bottom_right():
    """The last Nq queries of a causal Nk x Nk problem, run alone against all Nk
    keys, see the same keys: bottom-right alignment (j <= i + Nk - Nq)."""
    q, k, v = _randn(1, 30, 2, 8), _randn(1, 30, 2, 8), _randn(1, 30, 2, 8)
    O, L = oracle.attention(q, k, v, 0.4, causal=True)
    O2, L2 = oracle.attention(q[:, 18:], k, v, 0.4, causal=True)
    np.testing.assert_allclose(O2, O[:, 18:], atol=1e-13)
    np.testing.assert_allclose(L2, L[:, :, 18:], atol=1e-13)


def test_decode_equals_prefill_on_cache_prefix():
    B, max_len = 3, 50
    seqlens = np.array([50, 17, 1])
    q = _randn(B, 4, 16)
    kc, vc = _randn(B, max_len, 2, 16), _randn(B, max_len, 2, 16)
    O, L = oracle.decode(q, kc, vc, seqlens, 0.25)
    for b in range(B):
        n = seqlens[b]
        o, l = oracle.attention(q[b:b + 1, None], kc[b:b + 1, :n], vc[b:b + 1, :n], 0.25)
        np.testing.assert_allclose(O[b], o[0, 0], atol=1e-14)
        np.testing.assert_allclose(L[b], l[0, :, 0], atol=1e-14)
        # the new token sees the whole prefix: causal with Nq = 1 is the same thing
        o2, _ = oracle.attention(q[b:b + 1, None], kc[b:b + 1, :n], vc[b:b + 1, :n], 0.25, causal=True)
        np.testing.assert_allclose(O[b], o2[0, 0], atol=1e-14)


def test_decode_zero_length_sequence():
    q = _randn(1, 2, 8)
    kc, vc = _randn(1, 4, 1, 8), _randn(1, 4, 1, 8)
    O, L = oracle.decode(q, kc, vc, np.array([0]), 1.0)
    assert (O == 0).all() and np.isneginf(L).all()


# ---------------------------------------------------------------- block sparsity
def test_all_ones_block_mask_is_dense():
    q, k, v = _randn(1, 32, 2, 8), _randn(1, 48, 2, 8), _randn(1, 48, 2, 8)
    O, L = oracle.attention(q, k, v, 0.5)
    O2, L2 = oracle.attention(q, k, v, 0.5, block_mask=np.ones((2, 3), np.uint8), block_q=16, block_k=16)
    np.testing.assert_array_equal(O, O2); np.testing.assert_array_equal(L, L2)


def test_frame_mask_equals_frame_gather():
    """Frame-structured attention: each query frame attends to its own frame,
    its neighbours and reference frame 0 (TPU guide, 3단계). Built here by
    gathering those frames' keys and running dense attention -- no mask."""
    frames, flen, blk = 5, 32, 16
    n = frames * flen
    bm = frame_block_mask(frames, flen, blk)
    q, k, v = _randn(1, n, 2, 8), _randn(1, n, 2, 8), _randn(1, n, 2, 8)
    O, L = oracle.attention(q, k, v, 0.35, block_mask=bm, block_q=blk, block_k=blk)
    for f in range(frames):
        seen = sorted({0, f} | {g for g in (f - 1, f + 1) if 0 <= g < frames})
        idx = np.concatenate([np.arange(g * flen, (g + 1) * flen) for g in seen])
        rows = slice(f * flen, (f + 1) * flen)
        o, l = oracle.attention(q[:, rows], k[:, idx], v[:, idx], 0.35)
        np.testing.assert_allclose(O[:, rows], o, atol=1e-12)
        np.testing.assert_allclose(L[:, :, rows], l, atol=1e-12)


# ---------------------------------------------------------------- fixed max
@pytest.mark.parametrize("centered", [False, True])
def test_logit_bound_holds(centered):
    q = _randn(2, 40, 4, 32)
    k = _randn(2, 60, 2, 32) + (1.5 if centered else 0.0)
    M = oracle.logit_bound(q, k, 0.2, centered=centered)
    S = 0.2 * np.einsum("bihd,bjhd->bhij", q, np.repeat(k, 2, axis=2))
    assert (S <= M[..., None] + 1e-12).all()


def test_logit_bound_is_tight_when_query_parallel_to_longest_key():
    k = _randn(1, 30, 1, 16)
    j = int(np.argmax((k[0, :, 0] ** 2).sum(-1)))
    q = 2.5 * k[:, j:j + 1].copy()  # q parallel to the longest key
    M = oracle.logit_bound(q, k, 0.3)
    s = 0.3 * float(q[0, 0, 0] @ k[0, j, 0])
    assert abs(M[0, 0, 0] - s) <= 1e-12 * abs(s)


def test_centering_tightens_bound_on_shifted_keys():
    q = _randn(1, 20, 1, 16)
    k = _randn(1, 80, 1, 16) + 3.0
    M0 = oracle.logit_bound(q, k, 0.25)
    M1 = oracle.logit_bound(q, k, 0.25, centered=True)
    assert (M1 <= M0 + 1e-12).mean() > 0.9


@pytest.mark.parametrize("centered", [False, True])
def test_fixed_max_softmax_equals_running_max(centered):
    q, k, v = _randn(2, 33, 4, 16), _randn(2, 33, 2, 16), _randn(2, 33, 2, 16)
    M = oracle.logit_bound(q, k, 0.25, centered=centered)
    O, L = oracle.attention(q, k, v, 0.25, causal=True)
    O2, L2 = oracle.fixed_max_attention(q, k, v, 0.25, M, causal=True)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L, atol=1e-12)


def _scores(q, k, scale):
    """[B, Hq, Nq, Nk] scaled scores, GQA heads expanded (einsum, not the oracle)."""
    g = q.shape[2] // k.shape[2]
    return scale * np.einsum("bihd,bjhd->bhij", q, np.repeat(k, g, axis=2))


_MASKS = {
    "none": {},
    "causal": dict(causal=True),
    "block": dict(block_mask=np.array([[1, 0, 1, 1], [0, 1, 0, 1], [1, 1, 0, 0]], np.uint8),
                  block_q=16, block_k=16),
    "causal+block": dict(causal=True,
                         block_mask=np.array([[1, 1, 0, 1], [1, 0, 1, 1], [0, 1, 1, 1]], np.uint8),
                         block_q=16, block_k=16),
}


@pytest.mark.parametrize("centered", [False, True])
@pytest.mark.parametrize("mask", list(_MASKS))
def test_fixed_max_bounds_bracket_the_row_max(centered, mask):
    """Cauchy-Schwarz from both sides (TPU guide, 4단계): every visible logit of
    row i is at most M_i, and the row's largest visible logit is at least
    M_i - gap_i, so its normaliser against M_i is at least exp(-gap_i). Keys
    with a common offset, blocks of 24 keys (several blocks, partial ones under
    the causal rule), Nq != Nk."""
    kw = _MASKS[mask]
    q = _randn(2, 48, 4, 16)
    k = _randn(2, 64, 2, 16) + 0.7
    M, gap, el = oracle.fixed_max_bounds(q, k, 0.3, centered=centered, key_block=24, **kw)
    S = _scores(q, k, 0.3)
    allowed = oracle.element_mask(48, 64, **kw)[None, None]
    live = np.broadcast_to(allowed.any(-1), M.shape)
    assert (live == np.isfinite(M)).all()
    Sa = np.where(allowed, S, -np.inf)
    assert (Sa <= M[..., None] + 1e-12).all()
    rmax = Sa.max(-1)
    assert (rmax[live] >= (M - gap)[live] - 1e-12).all()
    l = np.where(allowed, np.exp(S - np.where(live, M, 0)[..., None]), 0).sum(-1)
    assert (l[live] >= np.exp(-gap[live]) * (1 - 1e-12)).all()
    assert not el[~live].any()


@pytest.mark.parametrize("centered", [False, True])
def test_fixed_max_bounds_ignore_keys_the_row_cannot_see(centered):
    """The bound of a row depends on its visible keys only: keys past the causal
    limit of rows 0..t, and the keys of a block row's dead blocks, can change
    (to 5x longer ones, with an offset) without changing M, gap or eligibility
    of those rows -- the premise of excluding masked keys bit-exactly."""
    q = _randn(1, 64, 2, 16)
    k = _randn(1, 64, 1, 16)
    t = 29
    k2 = k.copy()
    k2[:, t + 1:] = 5 * k2[:, t + 1:] + 2
    for kw in (dict(causal=True), dict(causal=True, key_block=16), dict(causal=True, key_block=7)):
        a = oracle.fixed_max_bounds(q, k, 0.25, centered=centered, **kw)
        b = oracle.fixed_max_bounds(q, k2, 0.25, centered=centered, **kw)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x[..., :t + 1], y[..., :t + 1])
        assert not np.array_equal(a[0][..., t + 1:], b[0][..., t + 1:])
    bm = np.array([[1, 0, 1, 0], [0, 1, 1, 0], [1, 1, 1, 1], [0, 0, 1, 0]], np.uint8)
    kb = dict(block_mask=bm, block_q=16, block_k=16)
    k3 = k.copy()
    k3[:, 16:32] = 5 * k3[:, 16:32] + 2   # key block 1: dead for block rows 0 and 3
    a = oracle.fixed_max_bounds(q, k, 0.25, centered=centered, **kb)
    b = oracle.fixed_max_bounds(q, k3, 0.25, centered=centered, **kb)
    for x, y in zip(a, b):
        for rows in (slice(0, 16), slice(48, 64)):
            np.testing.assert_array_equal(x[..., rows], y[..., rows])
    assert not np.array_equal(a[0][..., 16:32], b[0][..., 16:32])


def test_fixed_max_bounds_reduce_to_the_page_bound():
    """With no mask and all keys in one block the plain bound is the guide's
    scale * |q_i| * max_j |k_j| (logit_bound) with gap 2 M_i; the centred one is
    within |q_i| |c - kbar| of logit_bound's centred form (c is kbar rounded
    to bfloat16)."""
    q = _randn(2, 30, 4, 32)
    k = _randn(2, 50, 2, 32) + 1.0
    M, gap, _ = oracle.fixed_max_bounds(q, k, 0.2, key_block=64)
    np.testing.assert_allclose(M, oracle.logit_bound(q, k, 0.2), rtol=1e-13)
    np.testing.assert_allclose(gap, 2 * M, rtol=1e-13)
    Mc, _, _ = oracle.fixed_max_bounds(q, k, 0.2, centered=True, key_block=64)
    Mp = oracle.logit_bound(q, k, 0.2, centered=True)
    kbar = k.mean(axis=1)                                          # [B, Hkv, d]
    slack = np.linalg.norm(kbar - oracle.round_to_bf16(kbar), axis=-1)  # [B, Hkv]
    qn = np.linalg.norm(q, axis=-1).transpose(0, 2, 1)             # [B, Hq, Nq]
    tol = 0.2 * 2 * qn * np.repeat(slack, 2, axis=1)[..., None] + 1e-12
    assert (np.abs(Mc - Mp) <= tol).all()


def test_fixed_max_bounds_tight_for_query_parallel_to_longest_visible_key():
    """q_i parallel to the longest key the row sees: the plain bound equals that
    logit, even with a 10x longer key just past the row's causal limit."""
    k = _randn(1, 40, 1, 16)
    q = np.zeros((1, 40, 1, 16))
    i = 25
    j = int(np.argmax((k[0, :i + 1, 0] ** 2).sum(-1)))
    k[0, i + 1, 0] *= 10
    q[0, i, 0] = 1.5 * k[0, j, 0]
    M, _, _ = oracle.fixed_max_bounds(q, k, 0.3, causal=True, key_block=8)
    s = 0.3 * float(q[0, i, 0] @ k[0, j, 0])
    assert abs(M[0, 0, i] - s) <= 1e-12 * abs(s)


def test_eligible_rows_keep_normaliser_far_from_underflow():
    """Soundness of the eligibility rule: when it says yes, every row's
    normaliser against the bound is at least exp(-tau)."""
    d, scale = 128, 1 / math.sqrt(128)
    q, k = _randn(1, 64, 1, d), _randn(1, 256, 1, d)
    for centered in (False, True):
        M, gap, el = oracle.fixed_max_bounds(q, k, scale, centered=centered, causal=True)
        assert el.all()
        S = np.where(np.tril(np.ones((64, 256), bool), 192), scale * q[0, :, 0] @ k[0, :, 0].T,
                     -np.inf)
        l = np.exp(S - M[0, 0][:, None]).sum(-1)
        assert (l >= math.exp(-oracle.TAU)).all()


def test_scaled_queries_are_ineligible_and_would_underflow():
    """Queries x10 at d = 128 make the bound loose by far more than the float32
    exponent range: the rule must refuse them (the fallback case). Scaling
    one head only leaves the other eligible."""
    d, scale = 128, 1 / math.sqrt(128)
    q, k = _randn(1, 64, 2, d), _randn(1, 512, 1, d)
    q[:, :, 1] *= 10
    M, gap, el = oracle.fixed_max_bounds(q, k, scale)
    assert el[0, 0].all() and not el[0, 1].any()
    S = scale * q[0, :, 1] @ k[0, :, 0].T
    assert (M[0, 1] - S.max(-1)).max() > 87.4  # exp(-gap) would be below the fp32 minimum normal


def test_rows_without_keys_or_with_few_keys_are_ineligible():
    q, k = _randn(1, 10, 1, 8), _randn(1, 4, 1, 8)
    M, gap, el = oracle.fixed_max_bounds(q, k, 0.5, causal=True, min_keys=1)  # rows 0..5 see nothing
    assert np.isneginf(M[0, 0, :6]).all() and not el[0, 0, :6].any() and el[0, 0, 6:].all()
    # rows 6..9 see 1..4 keys: below the default minimum of one key tile
    _, _, el = oracle.fixed_max_bounds(q, k, 0.5, causal=True)
    assert not el.any()
    q, k = _randn(1, 100, 1, 8), _randn(1, 100, 1, 8)
    _, _, el = oracle.fixed_max_bounds(q, k, 0.05, causal=True)
    assert not el[0, 0, :oracle.MIN_KEYS - 1].any() and el[0, 0, oracle.MIN_KEYS - 1:].all()


def test_round_to_bf16_matches_torch():
    """Library pin: torch's float32 -> bfloat16 conversion (nearest, ties to even)."""
    x = np.concatenate([_randn(4000) * 10.0 ** rng.integers(-6, 6, 4000),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, 65504.0])])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(x), ref)


@pytest.mark.parametrize("centered", [False, True])
def test_fixed_max_softmax_with_visible_key_bound_equals_running_max(centered):
    """Shift invariance with the per-row bound (TPU guide, 4단계): the softmax
    against M_i is the exact softmax."""
    q, k, v = _randn(2, 40, 4, 16), _randn(2, 33, 2, 16) + 0.5, _randn(2, 33, 2, 16)
    M, _, _ = oracle.fixed_max_bounds(q, k, 0.25, centered=centered, causal=True, key_block=8)
    O, L = oracle.attention(q, k, v, 0.25, causal=True)
    O2, L2 = oracle.fixed_max_attention(q, k, v, 0.25, np.where(np.isfinite(M), M, 0.0),
                                        causal=True)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L, atol=1e-12)


# ---------------------------------------------------------------- brute force
def test_brute_force_tiny():
    """Pure-Python loops on a tiny GQA + causal + block case."""
    B, Nq, Nk, Hq, Hkv, d = 1, 6, 8, 4, 2, 3
    q, k, v = _randn(B, Nq, Hq, d), _randn(B, Nk, Hkv, d), _randn(B, Nk, Hkv, d)
    bm = np.array([[1, 0], [1, 1], [0, 1]], dtype=np.uint8)  # block_q=2, block_k=4
    O, L = oracle.attention(q, k, v, 0.9, causal=True, block_mask=bm, block_q=2, block_k=4)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(Nq):
            keys = [j for j in range(Nk) if j <= i + (Nk - Nq) and bm[i // 2][j // 4]]
            if not keys:
                assert (O[0, i, h] == 0).all() and L[0, h, i] == -math.inf
                continue
            s = [0.9 * sum(q[0, i, h, t] * k[0, j, g, t] for t in range(d)) for j in keys]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            for t in range(d):
                o = sum(e[a] / z * v[0, keys[a], g, t] for a in range(len(keys)))
                assert abs(O[0, i, h, t] - o) < 1e-12
            assert abs(L[0, h, i] - (mx + math.log(z))) < 1e-12


def test_values_a_row_cannot_see_are_no_term_of_its_output():
    """An Inf or NaN in V at a key the mask hides from a row leaves that row
    exactly as with a finite value there; rows that see the key propagate it
    (IEEE). Causal (with Nq != Nk), block mask, and decode past the length."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 12, 2, 8))
    k = rng.standard_normal((1, 15, 1, 8))
    v = rng.standard_normal((1, 15, 1, 8))
    off = 15 - 12
    for bad in (np.nan, np.inf):
        vb = v.copy()
        vb[0, 9, 0, :] = bad
        O0, L0 = oracle.attention(q, k, v, 0.3, causal=True)
        O1, L1 = oracle.attention(q, k, vb, 0.3, causal=True)
        sees = np.arange(12) + off >= 9
        assert np.array_equal(O1[0, ~sees], O0[0, ~sees])
        assert not np.isfinite(O1[0, sees]).any()
        assert np.array_equal(L1, L0)
    bm = np.array([[1, 0, 1], [0, 1, 1], [1, 1, 0]], dtype=np.uint8)
    q3 = rng.standard_normal((1, 12, 1, 8))
    k3 = rng.standard_normal((1, 15, 1, 8))
    v3 = rng.standard_normal((1, 15, 1, 8))
    v3b = v3.copy()
    v3b[0, 7, 0, 2] = np.nan  # key block 1: seen by block rows 1 and 2
    O0, _ = oracle.attention(q3, k3, v3, 0.5, block_mask=bm, block_q=4, block_k=5)
    O1, _ = oracle.attention(q3, k3, v3b, 0.5, block_mask=bm, block_q=4, block_k=5)
    rows = np.arange(12) // 4 >= 1
    assert np.array_equal(O1[0, ~rows], O0[0, ~rows])
    assert np.isnan(O1[0, rows, 0, 2]).all() and np.isfinite(O1[0, rows][..., [0, 1, 3]]).all()
    seqlens = np.array([5, 9])
    qd = rng.standard_normal((2, 2, 8))
    kc = rng.standard_normal((2, 12, 1, 8))
    vc = rng.standard_normal((2, 12, 1, 8))
    vcb = vc.copy()
    vcb[0, 5:] = np.nan
    vcb[1, 9:] = np.inf
    assert np.array_equal(oracle.decode(qd, kc, vcb, seqlens, 0.4)[0],
                          oracle.decode(qd, kc, vc, seqlens, 0.4)[0])
