"""attn_bwd on the GPU against the fp64 gradient oracle (element by element).

The GPU side takes O and the LSE from attn_fwd on the same inputs, as a caller
would; the oracle differentiates the definition from Q, K, V and dO alone.
Small cases span several 128-row / 64-row tiles with ragged tails; full-size
workloads are checked on sliced (batch, head group) pieces."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_attn_amd import attn_bwd, attn_fwd, prepare_bwd
from exact_io_aware_attn_amd.inputs import (WORKLOADS, backward_inputs, frame_block_mask,
                                            workload_inputs)

from parity import check_grad, check_grad_nonfinite, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu_grads(q, k, v, do, causal, scale=None):
    q, k, v, do = (t.to(DEV) for t in (q, k, v, do))
    o, lse = attn_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check(q, k, v, do, causal, where, scale=None):
    d = q.shape[-1]
    sc = 1 / math.sqrt(d) if scale is None else scale
    dq, dk, dv = _gpu_grads(q, k, v, do, causal, scale)
    ref = oracle.attention_backward(to64(q), to64(k), to64(v), to64(do), sc, causal=causal)
    errs = [check_grad(g, r, f"{where} {n}") for g, r, n in zip((dq, dk, dv), ref, "QKV")]
    print(where, " ".join(f"d{n} {e[0]:.2e}/{e[1]:.2e}" for n, e in zip("QKV", errs)))
    return (dq, dk, dv), ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (2, 2)])
@pytest.mark.parametrize("Nq,Nk", [(300, 333), (256, 256), (77, 200), (200, 77), (1, 130), (130, 1)])
def test_bwd_shapes(d, causal, Hq, Hkv, Nq, Nk):
    q, k, v, do = backward_inputs(2, Hq, Hkv, Nq, Nk, d, torch.bfloat16, seed=Nq * 5 + Nk + d)
    (dq, _, _), _ = _check(q, k, v, do, causal, f"d={d} c={causal} H={Hq}/{Hkv} {Nq}x{Nk}")
    if causal and Nq > Nk:
        # rows Nq - Nk and below see no key: their gradient is exactly zero
        assert (dq[:, : Nq - Nk].float() == 0).all()


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_mqa_and_wide_groups(d):
    q, k, v, do = backward_inputs(1, 8, 1, 190, 260, d, torch.bfloat16, seed=31 + d)
    _check(q, k, v, do, True, f"MQA d={d}")


def test_bwd_scale_argument():
    q, k, v, do = backward_inputs(2, 4, 2, 160, 96, 64, torch.bfloat16, seed=5)
    _check(q, k, v, do, False, "scale 0.3", scale=0.3)


def test_bwd_strided_views():
    # q, k, v as slices of one packed [B, N, 3, H, d] tensor; gradients written
    # into slices of another
    B, N, H, d = 2, 150, 4, 128
    g = torch.Generator().manual_seed(17)
    qkv = torch.randn(B, N, 3, H, d, generator=g).to(torch.bfloat16).to(DEV)
    do = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16).to(DEV)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    o, lse = attn_fwd(q, k, v, causal=True)
    grad = torch.zeros(B, N, 3, H, d, dtype=torch.bfloat16, device=DEV)
    attn_bwd(q, k, v, o, lse, do, causal=True, dq=grad[:, :, 0], dk=grad[:, :, 1], dv=grad[:, :, 2])
    torch.cuda.synchronize()
    ref = oracle.attention_backward(to64(q), to64(k), to64(v), to64(do), 1 / math.sqrt(d), causal=True)
    for i, n in enumerate("QKV"):
        check_grad(grad[:, :, i], ref[i], f"strided d{n}")


def test_bwd_empty_sides():
    # no query rows: every key's gradient is zero; no keys: dQ is zero
    q, k, v, do = (t.to(DEV) for t in backward_inputs(2, 4, 2, 0, 70, 64, torch.bfloat16, seed=1))
    o = torch.empty_like(q)
    lse = torch.empty(2, 4, 0, dtype=torch.float32, device=DEV)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(v, 7.0)
    attn_bwd(q, k, v, o, lse, do, causal=True, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert (dk.float() == 0).all() and (dv.float() == 0).all()
    q, k, v, do = (t.to(DEV) for t in backward_inputs(2, 4, 2, 70, 0, 64, torch.bfloat16, seed=2))
    o, lse = attn_fwd(q, k, v)
    dq = torch.full_like(q, 7.0)
    attn_bwd(q, k, v, o, lse, do, dq=dq)
    torch.cuda.synchronize()
    assert (dq.float() == 0).all()


def test_bwd_bitwise_repeatable():
    q, k, v, do = (t.to(DEV) for t in backward_inputs(1, 8, 2, 333, 333, 128, torch.bfloat16, seed=3))
    o, lse = attn_fwd(q, k, v, causal=True)
    call, grads = prepare_bwd(q, k, v, o, lse, do, causal=True)
    call()
    torch.cuda.synchronize()
    first = [g.clone() for g in grads]
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    for a, b in zip(first, grads):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name,pieces", [
    ("gpt2-medium-causal-bwd", [(0, 0), (63, 15), (17, 6)]),  # (batch, head)
    ("llama3-8b-gqa-causal-8k-bwd", [(0, 3)]),                 # (batch, KV head)
])
def test_bwd_full_workload_sliced(name, pieces):
    w = WORKLOADS[name]
    ins = workload_inputs(w, device=DEV)
    q, k, v, do = ins["q"], ins["k"], ins["v"], ins["dout"]
    o, lse = attn_fwd(q, k, v, causal=w.causal)
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, causal=w.causal)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    for b, hk in pieces:
        hs = slice(hk * G, (hk + 1) * G)
        ref = oracle.attention_backward(to64(q[b:b + 1, :, hs]), to64(k[b:b + 1, :, hk:hk + 1]),
                                        to64(v[b:b + 1, :, hk:hk + 1]), to64(do[b:b + 1, :, hs]),
                                        w.scale, causal=w.causal)
        got = (dq[b:b + 1, :, hs], dk[b:b + 1, :, hk:hk + 1], dv[b:b + 1, :, hk:hk + 1])
        errs = [check_grad(g_, r, f"{name} b={b} kv={hk} d{n}") for g_, r, n in zip(got, ref, "QKV")]
        print(name, b, hk, " ".join(f"d{n} {e[0]:.2e}/{e[1]:.2e}" for n, e in zip("QKV", errs)))


def _block_mask(nqb, nkb, seed):
    """Random live blocks (about half), with one block row and one block column
    left entirely dead."""
    rng = np.random.default_rng(seed)
    bm = (rng.random((nqb, nkb)) < 0.5).astype(np.uint8)
    bm[nqb // 2, :] = 0
    bm[:, nkb // 3] = 0
    return bm


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(16, 16), (32, 48), (48, 16), (80, 80)])
def test_bwd_block_mask(d, causal, bq, bk):
    nqb, nkb = max(2, 288 // bq), max(2, 320 // bk)
    Nq, Nk = nqb * bq, nkb * bk
    bm = _block_mask(nqb, nkb, seed=bq * 100 + bk + d)
    q, k, v, do = backward_inputs(2, 4, 2, Nq, Nk, d, torch.bfloat16, seed=bq + bk + d)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = attn_fwd(qd, kd, vd, causal=causal, block_mask=bm, block=(bq, bk))
    grads = attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, block_mask=bm, block=(bq, bk))
    torch.cuda.synchronize()
    ref = oracle.attention_backward(to64(q), to64(k), to64(v), to64(do), 1 / math.sqrt(d),
                                    causal=causal, block_mask=bm, block_q=bq, block_k=bk)
    where = f"block {bq}x{bk} d={d} c={causal}"
    errs = [check_grad(g, r, f"{where} d{n}") for g, r, n in zip(grads, ref, "QKV")]
    print(where, " ".join(f"d{n} {e[0]:.2e}/{e[1]:.2e}" for n, e in zip("QKV", errs)))
    # rows of the dead block row see no key: exactly zero dQ
    r0 = (nqb // 2) * bq
    assert (grads[0][:, r0:r0 + bq].float() == 0).all()
    # keys of the dead block column are seen by no row: exactly zero dK, dV
    c0 = (nkb // 3) * bk
    assert (grads[1][:, c0:c0 + bk].float() == 0).all() and (grads[2][:, c0:c0 + bk].float() == 0).all()


def test_bwd_video_workload_one_head():
    w = WORKLOADS["video-frames-16x880-bwd"]
    ins = workload_inputs(w, device=DEV)
    q, k, v, do, bm = ins["q"], ins["k"], ins["v"], ins["dout"], ins["block_mask"]
    blk = (w.block, w.block)
    o, lse = attn_fwd(q, k, v, block_mask=bm, block=blk)
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, block_mask=bm, block=blk)
    torch.cuda.synchronize()
    h = 17
    ref = oracle.attention_backward(to64(q[:, :, h:h + 1]), to64(k[:, :, h:h + 1]),
                                    to64(v[:, :, h:h + 1]), to64(do[:, :, h:h + 1]), w.scale,
                                    block_mask=bm, block_q=w.block, block_k=w.block)
    got = (dq[:, :, h:h + 1], dk[:, :, h:h + 1], dv[:, :, h:h + 1])
    errs = [check_grad(g, r, f"video head {h} d{n}") for g, r, n in zip(got, ref, "QKV")]
    print("video", h, " ".join(f"d{n} {e[0]:.2e}/{e[1]:.2e}" for n, e in zip("QKV", errs)))


# Inf/NaN planted where the mask hides it from part of the rows: (tensor,
# index [b, row or key, head, dim] or None for every dim). Row 70 sees keys
# up to 102 and key 180 is seen from row 148 on (Nq = 200, Nk = 232).
_PLANTS = [("v", (0, 180, 1, 5)), ("do", (0, 70, 2, 9)), ("k", (0, 180, 1, None)),
           ("q", (0, 70, 3, None))]


def _planted(d, seed, plants, bad, Nq=200, Nk=232):
    q, k, v, do = backward_inputs(1, 4, 2, Nq, Nk, d, torch.bfloat16, seed=seed)
    t = {"q": q, "k": k, "v": v, "do": do}
    for name, (b, r, hh, e) in plants:
        t[name][b, r, hh, slice(None) if e is None else e] = bad
    return t["q"], t["k"], t["v"], t["do"]


def _check_nonfinite_grads(q, k, v, do, where, **mask):
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = attn_fwd(qd, kd, vd, **mask)
    grads = attn_bwd(qd, kd, vd, o, lse, dod, **mask)
    torch.cuda.synchronize()
    okw = {kk: vv for kk, vv in mask.items() if kk in ("causal", "block_mask")}
    if "block" in mask:
        okw["block_q"], okw["block_k"] = mask["block"]
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle.attention_backward(to64(q), to64(k), to64(v), to64(do),
                                        1 / math.sqrt(q.shape[-1]), **okw)
    errs = [check_grad_nonfinite(g, r, f"{where} d{n}") for g, r, n in zip(grads, ref, "QKV")]
    print(where, " ".join(f"d{n} {e[0]:.2e}/{e[1]:.2e}" for n, e in zip("QKV", errs)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("plant", range(len(_PLANTS)))
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_bwd_nonfinite_at_hidden_pairs(d, plant, bad):
    """An Inf or NaN in Q, K, V or dO reaches exactly the gradient entries an
    allowed pair connects it to, as in the oracle; rows and keys the causal
    rule keeps away from it are unaffected (mixed tiles recompute exactly the
    keys or rows whose accumulators turned non-finite)."""
    name = _PLANTS[plant][0]
    if bad == float("inf") and name in ("k", "q"):
        pytest.skip("Inf in K or Q: the scores' signs decide; NaN covers the path")
    q, k, v, do = _planted(d, 40 + plant, [_PLANTS[plant]], bad)
    _check_nonfinite_grads(q, k, v, do, f"causal d={d} {name}={bad}", causal=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_nonfinite_block_mask(d, causal):
    """The same with a block mask (blocks of 48 x 48 over 192 x 240, about half
    live, one dead block row and column), NaN in V (key 180, block column 3)
    and dO (row 70, block row 1)."""
    bm = _block_mask(4, 5, seed=d + causal)
    bm[2, 3] = bm[1, 0] = bm[1, 2] = 1
    q, k, v, do = _planted(d, 50, [_PLANTS[0], _PLANTS[1]], float("nan"), Nq=192, Nk=240)
    _check_nonfinite_grads(q, k, v, do, f"block c={causal} d={d}", causal=causal,
                           block_mask=bm, block=(48, 48))


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_nonfinite_without_mask(d):
    """No mask: every pair is visible, so NaN in V and dO reaches exactly the
    entries the oracle's chain rule sends it to (no fix-up kernel runs)."""
    q, k, v, do = _planted(d, 60, [_PLANTS[0], _PLANTS[1]], float("nan"))
    _check_nonfinite_grads(q, k, v, do, f"no mask d={d}", causal=False)


def _random_case(seed):
    """A seeded random backward problem: batch 1-2, KV heads 1-2, group 1-4,
    Nq and Nk in 1..400, d 64 or 128, causal or not, and a block mask with
    block sizes that divide the lengths on about a third of the cases."""
    rng = np.random.default_rng(1000 + seed)
    B, Hkv, G = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    if rng.random() < 0.35:
        bq, bk = (int(x) for x in rng.choice([16, 32, 48, 64], size=2))
        Nq, Nk = bq * int(rng.integers(1, 7)), bk * int(rng.integers(1, 7))
        bm = (rng.random((Nq // bq, Nk // bk)) < 0.6).astype(np.uint8)
        return B, Hkv, G, Nq, Nk, d, causal, bm, (bq, bk)
    Nq, Nk = int(rng.integers(1, 401)), int(rng.integers(1, 401))
    return B, Hkv, G, Nq, Nk, d, causal, None, None


@pytest.mark.parametrize("seed", range(24))
def test_bwd_random_shapes(seed):
    B, Hkv, G, Nq, Nk, d, causal, bm, blk = _random_case(seed)
    q, k, v, do = backward_inputs(B, Hkv * G, Hkv, Nq, Nk, d, torch.bfloat16, seed=seed)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = attn_fwd(qd, kd, vd, causal=causal, block_mask=bm, block=blk)
    grads = attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, block_mask=bm, block=blk)
    torch.cuda.synchronize()
    kw = {} if bm is None else dict(block_mask=bm, block_q=blk[0], block_k=blk[1])
    ref = oracle.attention_backward(to64(q), to64(k), to64(v), to64(do), 1 / math.sqrt(d),
                                    causal=causal, **kw)
    where = f"seed {seed}: B={B} Hkv={Hkv} G={G} Nq={Nq} Nk={Nk} d={d} causal={causal} block={blk}"
    errs = [check_grad(g, r, f"{where} d{n}") for g, r, n in zip(grads, ref, "QKV")]
    print(where, " ".join(f"d{n} {e[0]:.2e}/{e[1]:.2e}" for n, e in zip("QKV", errs)))


@pytest.mark.parametrize("Hq,Hkv,Nq,Nk,d,causal", [(2, 1, 512, 65536, 128, True),
                                                   (4, 2, 300, 40000, 64, False),
                                                   (2, 1, 65536, 512, 128, False),
                                                   (4, 2, 40000, 300, 64, True)])
def test_bwd_long_keys(Hq, Hkv, Nq, Nk, d, causal):
    """Long key ranges (512 key workgroups per head, loops of up to 1024 key
    tiles in dQ, 64-bit row offsets) and long query ranges (up to 2048 steps
    per key workgroup; causal with 39700 rows that see no key: dQ = 0 there),
    every gradient entry against the oracle."""
    _check(*backward_inputs(1, Hq, Hkv, Nq, Nk, d, torch.bfloat16, seed=Nk % 97), causal,
           f"long keys {Hq}/{Hkv} {Nq}x{Nk} d={d} causal={causal}")
