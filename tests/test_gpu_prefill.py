"""attn_fwd on the GPU against the fp64 oracle (element by element).

Small cases span several 128-row query tiles and 64-key tiles with ragged
tails; full-size workloads are checked on sampled rows and heads."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_attn_amd import attn_fwd
from exact_io_aware_attn_amd.inputs import WORKLOADS, frame_block_mask, prefill_inputs

from parity import check, sample_rows, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(q, k, v, **kw):
    o, lse = attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), **kw)
    torch.cuda.synchronize()
    return o, lse


def _ref(q, k, v, scale, **kw):
    return oracle.attention(to64(q), to64(k), to64(v), scale, **kw)


def _lse_ref_layout(L):
    return L  # oracle LSE is [B, H, Nq], as the library's


# ------------------------------------------------------------------ tiny fp32
def test_tiny_f32_workload():
    w = WORKLOADS["tiny-f32"]
    q, k, v = prefill_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, torch.float32, w.seed)
    o, lse = _run(q, k, v)
    O, L = _ref(q, k, v, w.scale)
    check(o, O, lse, L, dtype="f32", where="tiny-f32")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_f32_ragged(causal, d):
    q, k, v = prefill_inputs(2, 4, 2, 200, 233, d, torch.float32, seed=11)
    o, lse = _run(q, k, v, causal=causal)
    O, L = _ref(q, k, v, 1 / math.sqrt(d), causal=causal)
    check(o, O, lse, L, dtype="f32", where=f"f32 d={d} causal={causal}")


# ------------------------------------------------------------------ bf16, small
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (4, 1), (2, 2)])
@pytest.mark.parametrize("Nq,Nk", [(300, 333), (256, 256), (77, 200), (200, 77), (1, 130)])
def test_bf16_shapes(d, causal, Hq, Hkv, Nq, Nk):
    q, k, v = prefill_inputs(2, Hq, Hkv, Nq, Nk, d, torch.bfloat16, seed=Nq * 7 + Nk + d)
    o, lse = _run(q, k, v, causal=causal)
    O, L = _ref(q, k, v, 1 / math.sqrt(d), causal=causal)
    check(o, O, lse, L, where=f"bf16 d={d} causal={causal} H={Hq}/{Hkv} N={Nq}x{Nk}")


@pytest.mark.parametrize("mode", ["online", "fixed_max"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_eight_wave_workgroups_ragged(d, causal, mode):
    """Enough (batch, head) pairs that the 256-row, 8-wave workgroups are used
    (>= 1024 of them), with ragged query and key tails and GQA. Dense causal
    d = 64 takes 4-wave workgroups at every size, so that case runs the
    4-wave kernel with many workgroups in flight."""
    B, Hq, Hkv, Nq, Nk = 32, 16, 4, 300, 333
    q, k, v = prefill_inputs(B, Hq, Hkv, Nq, Nk, d, torch.bfloat16, seed=d + causal)
    o, lse = _run(q, k, v, causal=causal, softmax=mode)
    heads = [0, 7, 15]
    O, L = _ref(q, k, v, 1 / math.sqrt(d), causal=causal, heads=heads)
    check(o[:, :, heads], O, lse[:, heads], L, where=f"8-wave d={d} causal={causal} {mode}")


@pytest.mark.parametrize("mode", ["online", "fixed_max"])
@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,causal", [
    (1, 4, 2, 333, 700, True),     # odd number of key tiles (11): shares of 6 and 5
    (2, 3, 1, 257, 1000, False),   # MQA, ragged key tail
    (1, 2, 2, 700, 333, True),     # Nq > Nk: the first 367 rows see no key
    (1, 8, 8, 1500, 1500, True),   # long rows, several 64-row workgroups per head
])
def test_bf16_key_split(B, Hq, Hkv, Nq, Nk, causal, mode):
    """d = 64 problems with few workgroups split each row's keys between two
    waves and merge their (m, l, O): every row against the oracle."""
    q, k, v = prefill_inputs(B, Hq, Hkv, Nq, Nk, 64, torch.bfloat16, seed=Nq + Nk + Hq)
    o, lse = _run(q, k, v, causal=causal, softmax=mode)
    O, L = _ref(q, k, v, 1 / 8.0, causal=causal)
    check(o, O, lse, L, where=f"key split {mode} B={B} H={Hq}/{Hkv} N={Nq}x{Nk} causal={causal}")


@pytest.mark.parametrize("mode", ["online", "fixed_max"])
def test_bf16_eight_wave_frame_mask(mode):
    frames, flen, blk = 5, 128, 64
    n = frames * flen
    bm = frame_block_mask(frames, flen, blk)
    q, k, v = prefill_inputs(16, 32, 32, n, n, 128, torch.bfloat16, seed=21)
    o, lse = _run(q, k, v, block_mask=bm, block=(blk, blk), softmax=mode)
    heads = [0, 31]
    O, L = _ref(q[:2], k[:2], v[:2], 1 / math.sqrt(128), block_mask=bm, block_q=blk, block_k=blk,
                heads=heads)
    check(o[:2][:, :, heads], O, lse[:2][:, heads], L, where=f"8-wave frames {mode}")


@pytest.mark.parametrize("mode", ["fixed_max", "fixed_max_centered"])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_fixed_max(mode, causal):
    q, k, v = prefill_inputs(1, 4, 2, 260, 300, 128, torch.bfloat16, seed=5)
    o, lse = _run(q, k, v, causal=causal, softmax=mode)
    O, L = _ref(q, k, v, 1 / math.sqrt(128), causal=causal)
    check(o, O, lse, L, where=f"{mode} causal={causal}")


def test_bf16_fixed_max_shifted_keys_centered():
    """Keys with a large common offset: the centred bound stays eligible."""
    q, k, v = prefill_inputs(1, 2, 1, 192, 256, 128, torch.bfloat16, seed=6)
    k = (k.float() + 2.0).to(torch.bfloat16)
    for mode in ("fixed_max", "fixed_max_centered"):
        o, lse = _run(q, k, v, softmax=mode)
        O, L = _ref(q, k, v, 1 / math.sqrt(128))
        check(o, O, lse, L, where=mode)


def test_bf16_fixed_max_fallback_with_scaled_queries():
    """Q x10 makes the bound far too loose (gap > 87 nats): the rule must fall
    back to the running max, and the result must still meet the band (without
    the fallback the row sums underflow and LSE is wrong). Q x10 makes each
    row's softmax nearly one-hot, so O is nearly a single V row; V is scaled
    by 1/4 to keep |O| in the range the bf16 band is stated for (bf16 rounding
    of P and of O alone reaches 1e-2 at |O| ~ 4)."""
    q, k, v = prefill_inputs(1, 2, 2, 320, 320, 128, torch.bfloat16, seed=7)
    q = (q.float() * 10).to(torch.bfloat16)
    v = (v.float() * 0.25).to(torch.bfloat16)
    o, lse = _run(q, k, v, softmax="fixed_max")
    O, L = _ref(q, k, v, 1 / math.sqrt(128))
    check(o, O, lse, L, where="fallback")


def test_f32_fixed_max():
    q, k, v = prefill_inputs(1, 2, 1, 150, 170, 64, torch.float32, seed=8)
    for mode in ("fixed_max", "fixed_max_centered"):
        o, lse = _run(q, k, v, causal=True, softmax=mode)
        O, L = _ref(q, k, v, 1 / 8, causal=True)
        check(o, O, lse, L, dtype="f32", where=mode)


# ------------------------------------------------------------------ block masks
@pytest.mark.parametrize("bq,bk", [(16, 16), (32, 48), (80, 80), (64, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_random_block_mask(bq, bk, causal):
    Nq, Nk = 4 * bq * (2 if bq < 64 else 1), 5 * bk
    rng = np.random.default_rng(bq + bk)
    bm = (rng.random((Nq // bq, Nk // bk)) < 0.45).astype(np.uint8)
    bm[0, 0] = 1
    q, k, v = prefill_inputs(1, 4, 2, Nq, Nk, 128, torch.bfloat16, seed=bq * bk)
    o, lse = _run(q, k, v, causal=causal, block_mask=bm, block=(bq, bk))
    O, L = _ref(q, k, v, 1 / math.sqrt(128), causal=causal, block_mask=bm, block_q=bq, block_k=bk)
    check(o, O, lse, L, where=f"block {bq}x{bk} causal={causal}")


def _runs_mask(rng, nqb, nkb, max_run):
    """Block mask whose rows come in runs of identical rows (1..max_run long),
    each run with its own random row; every run sees at least one block."""
    rows, lens = [], []
    while len(rows) < nqb:
        n = min(int(rng.integers(1, max_run + 1)), nqb - len(rows))
        r = (rng.random(nkb) < 0.5).astype(np.uint8)
        r[int(rng.integers(0, nkb))] = 1
        rows += [r] * n
        lens.append(n)
    return np.stack(rows), lens


@pytest.mark.parametrize("mode", ["online", "fixed_max"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(16, 32), (48, 16), (80, 80)])
def test_bf16_block_mask_runs_of_identical_rows(bq, bk, causal, mode):
    """Block rows with identical mask rows share 32-row segments (a segment
    may span two or three block rows of one run, never two runs): runs of
    1..4 block rows, so segments end mid-block-row and runs end mid-segment.
    Every row against the oracle."""
    rng = np.random.default_rng(bq * 7 + bk + causal)
    nqb = max(1536 // bq, 30)
    nkb = 6 * 80 // bk
    bm, lens = _runs_mask(rng, nqb, nkb, 4)
    assert len(lens) > 5 and max(lens) > 1
    Nq, Nk = nqb * bq, nkb * bk
    q, k, v = prefill_inputs(1, 4, 2, Nq, Nk, 128, torch.bfloat16, seed=bq + bk)
    o, lse = _run(q, k, v, causal=causal, block_mask=bm, block=(bq, bk), softmax=mode)
    O, L = _ref(q, k, v, 1 / math.sqrt(128), causal=causal, block_mask=bm, block_q=bq, block_k=bk)
    check(o, O, lse, L, where=f"runs {bq}x{bk} causal={causal} {mode}")


@pytest.mark.parametrize("bq", [48, 80])
def test_bf16_block_mask_runs_eight_wave(bq):
    """The same with enough (batch, head) pairs for 8-wave workgroups, which
    may span the end of one run and the start of the next."""
    rng = np.random.default_rng(bq)
    nqb, nkb = 960 // bq, 12
    bm, _ = _runs_mask(rng, nqb, nkb, 4)
    Nq, Nk = nqb * bq, nkb * 64
    q, k, v = prefill_inputs(16, 16, 4, Nq, Nk, 64, torch.bfloat16, seed=bq)
    o, lse = _run(q, k, v, block_mask=bm, block=(bq, 64))
    heads = [0, 9, 15]
    O, L = _ref(q[:2], k[:2], v[:2], 1 / 8, block_mask=bm, block_q=bq, block_k=64, heads=heads)
    check(o[:2][:, :, heads], O, lse[:2][:, heads], L, where=f"runs 8-wave bq={bq}")


def test_f32_block_mask():
    rng = np.random.default_rng(3)
    bm = (rng.random((6, 5)) < 0.5).astype(np.uint8)
    q, k, v = prefill_inputs(1, 2, 1, 96, 80, 64, torch.float32, seed=9)
    o, lse = _run(q, k, v, block_mask=bm, block=(16, 16))
    O, L = _ref(q, k, v, 1 / 8, block_mask=bm, block_q=16, block_k=16)
    check(o, O, lse, L, dtype="f32", where="f32 block")


@pytest.mark.parametrize("mode", ["online", "fixed_max"])
def test_bf16_frame_mask_small(mode):
    frames, flen, blk = 6, 160, 80
    n = frames * flen
    bm = frame_block_mask(frames, flen, blk)
    q, k, v = prefill_inputs(1, 3, 3, n, n, 128, torch.bfloat16, seed=10)
    o, lse = _run(q, k, v, block_mask=bm, block=(blk, blk), softmax=mode)
    O, L = _ref(q, k, v, 1 / math.sqrt(128), block_mask=bm, block_q=blk, block_k=blk)
    check(o, O, lse, L, where=f"frames {mode}")


# ------------------------------------------------------------------ edge cases
def test_no_keys_gives_zero_and_minus_inf():
    q, k, v = prefill_inputs(1, 2, 2, 40, 0, 64, torch.bfloat16, seed=1)
    o, lse = _run(q, k, v)
    assert (o.float() == 0).all() and torch.isneginf(lse).all()


def test_empty_rows_from_block_mask():
    bm = np.ones((4, 2), dtype=np.uint8)
    bm[2, :] = 0
    q, k, v = prefill_inputs(1, 2, 2, 64, 32, 64, torch.bfloat16, seed=2)
    o, lse = _run(q, k, v, block_mask=bm, block=(16, 16))
    O, L = _ref(q, k, v, 1 / 8, block_mask=bm, block_q=16, block_k=16)
    check(o, O, lse, L, where="empty rows")
    assert (o[:, 32:48].float() == 0).all()


@pytest.mark.parametrize("mode", ["online", "fixed_max", "fixed_max_centered"])
def test_single_key_returns_value_row_exactly(mode):
    q, k, v = prefill_inputs(1, 2, 1, 50, 1, 128, torch.bfloat16, seed=3)
    o, _ = _run(q, k, v, softmax=mode)
    assert torch.equal(o.cpu(), v.expand(1, 50, 2, 128).contiguous())


@pytest.mark.parametrize("mode", ["online", "fixed_max"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", [(1, 4, 300), (32, 16, 300), (1, 8, 1500)])
def test_first_causal_row_returns_first_value_row_exactly(mode, d, B, H, N):
    """Row 0 of a causal problem sees key 0 only, so O[0] = V[0] exactly in
    every kernel configuration (4- and 8-wave workgroups, key split) and in
    the fixed-max mode too, where the weight is a rounded value below 1."""
    q, k, v = prefill_inputs(B, H, H, N, N, d, torch.bfloat16, seed=N + d + B)
    o, lse = _run(q, k, v, causal=True, softmax=mode)
    assert torch.equal(o[:, 0].cpu(), v[:, 0])


def test_identical_keys_return_mean_value():
    q, k, v = prefill_inputs(1, 1, 1, 64, 96, 64, torch.bfloat16, seed=4)
    k = k[:, :1].expand(1, 96, 1, 64).contiguous()
    o, _ = _run(q, k, v)
    mean = to64(v)[0, :, 0].mean(axis=0)
    assert np.abs(to64(o)[0, :, 0] - mean).max() <= 1e-2


def test_joint_key_permutation():
    q, k, v = prefill_inputs(1, 2, 2, 128, 192, 64, torch.bfloat16, seed=5)
    perm = torch.randperm(192, generator=torch.Generator().manual_seed(0))
    o1, l1 = _run(q, k, v)
    o2, l2 = _run(q, k[:, perm], v[:, perm])
    O, L = _ref(q, k, v, 1 / 8)
    check(o1, O, l1, L, where="unpermuted")
    check(o2, O, l2, L, where="permuted")


def test_strided_views():
    """q, k, v as views into a packed [B, N, 3, H, d] tensor; o into a wider buffer."""
    B, N, H, d = 2, 150, 4, 64
    g = torch.Generator().manual_seed(12)
    qkv = torch.randn(B, N, 3, H, d, generator=g).to(torch.bfloat16).to(DEV)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    obuf = torch.zeros(B, N, H, 2 * d, dtype=torch.bfloat16, device=DEV)
    o, lse = attn_fwd(q, k, v, causal=True, out=obuf[..., :d])
    torch.cuda.synchronize()
    O, L = _ref(q, k, v, 1 / 8, causal=True)
    check(obuf[..., :d], O, lse, L, where="strided")
    assert (obuf[..., d:].float() == 0).all()


def test_repeatable_bitwise():
    q, k, v = prefill_inputs(1, 4, 2, 256, 256, 128, torch.bfloat16, seed=13)
    o1, l1 = _run(q, k, v, causal=True)
    o2, l2 = _run(q, k, v, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------ masked positions
def test_causal_future_keys_are_excluded_bitwise():
    """Changing keys/values j > t (to other finite values) leaves rows i <= t
    bit-identical: excluded pairs contribute exactly nothing."""
    q, k, v = prefill_inputs(1, 2, 2, 256, 256, 128, torch.bfloat16, seed=14)
    t = 150
    k2, v2 = k.clone(), v.clone()
    k2[:, t + 1:] = (k2[:, t + 1:].float() * 3 + 1).to(torch.bfloat16)
    v2[:, t + 1:] = (v2[:, t + 1:].float() * -2 + 5).to(torch.bfloat16)
    o1, l1 = _run(q, k, v, causal=True)
    o2, l2 = _run(q, k2, v2, causal=True)
    assert torch.equal(o1[:, :t + 1], o2[:, :t + 1])
    assert torch.equal(l1[:, :, :t + 1], l2[:, :, :t + 1])


@pytest.mark.parametrize("frames,flen,blk,heads,g", [
    (5, 128, 64, 2, 3),      # block rows a multiple of 32
    (6, 48, 48, 4, 3),       # block rows of 48: 32 + 16-row segments
    (16, 880, 80, 2, 7),     # the video shape, 4-wave workgroups
    (16, 880, 80, 24, 7),    # the video shape, 8-wave workgroups
])
@pytest.mark.parametrize("mode", ["online", "fixed_max"])
def test_dead_block_nan_never_read(mode, frames, flen, blk, heads, g):
    """NaN in the keys/values of key frame g: queries whose frames do not
    attend it are bit-identical to the clean run and finite, including block
    rows (80, 48) that are not a multiple of 32 rows.

    The fixed-max bound is a per-head statistic over all keys, so the frame's
    keys are scaled down in both runs: they never set max |k|, and NaN rows
    are ignored by that max, so the bound is the same in both runs."""
    n = frames * flen
    bm = frame_block_mask(frames, flen, blk)
    q, k, v = prefill_inputs(1, heads, heads, n, n, 128, torch.bfloat16, seed=15)
    k[:, g * flen:(g + 1) * flen] = (k[:, g * flen:(g + 1) * flen].float() * 0.25).to(torch.bfloat16)
    o1, l1 = _run(q, k, v, block_mask=bm, block=(blk, blk), softmax=mode)
    k2, v2 = k.clone(), v.clone()
    k2[:, g * flen:(g + 1) * flen] = float("nan")
    v2[:, g * flen:(g + 1) * flen] = float("nan")
    o2, l2 = _run(q, k2, v2, block_mask=bm, block=(blk, blk), softmax=mode)
    for f in range(frames):
        rows = slice(f * flen, (f + 1) * flen)
        if abs(f - g) <= 1:
            assert torch.isnan(o2[:, rows].float()).any(), f  # frame f attends g
            continue
        assert torch.equal(o1[:, rows], o2[:, rows]), f
        assert torch.equal(l1[:, :, rows], l2[:, :, rows]), f
        assert torch.isfinite(o2[:, rows].float()).all()


# ------------------------------------------------------------------ full-size workloads
def _full(name, mode="online", rows_per_head=None, heads=None):
    w = WORKLOADS[name]
    ins = {}
    q, k, v = prefill_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, torch.bfloat16, w.seed, device=DEV)
    bm = frame_block_mask(w.frames, w.frame_len, w.block) if w.frames else None
    kw = dict(causal=w.causal, softmax=mode)
    if bm is not None:
        kw.update(block_mask=bm, block=(w.block, w.block))
    o, lse = attn_fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    bounds = list(range(w.frame_len, w.Nq, w.frame_len)) if w.frames else []
    rows = sample_rows(w.Nq, boundaries=bounds, seed=w.seed)
    heads = list(range(w.Hq)) if heads is None else heads
    ok = dict(block_mask=bm, block_q=w.block or None, block_k=w.block or None) if bm is not None else {}
    rt = torch.as_tensor(rows, device=DEV)
    ht = torch.as_tensor(heads, device=DEV)
    for b in range(w.B):
        O, L = oracle.attention(to64(q[b:b + 1]), to64(k[b:b + 1]), to64(v[b:b + 1]), w.scale,
                                causal=w.causal, heads=heads, rows=rows, **ok)
        check(o[b:b + 1][:, rt][:, :, ht], O, lse[b:b + 1][:, ht][:, :, rt], L,
              where=f"{name} {mode} b={b}")


def test_full_gpt2_causal():
    _full("gpt2-causal", heads=[0, 5, 11])


def test_full_gpt2_medium_causal():
    _full("gpt2-medium-causal", heads=[0, 9, 15])


def test_full_llama3_8b_gqa_causal():
    _full("llama3-8b-gqa-causal-8k", heads=[0, 3, 4, 17, 31])


@pytest.mark.parametrize("mode", ["online", "fixed_max"])
def test_full_video_frames(mode):
    _full("video-frames-16x880", mode=mode, heads=[0, 13, 23])


@pytest.mark.parametrize("mode", ["fixed_max", "fixed_max_centered"])
def test_bf16_fixed_max_causal_large_late_keys(mode):
    # the last 64 keys are 3x longer: with a bound over every key the early
    # 32-row groups' gap (about 2 scale |q| max|k| = 84 nats) exceeds the 64-nat
    # limit; under the causal rule only the last rows see those keys, so the
    # bound over the splits a wave can see keeps the early groups eligible.
    # Their values are shrunk so the peaked last rows keep outputs of moderate
    # size (the bf16 rounding of a large output would dominate the error).
    q, k, v = prefill_inputs(2, 4, 2, 700, 700, 128, torch.bfloat16, seed=77)
    k[:, -64:] = (k[:, -64:].float() * 3).to(torch.bfloat16)
    v[:, -64:] = (v[:, -64:].float() * 0.25).to(torch.bfloat16)
    o, lse = _run(q, k, v, causal=True, softmax=mode)
    O, L = _ref(q, k, v, 1 / math.sqrt(128), causal=True)
    check(o, O, lse, L, where=f"{mode} causal large late keys")
