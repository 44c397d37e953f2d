"""attn_fwd on the GPU against the fp64 oracle (element by element).

Small cases span several 128-row query tiles and 64-key tiles with ragged
tails; the full-size workloads are checked on every row (of every head, or
of eight heads for the video workload); 65536-key sequences on sampled rows."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_attn_amd import attn_fwd, attn_fwd_workspace_bytes, fixed_max_decisions
from exact_io_aware_attn_amd.inputs import WORKLOADS, frame_block_mask, prefill_inputs

from parity import check, check_nonfinite, sample_rows, to64

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


@pytest.mark.parametrize("v_scale", [0.25, 1.0])
@pytest.mark.parametrize("mode", ["online", "fixed_max", "fixed_max_centered"])
def test_bf16_scaled_queries_peaked_rows(mode, v_scale):
    """Q x10 makes every row's softmax nearly one-hot, so O is nearly a single
    V row, and the fixed-max bound far too loose (gap > 87 nats): every row
    must fall back to the running max, and the result must still be exact
    (without the fallback the row sums underflow and the LSE is wrong).
    With V x1/4 |O| stays below 2 and the band applies; with V as drawn |O*|
    reaches 4 and more, and the bound for rows dominated by a few keys
    applies (see parity.py).
    The sum of the rounded weights divides O, so a row dominated by one key
    adds no error of its own on top of that rounding."""
    q, k, v = prefill_inputs(1, 2, 2, 320, 320, 128, torch.bfloat16, seed=7)
    q = (q.float() * 10).to(torch.bfloat16)
    v = (v.float() * v_scale).to(torch.bfloat16)
    o, lse = _run(q, k, v, softmax=mode)
    O, L = _ref(q, k, v, 1 / math.sqrt(128))
    if v_scale == 1:
        assert np.abs(O).max() > 3.5  # the case is reached
    check(o, O, lse, L, where=f"peaked {mode}", peaked=v_scale == 1)


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
@pytest.mark.parametrize("mode", ["online", "fixed_max", "fixed_max_centered"])
@pytest.mark.parametrize("B,Hq,Hkv,N,d,t", [
    (1, 2, 2, 256, 128, 150),     # 4-wave workgroups; row 150 inside a 32-row group
    (32, 16, 4, 300, 128, 140),   # 8-wave workgroups, GQA
    (1, 8, 8, 1500, 64, 777),     # d = 64, keys split between two waves
    (2, 4, 2, 700, 64, 400),      # d = 64, 4-wave workgroups
])
def test_causal_future_keys_are_excluded_bitwise(mode, B, Hq, Hkv, N, d, t):
    """Changing keys/values j > t (to other finite values: keys 8x longer and
    shifted, so the later rows' bounds, fallbacks and rescales change) leaves
    rows i <= t bit-identical in every softmax mode: excluded pairs contribute
    exactly nothing, and every decision a row's arithmetic depends on comes
    from its own visible keys. In the fixed-max modes rows 0..t keep the
    fixed max in both runs."""
    q, k, v = prefill_inputs(B, Hq, Hkv, N, N, d, torch.bfloat16, seed=14 + N + d)
    k2, v2 = k.clone(), v.clone()
    k2[:, t + 1:] = (k2[:, t + 1:].float() * 8 + 1).to(torch.bfloat16)
    v2[:, t + 1:] = (v2[:, t + 1:].float() * -2 + 5).to(torch.bfloat16)
    ws1, ws2 = _workspace(B, Hq, Hkv, N, N, d, mode), _workspace(B, Hq, Hkv, N, N, d, mode)
    o1, l1 = _run(q, k, v, causal=True, softmax=mode, workspace=ws1)
    o2, l2 = _run(q, k2, v2, causal=True, softmax=mode, workspace=ws2)
    assert torch.equal(o1[:, :t + 1], o2[:, :t + 1])
    assert torch.equal(l1[:, :, :t + 1], l2[:, :, :t + 1])
    if mode != "online":
        f1 = fixed_max_decisions(ws1, B, Hq, Hkv, N, N)
        f2 = fixed_max_decisions(ws2, B, Hq, Hkv, N, N)
        m = oracle.MIN_KEYS - 1  # rows before it see less than one key tile
        assert torch.equal(f1[:, :, :t + 1], f2[:, :, :t + 1])
        assert bool((f1[:, :, m:t + 1] == 1).all()) and bool((f1[:, :, :m] == 0).all())
        assert bool((f2[:, :, t + 1:] == 0).any())  # the longer keys moved later rows


def check_decisions(flags, q, k, mode, margin=0.05, **mask):
    """The kernel's per-row choice (fixed max or fallback) against the oracle's
    eligibility rule (fixed_max_bounds): equal on every row whose gap lies
    more than `margin` nats from tau (float32 sums may decide the rest either
    way; they must be few)."""
    M, gap, el = oracle.fixed_max_bounds(to64(q), to64(k), 1 / math.sqrt(q.shape[-1]),
                                         centered=mode == "fixed_max_centered", **mask)
    flags = np.asarray(flags)
    assert flags.shape == el.shape
    assert set(np.unique(flags)) <= {0, 1}
    clear = ~(np.abs(np.nan_to_num(gap, nan=np.inf) - oracle.TAU) <= margin)
    assert clear.mean() > 0.99
    bad = np.argwhere(((flags == 1) != el) & clear)
    assert bad.size == 0, f"{len(bad)} decisions differ, first {bad[:5].tolist()}"


def _workspace(B, Hq, Hkv, Nq, Nk, d, mode, mask_kind=1, bq=0, bk=0):
    from exact_io_aware_attn_amd.binding import SOFTMAX_MODES
    n = attn_fwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, mask_kind, bq, bk, SOFTMAX_MODES[mode])
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
@pytest.mark.parametrize("mode", ["online", "fixed_max", "fixed_max_centered"])
@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d", [
    (1, 4, 2, 300, 300, 128),     # 4-wave workgroups
    (32, 16, 4, 300, 300, 128),   # 8-wave workgroups
    (1, 4, 4, 520, 520, 64),      # keys split between two waves
    (2, 4, 2, 200, 333, 64),      # Nq != Nk, ragged key tail
])
def test_nonfinite_v_at_causal_masked_keys(B, Hq, Hkv, Nq, Nk, d, mode, bad):
    """Inf or NaN in V at keys inside diagonal tiles (some rows of a wave see
    them, some do not): a row that cannot see such a key gets the same
    result as with finite values there, a row that sees it propagates it in
    that value's columns, as the oracle (which sums over visible keys only)."""
    q, k, v = prefill_inputs(B, Hq, Hkv, Nq, Nk, d, torch.bfloat16, seed=Nk + d + B)
    for t, cols in ((Nk // 2 + 5, slice(0, 8)), (Nk - 40, slice(d - 4, d))):
        v[:, t, :, cols] = bad
    ws = _workspace(B, Hq, Hkv, Nq, Nk, d, mode, 1)
    o, lse = attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, softmax=mode, workspace=ws)
    torch.cuda.synchronize()
    O, L = _ref(q, k, v, 1 / math.sqrt(d), causal=True)
    check_nonfinite(o, O, lse, L, f"{mode} {bad} B={B} H={Hq}/{Hkv} {Nq}x{Nk} d={d}")


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_nonfinite_v_causal_block_mask(bad):
    """The same with a random block mask on top of the causal rule."""
    rng = np.random.default_rng(11)
    bq, bk = 48, 32
    Nq, Nk = 12 * bq, 18 * bk
    bm = (rng.random((Nq // bq, Nk // bk)) < 0.6).astype(np.uint8)
    bm[:, 0] = 1
    q, k, v = prefill_inputs(1, 4, 2, Nq, Nk, 128, torch.bfloat16, seed=12)
    for t in (5 * bk + 7, 11 * bk + 20, Nk - 3):
        v[:, t, :, 0:16] = bad
    o, lse = attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, block_mask=bm, block=(bq, bk))
    torch.cuda.synchronize()
    O, L = _ref(q, k, v, 1 / math.sqrt(128), causal=True, block_mask=bm, block_q=bq, block_k=bk)
    check_nonfinite(o, O, lse, L, f"block+causal {bad}")


@pytest.mark.parametrize("frames,flen,blk,heads,g", [
    (5, 128, 64, 2, 3),      # block rows a multiple of 32
    (6, 48, 48, 4, 3),       # block rows of 48: 32 + 16-row segments
    (16, 880, 80, 2, 7),     # the video shape, 4-wave workgroups
    (16, 880, 80, 24, 7),    # the video shape, 8-wave workgroups
])
@pytest.mark.parametrize("mode", ["online", "fixed_max", "fixed_max_centered"])
@pytest.mark.parametrize("poison", ["nan", "long_keys"])
def test_dead_block_nan_never_read(mode, poison, frames, flen, blk, heads, g):
    """Key frame g gets NaN keys/values, or finite keys 3x longer (and shifted)
    with other values: queries whose frames do not attend it are
    bit-identical to the clean run and finite, in every softmax mode,
    including block rows (80, 48) that are not a multiple of 32 rows. The
    fixed-max bound of a row comes from the key blocks it sees, so the
    frame's keys never enter the bound of a frame that does not attend it."""
    n = frames * flen
    bm = frame_block_mask(frames, flen, blk)
    q, k, v = prefill_inputs(1, heads, heads, n, n, 128, torch.bfloat16, seed=15)
    o1, l1 = _run(q, k, v, block_mask=bm, block=(blk, blk), softmax=mode)
    k2, v2 = k.clone(), v.clone()
    fr = slice(g * flen, (g + 1) * flen)
    if poison == "nan":
        k2[:, fr] = float("nan")
        v2[:, fr] = float("nan")
    else:
        k2[:, fr] = (k2[:, fr].float() * 3 + 0.5).to(torch.bfloat16)
        v2[:, fr] = (v2[:, fr].float() * -2 + 3).to(torch.bfloat16)
    o2, l2 = _run(q, k2, v2, block_mask=bm, block=(blk, blk), softmax=mode)
    for f in range(frames):
        rows = slice(f * flen, (f + 1) * flen)
        if abs(f - g) <= 1 or g == 0:
            if poison == "nan":
                assert torch.isnan(o2[:, rows].float()).any(), f  # frame f attends g
            continue
        assert torch.equal(o1[:, rows], o2[:, rows]), f
        assert torch.equal(l1[:, :, rows], l2[:, :, rows]), f
        assert torch.isfinite(o2[:, rows].float()).all()


# ------------------------------------------------------------------ full-size workloads
def _full(name, mode="online", heads=None):
    """The workload at its full size, in the launch configuration the bench
    times, against the oracle on every row of the given query heads (all by
    default); in the fixed-max modes the per-row decisions against the
    oracle's rule as well."""
    w = WORKLOADS[name]
    q, k, v = prefill_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, torch.bfloat16, w.seed, device=DEV)
    bm = frame_block_mask(w.frames, w.frame_len, w.block) if w.frames else None
    kw = dict(causal=w.causal, softmax=mode)
    mask = dict(causal=w.causal)
    if bm is not None:
        kw.update(block_mask=bm, block=(w.block, w.block))
        mask.update(block_mask=bm, block_q=w.block, block_k=w.block)
    kind = (1 if w.causal else 0) | (2 if bm is not None else 0)
    ws = _workspace(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, mode, kind, w.block, w.block)
    o, lse = attn_fwd(q, k, v, workspace=ws, **kw)
    torch.cuda.synchronize()
    heads = list(range(w.Hq)) if heads is None else heads
    ht = torch.as_tensor(heads, device=DEV)
    for b in range(w.B):
        qb, kb, vb = to64(q[b:b + 1]), to64(k[b:b + 1]), to64(v[b:b + 1])
        O, L = oracle.attention(qb, kb, vb, w.scale, heads=heads, **mask)
        check(o[b:b + 1][:, :, ht], O, lse[b:b + 1][:, ht], L, where=f"{name} {mode} b={b}")
    if mode != "online":
        f = fixed_max_decisions(ws, w.B, w.Hq, w.Hkv, w.Nq, w.Nk)[:, ht].cpu().numpy()
        # the oracle's rule over the same heads, each with its own KV head
        g = w.Hq // w.Hkv
        ks = k.cpu()[:, :, [h // g for h in heads]]
        check_decisions(f, q[:, :, ht].cpu(), ks, mode, **mask)


def test_full_gpt2_causal():
    _full("gpt2-causal")


def test_full_gpt2_medium_causal():
    _full("gpt2-medium-causal")


def test_full_llama3_8b_gqa_causal():
    _full("llama3-8b-gqa-causal-8k")


@pytest.mark.parametrize("mode", ["online", "fixed_max", "fixed_max_centered"])
def test_full_video_frames(mode):
    _full("video-frames-16x880", mode=mode, heads=[0, 3, 6, 9, 12, 15, 19, 23])


@pytest.mark.parametrize("mode", ["fixed_max", "fixed_max_centered"])
def test_full_llama3_8b_gqa_causal_fixed_max(mode):
    _full("llama3-8b-gqa-causal-8k", mode=mode, heads=[0, 1, 2, 3, 17, 30, 31])


@pytest.mark.parametrize("mode", ["online", "fixed_max"])
@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d", [
    (1, 2, 1, 65536, 65536, 128),   # 8-wave workgroups, 1024 key tiles per late row
    (1, 4, 2, 700, 65573, 64),      # a short query block at the end of a ragged long key range
])
def test_long_sequence_sampled_rows(mode, B, Hq, Hkv, Nq, Nk, d):
    """Causal prefill over 65536 keys: sampled rows (tile edges, first and last,
    random) against the oracle, each row given exactly the keys the causal
    rule lets it see (the row alone as the query, keys 0 .. i + Nk - Nq, no
    mask), so no N x N reference is formed."""
    q, k, v = prefill_inputs(B, Hq, Hkv, Nq, Nk, d, torch.bfloat16, seed=Nq + d, device=DEV)
    ws = _workspace(B, Hq, Hkv, Nq, Nk, d, mode, 1)
    o, lse = attn_fwd(q, k, v, causal=True, softmax=mode, workspace=ws)
    torch.cuda.synchronize()
    qc, kc, vc, oc, lc = (t.cpu() for t in (q, k, v, o, lse))
    scale = 1 / math.sqrt(d)
    for r in sample_rows(Nq, tile=256, extra=12, seed=d):
        last = r + Nk - Nq
        O, L = oracle.attention(to64(qc[:, r:r + 1]), to64(kc[:, :last + 1]), to64(vc[:, :last + 1]),
                                scale)
        check(oc[:, r:r + 1], O, lc[:, :, r:r + 1], L, where=f"{mode} Nq={Nq} Nk={Nk} row {r}")


@pytest.mark.parametrize("mode", ["fixed_max", "fixed_max_centered"])
def test_bf16_fixed_max_causal_large_late_keys(mode):
    """The last 64 keys are 8x longer: a bound over every key would put the
    early rows' gap near 100 nats, past the 64-nat limit; under the causal
    rule only the last rows see those keys, so the bound over the key blocks
    each row sees keeps the earlier rows (from the first one that sees a whole
    key tile) on the fixed max and sends the last ones back to the running
    max, each as the oracle's rule decides. The last rows are dominated by a
    few keys: the bound for such rows applies."""
    B, Hq, Hkv, N = 2, 4, 2, 700
    q, k, v = prefill_inputs(B, Hq, Hkv, N, N, 128, torch.bfloat16, seed=77)
    k[:, -64:] = (k[:, -64:].float() * 8).to(torch.bfloat16)
    ws = _workspace(B, Hq, Hkv, N, N, 128, mode)
    o, lse = _run(q, k, v, causal=True, softmax=mode, workspace=ws)
    O, L = _ref(q, k, v, 1 / math.sqrt(128), causal=True)
    check(o, O, lse, L, where=f"{mode} causal large late keys", peaked=True)
    f = fixed_max_decisions(ws, B, Hq, Hkv, N, N).cpu().numpy()
    assert (f[:, :, oracle.MIN_KEYS - 1:N - 64] == 1).all()
    assert (f[:, :, N - 64:] == 0).mean() > 0.5
    check_decisions(f, q, k, mode, causal=True)


# ------------------------------------------------------------ random problems
def _random_fwd_case(seed):
    """A seeded random prefill problem: batch 1-2, KV heads 1-2, group 1-4,
    Nq and Nk in 1..600, d 64 or 128, bf16 (fp32 on a quarter of the cases),
    causal or not, any softmax mode, and a block mask (block sizes 16-80
    dividing the lengths, about 60 % live) on about a third of the cases."""
    rng = np.random.default_rng(2000 + seed)
    B, Hkv, G = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
    causal = bool(rng.integers(0, 2))
    mode = str(rng.choice(["online", "fixed_max", "fixed_max_centered"]))
    bm = blk = None
    if rng.random() < 0.35:
        bq, bk = (int(x) for x in rng.choice([16, 32, 48, 64, 80], size=2))
        Nq, Nk = bq * int(rng.integers(1, 8)), bk * int(rng.integers(1, 8))
        bm = (rng.random((Nq // bq, Nk // bk)) < 0.6).astype(np.uint8)
        blk = (bq, bk)
    else:
        Nq, Nk = int(rng.integers(1, 601)), int(rng.integers(1, 601))
    return B, Hkv, G, Nq, Nk, d, dtype, causal, mode, bm, blk


@pytest.mark.parametrize("seed", range(32))
def test_fwd_random_problems(seed):
    B, Hkv, G, Nq, Nk, d, dtype, causal, mode, bm, blk = _random_fwd_case(seed)
    q, k, v = prefill_inputs(B, Hkv * G, Hkv, Nq, Nk, d, dtype, seed=seed)
    o, lse = _run(q, k, v, causal=causal, block_mask=bm, block=blk, softmax=mode)
    kw = {} if bm is None else dict(block_mask=bm, block_q=blk[0], block_k=blk[1])
    O, L = _ref(q, k, v, 1 / math.sqrt(d), causal=causal, **kw)
    check(o, O, lse, L, dtype="f32" if dtype == torch.float32 else "bf16",
          where=f"seed {seed}: B={B} Hkv={Hkv} G={G} Nq={Nq} Nk={Nk} d={d} {dtype} "
                f"causal={causal} {mode} block={blk}")
