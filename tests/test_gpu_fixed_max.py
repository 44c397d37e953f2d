"""The fixed-max softmax's per-row choice on the GPU against the oracle's rule.

Both modes give the exact result whichever rows take the fixed max, so the
output checks alone cannot tell a kernel that always falls back from one
that never does. The kernel records each row's choice in its workspace
(layout in include/miattn.h); these tests compare it with
oracle.fixed_max_bounds ("TPU attention 최적화 실전 가이드", 4단계: the bound, its
gap to the row max, and the fallback of loose rows) on inputs that are all
eligible (N(0,1)), all ineligible (Q x10) and mixed (Q x10 on some heads; keys
8x longer in one part of the sequence, which only some rows see), in every
kernel configuration: 4- and 8-wave workgroups, keys split between two
waves, block masks with and without row segments, and the fp32 kernel.
Outputs are checked against the oracle too.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_attn_amd import attn_fwd, attn_fwd_workspace_bytes, fixed_max_decisions
from exact_io_aware_attn_amd.binding import SOFTMAX_MODES
from exact_io_aware_attn_amd.inputs import frame_block_mask, prefill_inputs

from parity import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _decide(q, k, v, mode, causal=False, block_mask=None, block=None, dtype="bf16",
            peaked=False):
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    kind = (1 if causal else 0) | (2 if block_mask is not None else 0)
    bq, bk = block if block is not None else (0, 0)
    n = attn_fwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, kind, bq, bk, SOFTMAX_MODES[mode])
    ws = torch.full((n,), 7, dtype=torch.uint8, device=DEV)  # not a valid flag value
    o, lse = attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, block_mask=block_mask,
                      block=block, softmax=mode, workspace=ws)
    torch.cuda.synchronize()
    flags = fixed_max_decisions(ws, B, Hq, Hkv, Nq, Nk).cpu().numpy()
    mask = dict(causal=causal)
    if block_mask is not None:
        mask.update(block_mask=block_mask, block_q=bq, block_k=bk)
    scale = 1 / math.sqrt(d)
    M, gap, el = oracle.fixed_max_bounds(to64(q), to64(k), scale,
                                         centered=mode == "fixed_max_centered", **mask)
    assert set(np.unique(flags)) <= {0, 1}, "every row records a choice"
    clear = ~(np.abs(np.nan_to_num(gap, nan=np.inf) - oracle.TAU) <= 0.05)
    assert clear.mean() > 0.99
    bad = np.argwhere(((flags == 1) != el) & clear)
    assert bad.size == 0, f"{len(bad)} of {flags.size} decisions differ, first {bad[:5].tolist()}"
    O, L = oracle.attention(to64(q), to64(k), to64(v), scale, **mask)
    check(o, O, lse, L, dtype=dtype, where=mode, peaked=peaked)
    return flags, el


MODES = ["fixed_max", "fixed_max_centered"]
# (B, Hq, Hkv, N, d): 4-wave, 8-wave (>= 1024 workgroups of 256 rows), key split (d = 64, few rows)
SHAPES = [(1, 4, 2, 700, 128), (32, 16, 4, 300, 128), (1, 8, 8, 1500, 64), (2, 4, 4, 520, 64)]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B,Hq,Hkv,N,d", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_decisions_all_eligible(mode, B, Hq, Hkv, N, d, causal):
    """N(0,1): every row that sees at least one key tile (64 keys) takes the
    fixed max; under the causal rule rows 0..62 see fewer and keep the
    running max."""
    q, k, v = prefill_inputs(B, Hq, Hkv, N, N, d, torch.bfloat16, seed=N + d + B)
    flags, el = _decide(q, k, v, mode, causal=causal)
    first = oracle.MIN_KEYS - 1 if causal else 0
    assert (flags[..., first:] == 1).all() and (flags[..., :first] == 0).all()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B,Hq,Hkv,N,d", SHAPES)
def test_decisions_mixed_heads(mode, B, Hq, Hkv, N, d):
    """Q x10 on odd query heads: those rows fall back, the others (from the
    first row that sees a whole key tile) do not."""
    q, k, v = prefill_inputs(B, Hq, Hkv, N, N, d, torch.bfloat16, seed=N + 2 * d + B)
    q[:, :, 1::2] = (q[:, :, 1::2].float() * 10).to(torch.bfloat16)
    flags, el = _decide(q, k, v, mode, causal=True, peaked=True)
    m = oracle.MIN_KEYS - 1
    assert (flags[:, 0::2, m:] == 1).all() and (flags[:, 1::2] == 0).all()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B,Hq,Hkv,N,d", SHAPES)
def test_decisions_mixed_rows_causal(mode, B, Hq, Hkv, N, d):
    """Keys 8x longer from key N/2 + 40 on: under the causal rule only the rows
    from there on see them, so decisions change within a head (and within
    32-row groups); the oracle's rule decides each row."""
    q, k, v = prefill_inputs(B, Hq, Hkv, N, N, d, torch.bfloat16, seed=N + 3 * d + B)
    j0 = N // 2 + 40
    k[:, j0:] = (k[:, j0:].float() * 8).to(torch.bfloat16)
    flags, el = _decide(q, k, v, mode, causal=True, peaked=True)
    assert (flags[..., oracle.MIN_KEYS - 1:j0] == 1).all()
    assert (flags[..., j0:] == 0).mean() > 0.5


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B,frames,flen,blk,heads", [
    (1, 5, 128, 64, 2),     # block rows a multiple of 32
    (1, 6, 160, 80, 3),     # block rows of 80: row segments
    (9, 8, 160, 80, 24),    # 8-wave workgroups with row segments
])
def test_decisions_frame_mask(mode, B, frames, flen, blk, heads):
    """Frame mask with frame 3's keys 8x longer (and shifted): the frames that
    attend frame 3 (2, 3, 4) fall back, the rest keep the fixed max."""
    n = frames * flen
    bm = frame_block_mask(frames, flen, blk)
    q, k, v = prefill_inputs(B, heads, heads, n, n, 128, torch.bfloat16, seed=flen + heads)
    fr = slice(3 * flen, 4 * flen)
    k[:, fr] = (k[:, fr].float() * 8 + 0.5).to(torch.bfloat16)
    flags, el = _decide(q, k, v, mode, block_mask=bm, block=(blk, blk), peaked=True)
    for f in range(frames):
        rows = flags[..., f * flen:(f + 1) * flen]
        if f in (2, 3, 4):
            assert (rows == 0).mean() > 0.5, f
        else:
            assert (rows == 1).all(), f


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("causal", [False, True])
def test_decisions_random_block_mask(mode, causal):
    """Random block mask, with and without causal, blocks 48 x 32 (row
    segments, blocks cut by the causal rule), the keys of key blocks 5 and 6
    8x longer: rows whose block row sees either fall back."""
    rng = np.random.default_rng(5)
    bq, bk = 48, 32
    Nq, Nk = 20 * bq, 24 * bk
    bm = (rng.random((Nq // bq, Nk // bk)) < 0.5).astype(np.uint8)
    bm[:, 0] = 1
    q, k, v = prefill_inputs(1, 4, 2, Nq, Nk, 128, torch.bfloat16, seed=31)
    k[:, 5 * bk:7 * bk] = (k[:, 5 * bk:7 * bk].float() * 8).to(torch.bfloat16)
    flags, el = _decide(q, k, v, mode, causal=causal, block_mask=bm, block=(bq, bk), peaked=True)
    assert 0.05 < (flags == 1).mean() < 0.95


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("causal", [False, True])
def test_decisions_f32(mode, causal):
    """The fp32 kernel: half the heads x4 (ineligible), late keys 3x longer."""
    q, k, v = prefill_inputs(1, 4, 2, 300, 330, 64, torch.float32, seed=41)
    q[:, :, 2:] *= 4
    k[:, 250:] *= 3
    flags, el = _decide(q, k, v, mode, causal=causal, dtype="f32")
    assert (flags == 0).any() and (flags == 1).any()
