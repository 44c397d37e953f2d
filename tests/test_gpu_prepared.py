"""Prepared calls (arguments marshalled once) against the plain entry points.

A prepared call enqueues the same kernels with the same arguments, so its
outputs must be bitwise equal to attn_fwd / attn_decode on the same tensors,
on the first call and on later calls after the inputs were rewritten in
place."""

import pytest
import torch

from exact_io_aware_attn_amd import attn_decode, attn_fwd, prepare_decode, prepare_fwd
from exact_io_aware_attn_amd.inputs import decode_inputs, frame_block_mask, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _same(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("kw", [
    dict(causal=True),
    dict(causal=False, softmax="fixed_max"),
    dict(block=(48, 48), softmax="fixed_max_centered"),
])
def test_prepared_fwd_matches_plain(kw):
    q, k, v = (t.to(DEV) for t in prefill_inputs(2, 8, 2, 288, 336, 128, torch.bfloat16, seed=31))
    if "block" in kw:
        kw = dict(kw, block_mask=frame_block_mask(6, 48, 48))
        q, k = q[:, :288], k[:, :288]
        v = v[:, :288]
    call, o, lse = prepare_fwd(q, k, v, **kw)
    for step in range(3):
        call()
        ref_o, ref_lse = attn_fwd(q, k, v, **kw)
        torch.cuda.synchronize()
        assert _same(o, ref_o) and _same(lse, ref_lse), f"step {step}"
        q.mul_(-1.0)   # in-place change: the next call must see it


def test_prepared_decode_matches_plain():
    seqlens, q, kc, vc = decode_inputs(6, 32, 8, 900, 128, torch.bfloat16, seed=32,
                                       len_lo=0, len_hi=900)
    q, kc, vc, seqlens = q.to(DEV), kc.to(DEV), vc.to(DEV), seqlens.to(DEV)
    call, o, lse = prepare_decode(q, kc, vc, seqlens)
    for step in range(3):
        call()
        ref_o, ref_lse = attn_decode(q, kc, vc, seqlens)
        torch.cuda.synchronize()
        assert _same(o, ref_o) and _same(lse, ref_lse), f"step {step}"
        seqlens.sub_(1).clamp_(min=0)
