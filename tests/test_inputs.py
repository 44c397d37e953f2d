"""Seeded synthetic inputs: determinism, shapes, rounding and structure."""

import numpy as np
import torch

from exact_io_aware_attn_amd.inputs import (WORKLOADS, decode_inputs, frame_block_mask,
                                             prefill_inputs)


def test_prefill_inputs_deterministic_and_shaped():
    a = prefill_inputs(2, 4, 2, 33, 47, 64, torch.bfloat16, seed=7)
    b = prefill_inputs(2, 4, 2, 33, 47, 64, torch.bfloat16, seed=7)
    c = prefill_inputs(2, 4, 2, 33, 47, 64, torch.bfloat16, seed=8)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    assert a[0].shape == (2, 33, 4, 64) and a[1].shape == (2, 47, 2, 64) and a[2].shape == (2, 47, 2, 64)
    assert a[0].dtype == torch.bfloat16


def test_bf16_inputs_are_rounded_fp32_draws():
    g = torch.Generator().manual_seed(5)
    q32 = torch.randn(1, 16, 2, 64, generator=g)
    q, _, _ = prefill_inputs(1, 2, 2, 16, 16, 64, torch.bfloat16, seed=5)
    assert torch.equal(q, q32.to(torch.bfloat16))


def test_decode_inputs_lengths_and_order():
    seqlens, q, kc, vc = decode_inputs(8, 4, 2, 256, 64, torch.bfloat16, seed=3, len_lo=10, len_hi=256)
    assert seqlens.dtype == torch.int32 and seqlens.shape == (8,)
    assert int(seqlens.min()) >= 10 and int(seqlens.max()) <= 256
    g = torch.Generator().manual_seed(3)
    assert torch.equal(seqlens, torch.randint(10, 257, (8,), generator=g).to(torch.int32))
    assert q.shape == (8, 4, 64) and kc.shape == (8, 256, 2, 64) and vc.shape == kc.shape


def test_frame_mask_structure():
    bm = frame_block_mask(16, 880, 80)
    per = 11
    f = np.arange(176) // per
    for qb in (0, 5, 11, 100, 175):
        live_frames = sorted(set(f[np.nonzero(bm[qb])[0]]))
        fq = f[qb]
        expect = sorted({0, fq} | {g for g in (fq - 1, fq + 1) if 0 <= g < 16})
        assert live_frames == expect
    # 60 of the 256 frame pairs are attended
    frame_pairs = bm.reshape(16, per, 16, per)[:, 0, :, 0]
    assert int(frame_pairs.sum()) == 60


def test_named_workloads():
    assert set(WORKLOADS) == {"tiny-f32", "gpt2-causal", "llama3-8b-gqa-causal-8k",
                              "gqa-decode-b64", "video-frames-16x880",
                              "gpt2-medium-causal", "llama3-8b-gqa-causal-8k-bwd",
                              "gpt2-medium-causal-bwd", "video-frames-16x880-bwd",
                              "gqa-decode-b64-4tok", "gqa-decode-b64-paged"}
    assert WORKLOADS["llama3-8b-gqa-causal-8k"].scale == 1 / 128 ** 0.5


def test_backward_inputs_extend_the_prefill_draws():
    # same seed: Q, K, V are the prefill draws, dO comes after them
    from exact_io_aware_attn_amd.inputs import backward_inputs, prefill_inputs
    q, k, v = prefill_inputs(2, 4, 2, 33, 40, 64, torch.bfloat16, seed=9)
    q2, k2, v2, do = backward_inputs(2, 4, 2, 33, 40, 64, torch.bfloat16, seed=9)
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
    assert do.shape == q.shape and not torch.equal(do, q)


def test_paged_cache_holds_the_same_rows():
    from exact_io_aware_attn_amd.inputs import decode_inputs, paged_cache
    _, _, kc, vc = decode_inputs(3, 4, 2, 128, 64, torch.bfloat16, seed=5)
    kp, vp, table = paged_cache(kc, vc, 32, seed=2)
    assert table.shape == (3, 4) and sorted(table.reshape(-1).tolist()) == list(range(12))
    assert torch.equal(kp[table.long()].reshape(kc.shape), kc)
    assert torch.equal(vp[table.long()].reshape(vc.shape), vc)
