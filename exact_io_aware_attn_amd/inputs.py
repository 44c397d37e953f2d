"""Seeded synthetic inputs and the named workloads.

This module only draws random numbers and builds the input structure (shapes,
key lengths, the frame block mask). It holds none of the attention arithmetic,
so the oracle and the HIP path can both be fed from it.

Recipe: a ``torch.Generator`` on the target device, seeded with the workload's
seed; draw order is key lengths (decode only), then Q, K, V (then the upstream
gradient dO for the backward pass) as float32 standard normals; bf16 workloads
round those draws to bf16 (round to nearest even).
"""

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill", "decode" or "backward"
    B: int
    Hq: int
    Hkv: int
    Nq: int                   # prefill: query rows; decode: 1
    Nk: int                   # prefill: keys; decode: max_len of the cache
    d: int
    dtype: str                # "bf16" or "f32"
    causal: bool = False
    seed: int = 0
    frames: int = 0           # frame block mask: number of frames ...
    frame_len: int = 0        # ... tokens per frame
    block: int = 0            # ... block size (block_q == block_k)
    len_lo: int = 0           # decode key lengths, uniform in [len_lo, len_hi]
    len_hi: int = 0
    softmax: tuple = field(default=("online",))
    n_new: int = 1            # decode: new tokens per sequence (causal among themselves)
    page_size: int = 0        # decode: > 0 for a paged cache (pages placed at random)

    @property
    def scale(self):
        return 1.0 / float(self.d) ** 0.5

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


WORKLOADS = {
    "tiny-f32": Workload("tiny-f32", "prefill", B=1, Hq=1, Hkv=1, Nq=128, Nk=128,
                         d=64, dtype="f32", seed=1),
    "gpt2-causal": Workload("gpt2-causal", "prefill", B=8, Hq=12, Hkv=12, Nq=1024,
                            Nk=1024, d=64, dtype="bf16", causal=True, seed=2),
    "llama3-8b-gqa-causal-8k": Workload("llama3-8b-gqa-causal-8k", "prefill", B=1,
                                        Hq=32, Hkv=8, Nq=8192, Nk=8192, d=128,
                                        dtype="bf16", causal=True, seed=3),
    "gqa-decode-b64": Workload("gqa-decode-b64", "decode", B=64, Hq=32, Hkv=8, Nq=1,
                               Nk=32768, d=128, dtype="bf16", seed=4,
                               len_lo=1024, len_hi=32768),
    # GPT-2 medium attention (batch 64, 16 heads, length 1024, head dim 64): the shape
    # "플래시어텐션: 메모리를 아끼는 정확한 어텐션" reports its measurement on (§4 재계산)
    "gpt2-medium-causal": Workload("gpt2-medium-causal", "prefill", B=64, Hq=16, Hkv=16,
                                   Nq=1024, Nk=1024, d=64, dtype="bf16", causal=True,
                                   seed=6),
    # backward pass (dQ, dK, dV from Q, K, V, O, LSE and dO) on the prefill shapes
    "llama3-8b-gqa-causal-8k-bwd": Workload("llama3-8b-gqa-causal-8k-bwd", "backward", B=1,
                                            Hq=32, Hkv=8, Nq=8192, Nk=8192, d=128,
                                            dtype="bf16", causal=True, seed=7),
    # decode of 4 new tokens per sequence at once (4 tokens x 4 query heads fill the
    # 16 query rows a KV head's products carry)
    "gqa-decode-b64-4tok": Workload("gqa-decode-b64-4tok", "decode", B=64, Hq=32, Hkv=8, Nq=4,
                                    Nk=32768, d=128, dtype="bf16", seed=10, len_lo=1024,
                                    len_hi=32768, n_new=4),
    # the decode workload's cache held in pages of 64 rows placed in random order
    "gqa-decode-b64-paged": Workload("gqa-decode-b64-paged", "decode", B=64, Hq=32, Hkv=8,
                                     Nq=1, Nk=32768, d=128, dtype="bf16", seed=4,
                                     len_lo=1024, len_hi=32768, page_size=64),
    "gpt2-medium-causal-bwd": Workload("gpt2-medium-causal-bwd", "backward", B=64, Hq=16,
                                       Hkv=16, Nq=1024, Nk=1024, d=64, dtype="bf16",
                                       causal=True, seed=8),
    "video-frames-16x880-bwd": Workload("video-frames-16x880-bwd", "backward", B=1, Hq=24,
                                        Hkv=24, Nq=14080, Nk=14080, d=128, dtype="bf16",
                                        seed=9, frames=16, frame_len=880, block=80),
    "video-frames-16x880": Workload("video-frames-16x880", "prefill", B=1, Hq=24,
                                    Hkv=24, Nq=14080, Nk=14080, d=128, dtype="bf16",
                                    seed=5, frames=16, frame_len=880, block=80,
                                    softmax=("online", "fixed_max")),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, dtype, slab=1 << 26):
    """float32 N(0,1) draws, cast to dtype, produced in slabs along dim 0."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    per = max(1, slab // max(1, flat.shape[1]))
    for i in range(0, shape[0], per):
        j = min(shape[0], i + per)
        flat[i:j] = torch.randn((j - i, flat.shape[1]), generator=g, device=device,
                                dtype=torch.float32).to(dtype)
    return out


def prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype=torch.bfloat16, seed=0, device="cpu"):
    """Q [B,Nq,Hq,d], K and V [B,Nk,Hkv,d] (packed BSHD), drawn Q, K, V in order."""
    g = _gen(device, seed)
    q = _randn((B, Nq, Hq, d), g, device, dtype)
    k = _randn((B, Nk, Hkv, d), g, device, dtype)
    v = _randn((B, Nk, Hkv, d), g, device, dtype)
    return q, k, v


def backward_inputs(B, Hq, Hkv, Nq, Nk, d, dtype=torch.bfloat16, seed=0, device="cpu"):
    """Q, K, V as prefill_inputs draws them, then dO [B,Nq,Hq,d]."""
    g = _gen(device, seed)
    q = _randn((B, Nq, Hq, d), g, device, dtype)
    k = _randn((B, Nk, Hkv, d), g, device, dtype)
    v = _randn((B, Nk, Hkv, d), g, device, dtype)
    do = _randn((B, Nq, Hq, d), g, device, dtype)
    return q, k, v, do


def decode_inputs(B, Hq, Hkv, max_len, d, dtype=torch.bfloat16, seed=0, len_lo=1,
                  len_hi=None, device="cpu"):
    """seqlens int32 [B] uniform in [len_lo, len_hi], then q [B,Hq,d] and the
    caches [B,max_len,Hkv,d]; every cache row is drawn, also past seqlens."""
    len_hi = max_len if len_hi is None else len_hi
    g = _gen(device, seed)
    seqlens = torch.randint(len_lo, len_hi + 1, (B,), generator=g, device=device,
                            dtype=torch.int64).to(torch.int32)
    q = _randn((B, Hq, d), g, device, dtype)
    kc = _randn((B, max_len, Hkv, d), g, device, dtype)
    vc = _randn((B, max_len, Hkv, d), g, device, dtype)
    return seqlens, q, kc, vc


def paged_cache(k_cache, v_cache, page_size, seed=0):
    """The same cache rows scattered over pages [num_pages, page_size, Hkv, d] in a
    seeded random order, with the block table int32 [B, max_len / page_size]."""
    B, max_len, Hkv, d = k_cache.shape
    mp = max_len // page_size
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    table = torch.randperm(B * mp, generator=g).to(torch.int32).view(B, mp).to(k_cache.device)
    idx = table.reshape(-1).long()
    kp = torch.empty(B * mp, page_size, Hkv, d, dtype=k_cache.dtype, device=k_cache.device)
    vp = torch.empty_like(kp)
    kp[idx] = k_cache.reshape(B * mp, page_size, Hkv, d)
    vp[idx] = v_cache.reshape(B * mp, page_size, Hkv, d)
    return kp, vp, table


def decode_multi_inputs(B, n_new, Hq, Hkv, max_len, d, dtype=torch.bfloat16, seed=0, len_lo=1,
                        len_hi=None, device="cpu"):
    """As decode_inputs, with q [B, n_new, Hq, d] (the new tokens, whose own keys
    are the last n_new cached rows of each sequence)."""
    len_hi = max_len if len_hi is None else len_hi
    g = _gen(device, seed)
    seqlens = torch.randint(len_lo, len_hi + 1, (B,), generator=g, device=device,
                            dtype=torch.int64).to(torch.int32)
    q = _randn((B, n_new, Hq, d), g, device, dtype)
    kc = _randn((B, max_len, Hkv, d), g, device, dtype)
    vc = _randn((B, max_len, Hkv, d), g, device, dtype)
    return seqlens, q, kc, vc


def frame_block_mask(frames, frame_len, block, window=1, ref_frame=0):
    """uint8 [n, n] block mask, n = frames * frame_len / block.

    Query frame f sees key frames f-window .. f+window (clipped to the video)
    and the reference frame. The block size must divide the frame length, so
    every block lies inside one frame and is wholly live or wholly dead.
    """
    if frame_len % block:
        raise ValueError("block must divide the frame length")
    per = frame_len // block
    n = frames * per
    fq = np.arange(n) // per
    fk = np.arange(n) // per
    near = np.abs(fq[:, None] - fk[None, :]) <= window
    ref = fk[None, :] == ref_frame
    return (near | ref).astype(np.uint8)


def workload_inputs(w: Workload, device="cpu"):
    """Inputs of a named workload: prefill -> dict(q, k, v, block_mask?),
    decode -> dict(seqlens, q, k_cache, v_cache), backward -> dict(q, k, v, dout)."""
    if w.kind == "backward":
        q, k, v, do = backward_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.torch_dtype,
                                      w.seed, device)
        out = dict(q=q, k=k, v=v, dout=do)
        if w.frames:
            out["block_mask"] = frame_block_mask(w.frames, w.frame_len, w.block)
        return out
    if w.kind == "prefill":
        q, k, v = prefill_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.torch_dtype,
                                 w.seed, device)
        out = dict(q=q, k=k, v=v)
        if w.frames:
            out["block_mask"] = frame_block_mask(w.frames, w.frame_len, w.block)
        return out
    if w.n_new > 1:
        seqlens, q, kc, vc = decode_multi_inputs(w.B, w.n_new, w.Hq, w.Hkv, w.Nk, w.d,
                                                 w.torch_dtype, w.seed, w.len_lo, w.len_hi, device)
    else:
        seqlens, q, kc, vc = decode_inputs(w.B, w.Hq, w.Hkv, w.Nk, w.d, w.torch_dtype,
                                           w.seed, w.len_lo, w.len_hi, device)
    if w.page_size:
        kp, vp, table = paged_cache(kc, vc, w.page_size, w.seed)
        del kc, vc
        return dict(seqlens=seqlens, q=q, k_pages=kp, v_pages=vp, block_table=table)
    return dict(seqlens=seqlens, q=q, k_cache=kc, v_cache=vc)
