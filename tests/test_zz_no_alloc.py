"""attn_decode_noalloc: the decode entry point that allocates nothing.

For callers that cannot allocate device memory (graph capture, tight serving
loops). Its split-K partials live in the library's static per-device scratch;
its output must equal attn_decode's (same kernels, same split count) on two
calls in a row, the second smaller than the first, and meet the band against
the fp64 oracle. A request whose partials exceed the scratch is refused.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_attn_amd import attn_decode, attn_decode_noalloc
from exact_io_aware_attn_amd.binding import MiattnError
from exact_io_aware_attn_amd.inputs import WORKLOADS, decode_inputs

from parity import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(B, Hq, Hkv, max_len, d, seed, len_lo, len_hi, kv_splits=0):
    seqlens, q, kc, vc = decode_inputs(B, Hq, Hkv, max_len, d, torch.bfloat16, seed,
                                       len_lo, len_hi, device=DEV)
    o_ref, l_ref = attn_decode(q, kc, vc, seqlens, kv_splits=kv_splits)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    attn_decode_noalloc(q, kc, vc, seqlens, o, lse, kv_splits=kv_splits)
    torch.cuda.synchronize()
    return (seqlens, q, kc, vc), (o, lse), (o_ref, l_ref)


def _oracle_check(ins, o, lse, where):
    seqlens, q, kc, vc = ins
    sl = seqlens.cpu().numpy()
    d = q.shape[-1]
    for b in range(q.shape[0]):
        n = int(sl[b])
        O, L = oracle.decode(to64(q[b:b + 1]), to64(kc[b:b + 1, :n]), to64(vc[b:b + 1, :n]),
                             np.array([n]), 1 / math.sqrt(d))
        check(o[b:b + 1], O, lse[b:b + 1], L, where=f"{where} b={b}")


def test_noalloc_two_calls_second_smaller():
    """The decode workload's shape (64 sequences, lengths U[1024, 32768]), then
    a smaller one (5 sequences, short lengths, another head count): each
    bitwise equal to attn_decode and within the band against the oracle. The
    second call reuses the scratch the first one left full of its partials."""
    w = WORKLOADS["gqa-decode-b64"]
    ins, (o, lse), (o_ref, l_ref) = _pair(w.B, w.Hq, w.Hkv, w.Nk, w.d, w.seed, w.len_lo, w.len_hi)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    _oracle_check(ins, o, lse, "noalloc call 1")
    free0 = torch.cuda.mem_get_info()[0]
    ins, (o, lse), (o_ref, l_ref) = _pair(5, 8, 2, 700, 64, 31, 1, 700, kv_splits=7)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    _oracle_check(ins, o, lse, "noalloc call 2")
    # the second noalloc call (after the first has loaded the scratch) takes no
    # device memory: free memory is unchanged around one more call
    o2 = torch.empty_like(o)
    torch.cuda.synchronize()
    before = torch.cuda.mem_get_info()[0]
    attn_decode_noalloc(ins[1], ins[2], ins[3], ins[0], o2, None, kv_splits=7)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == before
    assert torch.equal(o2, o)
    assert free0 > 0


def test_noalloc_refuses_partials_beyond_the_scratch():
    """4096 ranges x (4096 + 64 slots) x 32 heads x 129 floats is far past the
    32 MiB scratch: refused with the workspace status, nothing launched."""
    seqlens, q, kc, vc = decode_inputs(64, 32, 8, 256, 128, torch.bfloat16, 3, 1, 256, device=DEV)
    o = torch.zeros_like(q)
    with pytest.raises(MiattnError) as e:
        attn_decode_noalloc(q, kc, vc, seqlens, o, None, kv_splits=4096)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert (o.float() == 0).all()
