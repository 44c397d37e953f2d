"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay equals, bit for bit, an eager call on the same inputs.
Between replays the inputs change in place, with the program's own eager work
and synchronisations in between. The library issues no memset, copy or
allocation, so a captured call is only its kernels."""


import pytest
import torch

from exact_io_aware_attn_amd import attn_bwd, attn_decode, attn_decode_workspace_bytes, attn_fwd
from exact_io_aware_attn_amd.inputs import backward_inputs, decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _same(a, b):
    """Bitwise equality, NaN included."""
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm (outside the graph)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_fwd_replays():
    q, k, v = (x.to(DEV) for x in prefill_inputs(1, 4, 2, 300, 333, 128, torch.bfloat16, seed=3))
    o = torch.empty_like(q)
    lse = torch.empty((1, 4, 300), dtype=torch.float32, device=DEV)
    g = _capture(lambda: attn_fwd(q, k, v, causal=True, out=o, lse_out=lse))
    q0 = q.clone()
    for i in range(4):
        q.copy_(q0 * (1.0 + 0.5 * i))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = attn_fwd(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert _same(o, o_e) and _same(lse, lse_e), f"replay {i}"


def test_graph_decode_replays():
    seqlens, q, kc, vc = decode_inputs(6, 8, 2, 900, 128, torch.bfloat16, seed=4, len_lo=0)
    seqlens, q, kc, vc = (x.to(DEV) for x in (seqlens, q, kc, vc))
    o = torch.empty_like(q)
    lse = torch.empty((6, 8), dtype=torch.float32, device=DEV)
    ws = torch.empty(attn_decode_workspace_bytes(6, 8, 2, 900, 128), dtype=torch.uint8, device=DEV)
    g = _capture(lambda: attn_decode(q, kc, vc, seqlens, out=o, lse_out=lse, workspace=ws))
    lens = [[900, 1, 0, 450, 33, 64], [5, 900, 899, 0, 0, 128], [0, 0, 0, 0, 0, 0],
            [17, 300, 600, 900, 2, 1]]
    for i, ls in enumerate(lens):
        seqlens.copy_(torch.tensor(ls, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = attn_decode(q, kc, vc, seqlens)
        torch.cuda.synchronize()
        assert _same(o, o_e) and _same(lse, lse_e), f"replay {i}"


@pytest.mark.parametrize("d", [64, 128])
def test_graph_bwd_replays(d):
    """Alternate replays carry a NaN in dO at row 70, which keys above 70 + 32
    cannot see: the workspace flag is cleared and raised again on each replay,
    and the fix-up kernel's recompute appears in exactly those replays."""
    q, k, v, do = (x.to(DEV) for x in backward_inputs(1, 4, 2, 200, 232, d, torch.bfloat16, seed=5))
    o, lse = attn_fwd(q, k, v, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    g = _capture(lambda: attn_bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv,
                                  workspace=ws))
    do0 = do.clone()
    for i in range(6):
        do.copy_(do0)
        if i % 2:
            do[0, 70, 1, 3] = float("nan")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e = attn_bwd(q, k, v, o, lse, do, causal=True)
        torch.cuda.synchronize()
        for got, ref, n in zip((dq, dk, dv), e, "QKV"):
            assert _same(got, ref), f"replay {i} d{n}"
        # the NaN reaches dV only of the keys row 70 sees (0 .. 102)
        bad_keys = torch.isnan(dv.float()).any(dim=-1).any(dim=-1)[0]
        assert bool(bad_keys[103:].any()) is False, f"replay {i}"
        assert bool(bad_keys[:103].any()) is bool(i % 2), f"replay {i}"


def test_graph_decode_noalloc_and_paged_replays():
    """The allocation-free decode (static per-device scratch) and the paged
    multi-token decode, each captured and replayed with changed lengths."""
    import numpy as np
    from exact_io_aware_attn_amd import (attn_decode_multi_workspace_bytes, attn_decode_noalloc,
                                         attn_decode_paged)
    from exact_io_aware_attn_amd.inputs import decode_multi_inputs

    seqlens, q, kc, vc = decode_inputs(5, 16, 4, 1024, 64, torch.bfloat16, seed=6, len_lo=0)
    seqlens, q, kc, vc = (x.to(DEV) for x in (seqlens, q, kc, vc))
    o, lse = torch.empty_like(q), torch.empty((5, 16), dtype=torch.float32, device=DEV)
    g1 = _capture(lambda: attn_decode_noalloc(q, kc, vc, seqlens, o, lse))

    B, nt, Hq, Hkv, max_len, d, page = 4, 3, 8, 2, 512, 128, 64
    sl2, q2, kc2, vc2 = decode_multi_inputs(B, nt, Hq, Hkv, max_len, d, seed=7, len_lo=0)
    mp = max_len // page
    perm = np.random.default_rng(7).permutation(B * mp + 2)[:B * mp].astype(np.int32)
    table = torch.from_numpy(perm).view(B, mp)
    kp = torch.zeros(B * mp + 2, page, Hkv, d, dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    kp[table.reshape(-1).long()] = kc2.reshape(B * mp, page, Hkv, d)
    vp[table.reshape(-1).long()] = vc2.reshape(B * mp, page, Hkv, d)
    sl2, q2, kp, vp, table = (x.to(DEV) for x in (sl2, q2, kp, vp, table))
    o2 = torch.empty_like(q2)
    lse2 = torch.empty((B, nt, Hq), dtype=torch.float32, device=DEV)
    ws = torch.empty(attn_decode_multi_workspace_bytes(B, nt, Hq, Hkv, max_len, d), dtype=torch.uint8,
                     device=DEV)
    g2 = _capture(lambda: attn_decode_paged(q2, kp, vp, table, sl2, out=o2, lse_out=lse2,
                                            workspace=ws))
    lens1 = [[1024, 0, 1, 700, 63], [3, 1024, 512, 0, 1000], [0, 0, 0, 0, 0]]
    lens2 = [[512, 0, 2, 300], [1, 512, 511, 64], [5, 6, 7, 8]]
    for i in range(3):
        seqlens.copy_(torch.tensor(lens1[i], dtype=torch.int32))
        sl2.copy_(torch.tensor(lens2[i], dtype=torch.int32))
        torch.cuda.synchronize()
        g1.replay()
        g2.replay()
        torch.cuda.synchronize()
        e1 = attn_decode(q, kc, vc, seqlens)
        e2 = attn_decode_paged(q2, kp, vp, table, sl2)
        torch.cuda.synchronize()
        assert _same(o, e1[0]) and _same(lse, e1[1]), f"noalloc replay {i}"
        assert _same(o2, e2[0]) and _same(lse2, e2[1]), f"paged replay {i}"
