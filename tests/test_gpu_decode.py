"""attn_decode on the GPU against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_attn_amd import attn_decode, attn_decode_multi, attn_decode_paged
from exact_io_aware_attn_amd.inputs import WORKLOADS, decode_inputs, decode_multi_inputs

from parity import check, check_nonfinite, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(seqlens, q, kc, vc, **kw):
    o, lse = attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), seqlens.to(DEV), **kw)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (16, 1)])
@pytest.mark.parametrize("kv_splits", [0, 1, 3, 40])
def test_decode_small(d, Hq, Hkv, kv_splits):
    seqlens, q, kc, vc = decode_inputs(5, Hq, Hkv, 700, d, torch.bfloat16, seed=d + Hq, len_lo=1, len_hi=700)
    seqlens[0] = 700
    seqlens[1] = 1
    seqlens[2] = 64
    o, lse = _run(seqlens, q, kc, vc, kv_splits=kv_splits)
    O, L = oracle.decode(to64(q), to64(kc), to64(vc), seqlens.numpy(), 1 / math.sqrt(d))
    check(o, O, lse, L, where=f"decode d={d} H={Hq}/{Hkv} splits={kv_splits}")


@pytest.mark.parametrize("kv_splits", [0, 7, 2000])
def test_decode_ragged_lengths_and_split_counts(kv_splits):
    """Lengths around slice and range edges, zeros in between, more ranges
    than rows (2000 > sum of lengths caps at one row per range)."""
    lens = [0, 1, 31, 32, 33, 0, 95, 200, 0, 17]
    seqlens, q, kc, vc = decode_inputs(len(lens), 8, 2, 200, 128, torch.bfloat16, seed=9)
    seqlens = torch.tensor(lens, dtype=torch.int32)
    o, lse = _run(seqlens, q, kc, vc, kv_splits=kv_splits)
    O, L = oracle.decode(to64(q), to64(kc), to64(vc), seqlens.numpy(), 1 / math.sqrt(128))
    check(o, O, lse, L, where=f"ragged splits={kv_splits}")


def test_decode_all_lengths_zero():
    seqlens, q, kc, vc = decode_inputs(3, 4, 2, 64, 64, torch.bfloat16, seed=10)
    seqlens = torch.zeros(3, dtype=torch.int32)
    o, lse = _run(seqlens, q, kc, vc)
    assert (o.float() == 0).all() and torch.isneginf(lse).all()


def test_decode_zero_length():
    seqlens, q, kc, vc = decode_inputs(3, 8, 2, 256, 128, torch.bfloat16, seed=1, len_lo=0, len_hi=256)
    seqlens[1] = 0
    o, lse = _run(seqlens, q, kc, vc)
    O, L = oracle.decode(to64(q), to64(kc), to64(vc), seqlens.numpy(), 1 / math.sqrt(128))
    check(o, O, lse, L, where="zero length")
    assert (o[1].float() == 0).all() and torch.isneginf(lse[1]).all()


def test_decode_rows_past_length_never_read():
    """NaN in every cache row at or past seqlens[b]: output bit-identical to the
    run with zeros there."""
    seqlens, q, kc, vc = decode_inputs(4, 8, 2, 512, 128, torch.bfloat16, seed=2, len_lo=1, len_hi=500)
    kz, vz, kn, vn = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    for b, n in enumerate(seqlens.tolist()):
        kz[b, n:] = 0
        vz[b, n:] = 0
        kn[b, n:] = float("nan")
        vn[b, n:] = float("nan")
    o1, l1 = _run(seqlens, q, kz, vz)
    o2, l2 = _run(seqlens, q, kn, vn)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.isfinite(o2.float()).all()


def test_decode_repeatable_bitwise():
    seqlens, q, kc, vc = decode_inputs(4, 8, 2, 1000, 128, torch.bfloat16, seed=3, len_lo=100, len_hi=1000)
    o1, l1 = _run(seqlens, q, kc, vc)
    o2, l2 = _run(seqlens, q, kc, vc)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_equals_prefill_with_one_query():
    """Decode against cache[:len] equals attn_fwd with Nq = 1 on that prefix."""
    from exact_io_aware_attn_amd import attn_fwd
    seqlens, q, kc, vc = decode_inputs(2, 8, 2, 300, 128, torch.bfloat16, seed=4, len_lo=200, len_hi=300)
    o, _ = _run(seqlens, q, kc, vc)
    for b, n in enumerate(seqlens.tolist()):
        of, _ = attn_fwd(q[b:b + 1, None].to(DEV), kc[b:b + 1, :n].to(DEV), vc[b:b + 1, :n].to(DEV), causal=True)
        torch.cuda.synchronize()
        assert (o[b].float() - of[0, 0].float()).abs().max() <= 1e-2


def test_full_gqa_decode_b64():
    """The full decode workload on the GPU (the launch the bench times),
    checked on every one of the 64 sequences, all 32 query heads each (each
    sequence's cache slice is copied to the host and widened on its own)."""
    w = WORKLOADS["gqa-decode-b64"]
    seqlens, q, kc, vc = decode_inputs(w.B, w.Hq, w.Hkv, w.Nk, w.d, torch.bfloat16, w.seed,
                                       w.len_lo, w.len_hi, device=DEV)
    o, lse = attn_decode(q, kc, vc, seqlens)
    torch.cuda.synchronize()
    sl = seqlens.cpu().numpy()
    for b in range(w.B):
        n = int(sl[b])
        O, L = oracle.decode(to64(q[b:b + 1]), to64(kc[b:b + 1, :n]), to64(vc[b:b + 1, :n]),
                             np.array([n]), w.scale)
        check(o[b:b + 1], O, lse[b:b + 1], L, where=f"full decode b={b} len={n}")


@pytest.mark.parametrize("paged", [False, True])
def test_lengths_outside_the_cache_are_clamped(paged):
    """Lengths live on the device and are not checked on the host: a length
    above the cache size acts as the cache size and a negative one as 0, in
    both kernels (so no row outside a sequence's cache is read), bitwise equal
    to the call with the clamped lengths, and against the oracle."""
    B, Hq, Hkv, max_len, d = 5, 8, 2, 300, 128
    seqlens, q, kc, vc = decode_inputs(B, Hq, Hkv, max_len, d, torch.bfloat16, seed=23, len_lo=1)
    bad = torch.tensor([max_len + 1, 10 ** 9, -7, 150, max_len], dtype=torch.int32)
    good = bad.clamp(0, max_len)
    if not paged:
        o1, l1 = attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), bad.to(DEV))
        o2, l2 = attn_decode(q.to(DEV), kc.to(DEV), vc.to(DEV), good.to(DEV))
    else:
        page = 64  # max_len = 300 -> 5 pages of 64 per sequence (320 rows)
        npg = (max_len + page - 1) // page
        kp = torch.zeros(B * npg, page, Hkv, d, dtype=torch.bfloat16)
        vp = torch.zeros_like(kp)
        for b in range(B):
            for j in range(npg):
                r = slice(j * page, min(max_len, (j + 1) * page))
                kp[b * npg + j, : r.stop - r.start] = kc[b, r]
                vp[b * npg + j, : r.stop - r.start] = vc[b, r]
        table = torch.arange(B * npg, dtype=torch.int32).view(B, npg)
        bad_p = bad.clone()
        bad_p[0] = npg * page + 1  # past page_size * max_pages
        good = bad_p.clamp(0, npg * page)
        o1, l1 = attn_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), bad_p.to(DEV))
        o2, l2 = attn_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), good.to(DEV))
        o1, l1, o2, l2 = o1[:, 0], l1[:, 0], o2[:, 0], l2[:, 0]
        kc = torch.cat([kp.view(B, npg * page, Hkv, d)], 1)
        vc = torch.cat([vp.view(B, npg * page, Hkv, d)], 1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O, L = oracle.decode(to64(q), to64(kc), to64(vc), good.numpy(), 1 / math.sqrt(d))
    check(o1, O, l1, L, where=f"clamped lengths paged={paged}")
    assert (o1[2].float() == 0).all() and torch.isneginf(l1[2]).all()


# ------------------------------------------------------------ several new tokens
def _multi_ref(q, kc, vc, seqlens, scale):
    """Per sequence: the new tokens' rows against its first seqlens[b] cached rows,
    causal with the rows aligned at the end (the oracle's prefill rule)."""
    B, nt, Hq, d = q.shape
    O = np.zeros((B, nt, Hq, d))
    L = np.full((B, nt, Hq), -np.inf)
    for b in range(B):
        n = int(seqlens[b])
        if n == 0:
            continue
        Ob, Lb = oracle.attention(to64(q[b:b + 1]), to64(kc[b:b + 1, :n]), to64(vc[b:b + 1, :n]),
                                  scale, causal=True)
        O[b] = Ob[0]
        L[b] = Lb[0].T
    return O, L


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nt,Hq,Hkv", [(2, 8, 2), (3, 8, 2), (4, 8, 2), (16, 2, 2), (2, 16, 2)])
@pytest.mark.parametrize("kv_splits", [0, 1, 7])
def test_decode_multi_tokens(d, nt, Hq, Hkv, kv_splits):
    seqlens, q, kc, vc = decode_multi_inputs(5, nt, Hq, Hkv, 700, d, seed=nt * 10 + d, len_lo=1)
    seqlens[0] = 0                     # empty sequence
    seqlens[1] = max(1, nt - 1)        # fewer cached rows than new tokens: the first rows see none
    o, lse = attn_decode_multi(q.to(DEV), kc.to(DEV), vc.to(DEV), seqlens.to(DEV), kv_splits=kv_splits)
    torch.cuda.synchronize()
    O, L = _multi_ref(q, kc, vc, seqlens.numpy(), 1 / math.sqrt(d))
    check(o, O, lse, L, where=f"multi nt={nt} H={Hq}/{Hkv} d={d} splits={kv_splits}")


def test_decode_multi_one_token_equals_decode():
    seqlens, q, kc, vc = decode_inputs(6, 32, 8, 900, 128, seed=12, len_lo=0)
    args = (kc.to(DEV), vc.to(DEV), seqlens.to(DEV))
    o1, l1 = attn_decode(q.to(DEV), *args)
    o2, l2 = attn_decode_multi(q[:, None].contiguous().to(DEV), *args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[:, 0]) and torch.equal(l1, l2[:, 0])


def test_full_gqa_decode_b64_4tok_sampled():
    w = WORKLOADS["gqa-decode-b64-4tok"]
    from exact_io_aware_attn_amd.inputs import workload_inputs
    ins = workload_inputs(w, device=DEV)
    o, lse = attn_decode_multi(ins["q"], ins["k_cache"], ins["v_cache"], ins["seqlens"])
    torch.cuda.synchronize()
    sl = ins["seqlens"].cpu()
    for b in (0, 17, 63):
        O, L = _multi_ref(ins["q"][b:b + 1].cpu(), ins["k_cache"][b:b + 1].cpu(),
                          ins["v_cache"][b:b + 1].cpu(), sl[b:b + 1].numpy(), w.scale)
        check(o[b:b + 1], O, lse[b:b + 1], L, where=f"gqa-decode-b64-4tok b={b}")


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("d,nt,kv_splits", [(64, 2, 0), (128, 4, 0), (128, 4, 7), (64, 3, 1)])
def test_decode_multi_nonfinite_own_rows(d, nt, kv_splits, paged, bad):
    """Inf or NaN in V at a new token's own cache row: the earlier new tokens,
    which cannot see that row, get the same result as with finite values
    there; the token itself and the later ones propagate it in its columns."""
    seqlens, q, kc, vc = decode_multi_inputs(5, nt, 8, 2, 512, d, seed=nt + d + 3, len_lo=nt)
    for b in range(5):
        n = int(seqlens[b])
        vc[b, n - 1, :, 0:4] = bad          # the last new token's row
        vc[b, n - nt + 1, :, d - 8:] = bad  # the second new token's row
    if paged:
        kp, vp, table = _to_pages(kc, vc, 64, seed=d + nt)
        o, lse = attn_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV),
                                   seqlens.to(DEV), kv_splits=kv_splits)
    else:
        o, lse = attn_decode_multi(q.to(DEV), kc.to(DEV), vc.to(DEV), seqlens.to(DEV),
                                   kv_splits=kv_splits)
    torch.cuda.synchronize()
    O, L = _multi_ref(q, kc, vc, seqlens.numpy(), 1 / math.sqrt(d))
    check_nonfinite(o, O, lse, L, where=f"multi nonfinite d={d} nt={nt} paged={paged} {bad}")


# ------------------------------------------------------------------ paged cache
def _to_pages(kc, vc, page_size, seed, spare=3):
    """Scatter a contiguous cache [B, max_len, Hkv, d] into randomly placed pages
    (plus a few unused ones) and return (k_pages, v_pages, block_table)."""
    B, max_len, Hkv, d = kc.shape
    mp = max_len // page_size
    n_pages = B * mp + spare
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(n_pages)[:B * mp].astype(np.int32))
    table = perm.view(B, mp)
    kp = torch.zeros(n_pages, page_size, Hkv, d, dtype=kc.dtype)
    vp = torch.zeros_like(kp)
    kp[table.reshape(-1).long()] = kc.reshape(B * mp, page_size, Hkv, d)
    vp[table.reshape(-1).long()] = vc.reshape(B * mp, page_size, Hkv, d)
    return kp, vp, table


@pytest.mark.parametrize("page_size", [16, 64, 256])
@pytest.mark.parametrize("nt", [1, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_paged(page_size, nt, d):
    max_len = 1024
    seqlens, q, kc, vc = decode_multi_inputs(5, nt, 8, 2, max_len, d, seed=page_size + nt + d,
                                             len_lo=0)
    seqlens[1] = max_len
    kp, vp, table = _to_pages(kc, vc, page_size, seed=page_size * 7 + d)
    o, lse = attn_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), seqlens.to(DEV))
    o2, lse2 = attn_decode_multi(q.to(DEV), kc.to(DEV), vc.to(DEV), seqlens.to(DEV))
    torch.cuda.synchronize()
    # the same rows in the same order: identical to the contiguous cache, bit for bit
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    O, L = _multi_ref(q, kc, vc, seqlens.numpy(), 1 / math.sqrt(d))
    check(o, O, lse, L, where=f"paged P={page_size} nt={nt} d={d}")


def test_full_gqa_decode_b64_paged_equals_contiguous():
    # same seed, same rows: the paged workload must reproduce the contiguous one bit for bit
    from exact_io_aware_attn_amd.inputs import workload_inputs
    w = WORKLOADS["gqa-decode-b64"]
    ins = workload_inputs(w, device=DEV)
    o1, l1 = attn_decode(ins["q"], ins["k_cache"], ins["v_cache"], ins["seqlens"])
    torch.cuda.synchronize()
    del ins
    wp = WORKLOADS["gqa-decode-b64-paged"]
    ins = workload_inputs(wp, device=DEV)
    o2, l2 = attn_decode_paged(ins["q"], ins["k_pages"], ins["v_pages"], ins["block_table"],
                               ins["seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[:, 0]) and torch.equal(l1, l2[:, 0])


# ------------------------------------------------------------ random problems
@pytest.mark.parametrize("seed", range(16))
def test_decode_random_problems(seed):
    """Seeded random decode problems: batch 1-9, KV heads 1-4, group 1-8,
    d 64 or 128, 1-4 new tokens (group x tokens at most 16, the library's
    limit), lengths 0..max_len, a random split count, and every other case
    through a paged cache (pages of 16-256 rows)."""
    rng = np.random.default_rng(3000 + seed)
    B, Hkv, G = int(rng.integers(1, 10)), int(rng.integers(1, 5)), int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    nt = int(rng.integers(1, min(4, 16 // G) + 1))
    page = int(rng.choice([16, 64, 256]))
    max_len = page * int(rng.integers(1, 9))
    kv_splits = int(rng.choice([0, 0, 1, 3, 17]))
    seqlens, q, kc, vc = decode_multi_inputs(B, nt, Hkv * G, Hkv, max_len, d, seed=seed, len_lo=0)
    where = f"seed {seed}: B={B} Hkv={Hkv} G={G} d={d} nt={nt} max_len={max_len} splits={kv_splits}"
    if seed % 2:
        kp, vp, table = _to_pages(kc, vc, page, seed=seed)
        o, lse = attn_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV),
                                   seqlens.to(DEV), kv_splits=kv_splits)
        where += f" paged {page}"
    else:
        o, lse = attn_decode_multi(q.to(DEV), kc.to(DEV), vc.to(DEV), seqlens.to(DEV),
                                   kv_splits=kv_splits)
    torch.cuda.synchronize()
    O, L = _multi_ref(q, kc, vc, seqlens.numpy(), 1 / math.sqrt(d))
    check(o, O, lse, L, where=where)
