"""The C-ABI library: it loads, exports every function include/miattn.h declares,
and its host-side validation answers without touching the GPU."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

from exact_io_aware_attn_amd import binding as bd

HEADER = os.path.join(ROOT, "include", "miattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(bd.LIB_PATH),
                                reason="libmiattn.so not built (python -m exact_io_aware_attn_amd.build)")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*([A-Za-z_]\w*)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(bd._EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bd.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(7):
        assert bd.attn_status_str(code)
    assert bd.attn_status_str(0) == "ok"
    assert bd.attn_status_str(99) == "unknown status"


def test_workspace_sizes():
    NONE, CAUSAL, BLOCK = bd.MIATTN_MASK_NONE, bd.MIATTN_MASK_CAUSAL, bd.MIATTN_MASK_BLOCK
    ws = bd.attn_fwd_workspace_bytes
    assert ws(1, 24, 24, 14080, 14080, 128, NONE, 0, 0, 0) == 0
    assert ws(1, 24, 24, 14080, 14080, 128, CAUSAL, 80, 80, 0) == 0
    # fixed max: prefix maxima [B*Hkv][Nk] fp32, then per-row decisions [B][Hq][Nq]
    plain = ws(1, 24, 24, 14080, 14080, 128, NONE, 0, 0, 1)
    assert plain >= 24 * 14080 * 4 + 24 * 14080
    # centred: radii [B*Hkv][nkb] and bf16 centres [B*Hkv][nkb][d], nkb = ceil(Nk/256) = 55
    centred = ws(1, 24, 24, 14080, 14080, 128, NONE, 0, 0, 2)
    assert centred >= plain + 24 * 55 * (4 + 2 * 128)
    # with a block mask the key blocks are the mask's: 176 blocks of 80
    assert ws(1, 24, 24, 14080, 14080, 128, BLOCK, 80, 80, 2) >= plain + 24 * 176 * (4 + 256)
    # GQA: decisions per query head, statistics per KV head
    assert ws(1, 32, 8, 8192, 8192, 128, CAUSAL, 0, 0, 1) >= 8 * 8192 * 4 + 32 * 8192
    # block masks with block_q not a multiple of 32 carry a row-segment table:
    # 176 block rows of 80 -> at most 3 segments each, 8 bytes per segment
    seg = ws(1, 24, 24, 14080, 14080, 128, BLOCK, 80, 80, 0)
    assert seg >= 176 + 176 * 3 * 8
    assert ws(1, 24, 24, 14080, 14080, 128, BLOCK, 64, 64, 0) == 0
    assert ws(1, 24, 24, 14080, 14080, 128, BLOCK | CAUSAL, 80, 80, 1) >= plain + seg
    assert ws(-1, 24, 24, 14080, 14080, 128, BLOCK, 80, 80, 1) == 0
    ws = bd.attn_decode_workspace_bytes(64, 32, 8, 32768, 128, 0)
    assert ws >= (4096 + 64) * 32 * 129 * 4
    assert ws == bd.attn_decode_workspace_bytes(64, 32, 8, 100, 128, 17)


def _fwd(**kw):
    a = dict(q=16, k=16, v=16, o=16, lse=None, dtype=0, B=1, Hq=4, Hkv=2, Nq=64, Nk=64, d=64,
             scale=0.125, mask_kind=0, block_mask=None, block_q=0, block_k=0, mode=0,
             strides=None, ws=None, ws_bytes=0)
    a.update(kw)
    P = ctypes.c_void_p
    return bd.library().attn_fwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["o"]), P(a["lse"]), a["dtype"],
                                 a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                 a["mask_kind"], P(a["block_mask"]), a["block_q"], a["block_k"],
                                 a["mode"], a["strides"], P(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 3), (dict(d=96), 3), (dict(Hq=3), 2), (dict(B=-1), 2),
    (dict(scale=0.0), 6), (dict(scale=float("nan")), 6), (dict(mask_kind=4), 6),
    (dict(mode=3), 6), (dict(q=None), 1),
    (dict(mask_kind=2, block_mask=16, block_q=8, block_k=16), 2),
    (dict(mask_kind=2, block_mask=16, block_q=48, block_k=16), 2),
    (dict(mask_kind=2, block_mask=None, block_q=16, block_k=16), 1),
    (dict(mode=1), 4), (dict(q=18), 3),
    # block_q not a multiple of 32: the row-segment table needs workspace
    (dict(mask_kind=2, block_mask=16, block_q=16, block_k=16), 4),
    (dict(B=0), 0), (dict(Nq=0), 0),
    # limits: at most 4096 key blocks per mask row; one (batch, KV head) of K
    # or V under 2 GiB (32-bit row offsets)
    (dict(mask_kind=2, block_mask=16, block_q=16, block_k=16, Nk=16 * 4097), 3),
    (dict(Nk=1 << 23), 3),
])
def test_fwd_validation(kw, status):
    """Each of these returns before anything is enqueued (no GPU needed)."""
    assert _fwd(**kw) == status


def test_fwd_rejects_unaligned_strides():
    st = (bd._Strides * 4)(bd._Strides(4096, 256, 63), bd._Strides(4096, 128, 64),
                           bd._Strides(4096, 128, 64), bd._Strides(4096, 256, 64))
    assert _fwd(strides=st) == 3


def _dec(**kw):
    a = dict(q=16, k=16, v=16, seqlens=16, o=16, lse=None, dtype=0, B=2, Hq=8, Hkv=2,
             max_len=256, d=128, scale=0.1, chunk=0, ws=None, ws_bytes=0)
    a.update(kw)
    P = ctypes.c_void_p
    return bd.library().attn_decode(P(a["q"]), P(a["k"]), P(a["v"]), P(a["seqlens"]), P(a["o"]),
                                    P(a["lse"]), a["dtype"], a["B"], a["Hq"], a["Hkv"],
                                    a["max_len"], a["d"], a["scale"], a["chunk"], None,
                                    P(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=1), 3), (dict(d=80), 3), (dict(Hq=7), 2), (dict(Hq=34, Hkv=2), 3),
    (dict(scale=-1.0), 6), (dict(chunk=-1), 6), (dict(chunk=5000), 6), (dict(seqlens=None), 1),
    (dict(ws=None), 4), (dict(B=0), 0),
    # one (sequence, KV head) of the cache must span < 2 GiB (32-bit offsets)
    (dict(max_len=1 << 23), 3),
])
def test_decode_validation(kw, status):
    assert _dec(**kw) == status


def _dec_noalloc(**kw):
    a = dict(q=16, k=16, v=16, seqlens=16, o=16, lse=None, dtype=0, B=2, Hq=8, Hkv=2,
             max_len=256, d=128, scale=0.1, chunk=0)
    a.update(kw)
    P = ctypes.c_void_p
    return bd.library().attn_decode_noalloc(P(a["q"]), P(a["k"]), P(a["v"]), P(a["seqlens"]),
                                            P(a["o"]), P(a["lse"]), a["dtype"], a["B"], a["Hq"],
                                            a["Hkv"], a["max_len"], a["d"], a["scale"], a["chunk"],
                                            None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=1), 3), (dict(d=80), 3), (dict(Hq=7), 2), (dict(scale=-1.0), 6),
    (dict(chunk=-1), 6), (dict(seqlens=None), 1), (dict(B=0), 0),
    # partials past the 32 MiB static scratch: (4096 + 64) slots x 32 heads x 129 floats
    (dict(B=64, Hq=32, Hkv=8, chunk=4096), 4),
])
def test_decode_noalloc_validation(kw, status):
    """The allocation-free decode validates like attn_decode (no workspace
    argument) and refuses partials beyond its static scratch, all on the host."""
    assert _dec_noalloc(**kw) == status


def test_bwd_workspace_size():
    # two fp32 rows of Nq rounded up to 64 per (batch, query head), then one
    # 256-byte slot for the non-finite flag
    assert bd.attn_bwd_workspace_bytes(2, 4, 100) == 2 * 2 * 4 * 128 * 4 + 256
    assert bd.attn_bwd_workspace_bytes(1, 32, 8192) == 2 * 32 * 8192 * 4 + 256
    assert bd.attn_bwd_workspace_bytes(-1, 4, 100) == 0
    assert bd.attn_bwd_workspace_bytes(2, 4, 0) == 0


def _bwd(**kw):
    a = dict(q=16, k=16, v=16, o=16, dout=16, lse=16, dq=16, dk=16, dv=16, dtype=0, B=2, Hq=4,
             Hkv=2, Nq=96, Nk=80, d=128, scale=0.1, mask_kind=1, block_mask=None, block_q=0,
             block_k=0, ws=16, ws_bytes=1 << 20)
    a.update(kw)
    P = ctypes.c_void_p
    return bd.library().attn_bwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["o"]), P(a["dout"]),
                                 P(a["lse"]), P(a["dq"]), P(a["dk"]), P(a["dv"]), a["dtype"],
                                 a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                 a["mask_kind"], P(a["block_mask"]), a["block_q"], a["block_k"],
                                 None, P(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=1), 3), (dict(d=96), 3), (dict(Hq=3), 2), (dict(B=-1), 2), (dict(Nk=-1), 2),
    (dict(scale=0.0), 6), (dict(scale=float("inf")), 6), (dict(mask_kind=4), 6),
    (dict(mask_kind=2, block_q=32, block_k=16), 1),            # block mask pointer missing
    (dict(mask_kind=3, block_mask=16, block_q=24, block_k=16), 2),  # not a multiple of 16
    (dict(mask_kind=2, block_mask=16, block_q=64, block_k=16), 2),  # 64 does not divide 96
    (dict(q=None), 1), (dict(lse=None), 1), (dict(dk=None), 1), (dict(dout=None), 1),
    (dict(q=18), 3), (dict(dv=24), 3),
    (dict(ws=None), 4), (dict(ws_bytes=100), 4),
    (dict(B=0), 0), (dict(Nq=0, Nk=0), 0),
    # limits: at most 4096 streamed 64-row tiles per side under a block mask;
    # one (batch, head) of Q, dO, K or V under 2 GiB (32-bit offsets)
    (dict(mask_kind=2, block_mask=16, block_q=16, block_k=16, Nq=64 * 4097), 3),
    (dict(mask_kind=2, block_mask=16, block_q=16, block_k=16, Nk=64 * 4097), 3),
    (dict(mask_kind=0, Nk=1 << 23), 3),
    (dict(mask_kind=0, Nq=1 << 22), 3),
])
def test_bwd_validation(kw, status):
    """Each of these returns before anything is enqueued (no GPU needed)."""
    assert _bwd(**kw) == status


def _decm(**kw):
    a = dict(q=16, k=16, v=16, seqlens=16, o=16, lse=None, dtype=0, B=2, nt=4, Hq=8, Hkv=2,
             max_len=256, d=128, scale=0.1, chunk=0, ws=None, ws_bytes=0)
    a.update(kw)
    P = ctypes.c_void_p
    return bd.library().attn_decode_multi(P(a["q"]), P(a["k"]), P(a["v"]), P(a["seqlens"]),
                                          P(a["o"]), P(a["lse"]), a["dtype"], a["B"], a["nt"],
                                          a["Hq"], a["Hkv"], a["max_len"], a["d"], a["scale"],
                                          a["chunk"], None, P(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(nt=0), 2), (dict(nt=5), 3),            # 5 tokens x 4 heads > 16 rows
    (dict(nt=16, Hq=2, Hkv=2), 4),               # 16 x 1 fits; workspace missing
    (dict(dtype=1), 3), (dict(d=80), 3), (dict(Hq=7), 2), (dict(scale=-1.0), 6),
    (dict(seqlens=None), 1), (dict(ws=None), 4), (dict(B=0), 0),
])
def test_decode_multi_validation(kw, status):
    assert _decm(**kw) == status


def test_decode_multi_workspace_scales_with_tokens():
    one = bd.attn_decode_workspace_bytes(64, 32, 8, 32768, 128, 0)
    assert bd.attn_decode_multi_workspace_bytes(64, 1, 32, 8, 32768, 128, 0) == one
    assert bd.attn_decode_multi_workspace_bytes(64, 4, 32, 8, 32768, 128, 0) >= 4 * one - 4096
    assert bd.attn_decode_multi_workspace_bytes(64, 0, 32, 8, 32768, 128, 0) == 0


def _decp(**kw):
    a = dict(q=16, k=16, v=16, table=16, seqlens=16, o=16, lse=None, dtype=0, B=2, nt=1, Hq=8,
             Hkv=2, page_size=64, max_pages=10, d=128, scale=0.1, chunk=0, ws=None, ws_bytes=0)
    a.update(kw)
    P = ctypes.c_void_p
    return bd.library().attn_decode_paged(P(a["q"]), P(a["k"]), P(a["v"]), P(a["table"]),
                                          P(a["seqlens"]), P(a["o"]), P(a["lse"]), a["dtype"],
                                          a["B"], a["nt"], a["Hq"], a["Hkv"], a["page_size"],
                                          a["max_pages"], a["d"], a["scale"], a["chunk"], None,
                                          P(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(page_size=8), 2), (dict(page_size=48), 2), (dict(max_pages=-1), 2),
    (dict(table=None), 1), (dict(nt=5), 3), (dict(d=96), 3), (dict(ws=None), 4), (dict(B=0), 0),
])
def test_decode_paged_validation(kw, status):
    assert _decp(**kw) == status


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library every entry point raises; there is no
    other implementation to fall back on."""
    import torch
    monkeypatch.setattr(bd, "_lib", None)
    monkeypatch.setattr(bd, "LIB_PATH", str(tmp_path / "libmiattn.so"))
    with pytest.raises(RuntimeError, match="not built"):
        bd.library()
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    kv = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16)
    with pytest.raises((RuntimeError, ValueError)):
        bd.attn_fwd(q, kv, kv)


def test_product_code_does_not_use_the_oracle():
    """The package (binding, inputs, build, kernels) never imports or names
    the oracle package."""
    import pathlib
    import re
    root = pathlib.Path(bd.__file__).parent
    pat = re.compile(r"^\s*(import|from)\s+oracle\b|\boracle\.", re.M)
    for f in list(root.rglob("*.py")) + list(root.rglob("*.hip")) + list(root.rglob("*.cpp")):
        assert not pat.search(f.read_text()), f


# ---------------------------------------------------------------- clock probe
CLOCK_HEADER = os.path.join(ROOT, "include", "miclock.h")


@pytest.mark.skipif(not os.path.exists(os.path.join(ROOT, "exact_io_aware_attn_amd", "libmiclock.so")),
                    reason="libmiclock.so not built")
def test_clock_probe_library_exports_and_validates():
    """libmiclock.so exports what include/miclock.h declares, and refuses a
    NULL buffer or sizes out of range before launching anything."""
    from exact_io_aware_attn_amd import clock
    text = re.sub(r"/\*.*?\*/", "", open(CLOCK_HEADER).read(), flags=re.S)
    names = re.findall(r"^\s*int\s+([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    assert names == ["miclock_probe"]
    lib = clock.library()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation
    assert lib.miclock_probe(None, 8, 0, 100, None) == 1
    assert lib.miclock_probe(fake, 0, 0, 100, None) == 2
    assert lib.miclock_probe(fake, 1025, 0, 100, None) == 2
    assert lib.miclock_probe(fake, 8, 0, 0, None) == 2
    assert lib.miclock_probe(fake, 8, (1 << 32) + 1, 100, None) == 2
    assert lib.miclock_probe(fake, 8, 0, (1 << 32) + 1, None) == 2


def test_clock_summary_groups_probes_by_xcd():
    from exact_io_aware_attn_amd import clock
    mhz = [2000.0 + x for x in range(8)] * 2
    s = clock.summary(mhz)
    assert s["mhz_per_xcd"] == [2000.0 + x for x in range(8)]
    assert s["mhz_min"] == 2000.0 and s["mhz_max"] == 2007.0
    assert abs(s["mhz_mean"] - 2003.5) < 1e-9
