"""Comparison helpers for the GPU parity tests (HIP path vs the fp64 oracle).

Tolerances: bf16 inputs with fp32 accumulation -- O max-abs <= 1e-2 and
relative Frobenius <= 5e-3 over the tensor, LSE max-abs <= 1e-3; fp32 inputs --
O and LSE max-abs <= 1e-5. Rows with no visible key must be exactly O = 0 and
LSE = -inf on both sides.

Reading of the bf16 max-abs band: it is stated for outputs below 4 in
magnitude. A bf16 output is itself rounded to the nearest multiple of 2^-7 on
[1, 2), 2^-6 on [2, 4) and 2^-5 on [4, 8), so its own rounding error is at
most 0.0039, 0.0078 and 0.0156 there: below |O*| = 4 the band holds whatever
the kernel does right, from |O*| = 4 up no bf16 result can meet a flat 1e-2.
There the bound per element is 1e-2 + 2^-8 |O*| (the output's rounding,
at most 2^-8 |O*|, on top of the band).

Rows dominated by a few keys (inputs built for it: queries x10, keys several
times longer than the rest) carry, besides the output's rounding, the bf16
rounding of their few large weights in P (relative 2^-9, weighted by the
spread of the dominant values): for them (peaked=True) the bound per element
is 1e-2 + 2^-8 |O*| at every magnitude.

Gradients (bf16 backward): per tensor, relative Frobenius error <= 1e-2 and
max-abs error <= 2e-2 * max|reference|. Every product consumes bf16 operands
(Q, K, V, dO as given, P and dS rounded, relative error <= 2^-9 each), D_i is
formed from the bf16 output O, and each result is rounded to bf16 (2^-9):
a handful of independent 2^-9 terms per element. Where the exact gradient is
identically zero, max-abs <= 1e-4 (fp32 cancellation noise).
"""

import numpy as np
import torch

TOL = {
    "bf16": dict(o_abs=1e-2, o_rel_fro=5e-3, lse_abs=1e-3),
    "f32": dict(o_abs=1e-5, o_rel_fro=None, lse_abs=1e-5),
}


def to64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def check(o_gpu, O_ref, lse_gpu=None, LSE_ref=None, dtype="bf16", where="", peaked=False):
    tol = TOL[dtype]
    o = to64(o_gpu)
    assert o.shape == O_ref.shape, (o.shape, O_ref.shape)
    assert np.isfinite(o).all(), f"{where}: non-finite output"
    err = np.abs(o - O_ref)
    mx = float(err.max()) if err.size else 0.0
    lim = tol["o_abs"]
    if dtype == "bf16":
        big = np.abs(O_ref) >= 4.0
        if peaked:
            big = np.ones_like(big)
        lim = tol["o_abs"] + np.where(big, 2.0 ** -8 * np.abs(O_ref), 0.0)
    over = err - lim
    if err.size and float(over.max()) > 0:
        i = np.unravel_index(int(np.argmax(over)), err.shape)
        raise AssertionError(f"{where}: O error {err[i]:.3e} at {tuple(int(x) for x in i)} "
                             f"(got {o[i]:.5f}, exact {O_ref[i]:.5f}) exceeds the band; "
                             f"max-abs {mx:.3e}")
    if tol["o_rel_fro"] is not None and err.size:
        rel = float(np.linalg.norm(o - O_ref) / max(np.linalg.norm(O_ref), 1e-300))
        assert rel <= tol["o_rel_fro"], f"{where}: O rel-Frobenius {rel:.3e} > {tol['o_rel_fro']}"
    if lse_gpu is not None:
        l = to64(lse_gpu)
        assert l.shape == LSE_ref.shape, (l.shape, LSE_ref.shape)
        fin = np.isfinite(LSE_ref)
        assert np.array_equal(np.isneginf(l), np.isneginf(LSE_ref)), f"{where}: -inf rows differ"
        if fin.any():
            le = float(np.abs(l[fin] - LSE_ref[fin]).max())
            assert le <= tol["lse_abs"], f"{where}: LSE max-abs {le:.3e} > {tol['lse_abs']}"
    return mx


def check_nonfinite(o_gpu, O_ref, lse_gpu, LSE_ref, where=""):
    """Inputs with Inf/NaN values: non-finite outputs exactly where the oracle
    has them (the rows that see a key with such a value, in that value's
    columns), the rest within the band."""
    o = to64(o_gpu)
    bad_o, bad_ref = ~np.isfinite(o), ~np.isfinite(O_ref)
    assert np.array_equal(bad_o, bad_ref), (
        f"{where}: {int((bad_o & ~bad_ref).sum())} non-finite outputs the oracle has finite, "
        f"{int((bad_ref & ~bad_o).sum())} the other way")
    assert bad_ref.any(), f"{where}: the non-finite value must reach some row"
    return check(np.where(bad_o, 0.0, o), np.where(bad_ref, 0.0, O_ref), lse_gpu, LSE_ref,
                 where=where)


GRAD_TOL = dict(rel_fro=1e-2, rel_max=2e-2)
GRAD_ZERO_ABS = 1e-4


def check_grad(g_gpu, G_ref, where=""):
    """Gradient tensor against the fp64 reference; returns (rel_fro, rel_max)."""
    g = to64(g_gpu)
    assert g.shape == G_ref.shape, (g.shape, G_ref.shape)
    assert np.isfinite(g).all(), f"{where}: non-finite gradient"
    if G_ref.size == 0:
        return 0.0, 0.0
    scale = float(np.abs(G_ref).max())
    if scale == 0.0:
        # an exactly-zero gradient (one visible key: P = 1 and dP - D cancels)
        # comes out as fp32 cancellation noise between dP (MFMA sums) and D
        # (the pre-pass's sums), each of size |dO| |v| ~ sqrt(d)
        got = float(np.abs(g).max())
        assert got <= GRAD_ZERO_ABS, f"{where}: zero gradient expected, max-abs {got:.3e}"
        return 0.0, got
    rel = float(np.linalg.norm(g - G_ref) / np.linalg.norm(G_ref))
    rmax = float(np.abs(g - G_ref).max() / scale)
    assert rel <= GRAD_TOL["rel_fro"], f"{where}: rel-Frobenius {rel:.3e} > {GRAD_TOL['rel_fro']}"
    assert rmax <= GRAD_TOL["rel_max"], f"{where}: max-abs/max|ref| {rmax:.3e} > {GRAD_TOL['rel_max']}"
    return rel, rmax


def check_grad_nonfinite(g_gpu, G_ref, where=""):
    """A gradient of inputs holding Inf/NaN values: non-finite entries exactly
    where the oracle has them (the entries an allowed pair connects to such a
    value), the finite rest within the gradient band."""
    g = to64(g_gpu)
    bad_g, bad_ref = ~np.isfinite(g), ~np.isfinite(G_ref)
    assert np.array_equal(bad_g, bad_ref), (
        f"{where}: {int((bad_g & ~bad_ref).sum())} non-finite entries the oracle has finite, "
        f"{int((bad_ref & ~bad_g).sum())} the other way")
    return check_grad(np.where(bad_g, 0.0, g), np.where(bad_ref, 0.0, G_ref), where=where)


def sample_rows(n, tile=128, extra=16, seed=0, boundaries=()):
    """First and last rows, rows around every tile edge up to a cap, the given
    boundaries (and their neighbours), plus random rows -- sorted, unique."""
    rng = np.random.default_rng(seed)
    rows = {0, n - 1}
    for e in list(range(tile, n, tile))[:8] + list(range(tile, n, tile))[-4:]:
        rows |= {e - 1, e}
    for e in boundaries:
        rows |= {max(0, e - 1), min(n - 1, e)}
    rows |= set(rng.integers(0, n, size=extra).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n))
