"""fp64 reference attention, written out from its definition.

Pages cited (by title and section):

* "Attention Mechanism Optimization for Efficient LLM Inference"
  (pyy0715.github.io): "Background: Scaled Dot-Product Attention" (the formula),
  "Multi-Query Attention (MQA) / Comparison" (the [batch, seq, h, d_k] layout),
  "Grouped-Query Attention (GQA)" (the head-group diagram), "Role of KV Cache"
  and "Two Phases of Inference / Decode" (one new query against the cache),
  "FlashAttention / Tiling" (the softmax row sum), "Online-Softmax" (the
  running max / running sum recurrence and its worked example).
* "플래시어텐션: 메모리를 아끼는 정확한 어텐션" (FlashAttention explainer, base.kaita.kr):
  §2 타일링 (block max m and sum l, rescaled by exp(m_block - m_total)),
  §3 알고리즘 (Theorem 1: the tiled result is exactly softmax(QK^T)V),
  §4 재계산 (only O and the statistics (m, l) are kept), §6 블록 희소 (zero
  blocks of the block mask are not computed).
* "TPU attention 최적화 실전 가이드" (aibase.it): 3단계 (frame-aligned blocks, no
  partial blocks), 4단계 (logit upper bound from the query norm and the largest
  key norm; mean-centred keys; per-head eligibility with fallback).

Everything is float64 NumPy. S and P are materialised per (batch, head) in row
chunks; rows are independent, so chunking changes nothing.
"""

import numpy as np

# Eligibility threshold for the fixed-max softmax, in nats. Parity unpinned:
# chosen here, not given by the pages (see fixed_max_bounds).
TAU = 64.0
# ... and a row must see at least this many keys to take the fixed max
# (parity unpinned as well; see fixed_max_bounds).
MIN_KEYS = 64

_ROW_CHUNK = 2048


def _check_heads(hq, hkv):
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"query heads ({hq}) must be a multiple of KV heads ({hkv})")
    return hq // hkv


def element_mask(nq, nk, *, causal=False, block_mask=None, block_q=None,
                 block_k=None, kv_len=None, rows=None):
    """Boolean [len(rows), nk] mask of allowed (query i, key j) pairs.

    Each rule is ANDed in, element by element:

    * causal: key j is visible to query i iff j <= i + (nk - nq). With nq == nk
      this is j <= i; with nq == 1 the single query sees every key, as a new
      token sees the whole cache ("Two Phases of Inference / Decode").
    * block: block_mask[i // block_q, j // block_k] != 0; a zero block is not
      computed (FlashAttention explainer §6 블록 희소).
    * kv_len: j < kv_len (the keys that exist in the cache).
    """
    if rows is None:
        rows = np.arange(nq)
    rows = np.asarray(rows)
    cols = np.arange(nk)
    allowed = np.ones((rows.size, nk), dtype=bool)
    if causal:
        allowed &= cols[None, :] <= rows[:, None] + (nk - nq)
    if block_mask is not None:
        bm = np.asarray(block_mask)
        allowed &= bm[(rows // block_q)[:, None], (cols // block_k)[None, :]] != 0
    if kv_len is not None:
        allowed &= cols[None, :] < int(kv_len)
    return allowed


def attention(q, k, v, scale, *, causal=False, block_mask=None, block_q=None,
              block_k=None, kv_len=None, heads=None, rows=None):
    """Exact attention O = softmax(scale * Q K^T) V and per-row LSE.

    q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d] (any float dtype; computed in fp64).
    kv_len: optional [B] ints, keys j >= kv_len[b] are excluded.
    heads / rows: optional subsets of query heads / query rows to evaluate
    (for sampling large problems); the result then has those extents.

    Returns (O [B, len(rows), len(heads), d] fp64, LSE [B, len(heads), len(rows)]).

    Steps, per batch b and query head h:
    1. GQA: query head h reads KV head h // (Hq / Hkv) -- contiguous groups, as
       in the GQA diagram where with 2 KV groups Q1..Q4 use KV1 and Q5..Q8 use
       KV2 ("Grouped-Query Attention (GQA)"); Hkv == 1 is MQA, Hkv == Hq is MHA.
    2. S = scale * Q K^T, materialised ("Background: Scaled Dot-Product
       Attention"; scale = 1/sqrt(d_k) there, an explicit argument here).
    3. Disallowed pairs get -inf, so they contribute exactly 0 below.
    4. m = row max of S; P = exp(S - m); l = row sum of P; P = P / l
       (the safe softmax of "FlashAttention / Tiling" and "Online-Softmax").
    5. O = P V over the allowed keys only (an Inf or NaN value at a key the row
       cannot see is no term of its sum); LSE = m + ln l (natural log of the row's normaliser over the
       scaled scores, the statistic kept for the backward pass, FlashAttention
       explainer §4 재계산).
    A row with no allowed key returns O = 0 and LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("q/k/v shapes do not agree")
    group = _check_heads(Hq, Hkv)
    heads = np.arange(Hq) if heads is None else np.asarray(heads)
    rows = np.arange(Nq) if rows is None else np.asarray(rows)

    O = np.zeros((B, rows.size, heads.size, d), dtype=np.float64)
    LSE = np.full((B, heads.size, rows.size), -np.inf, dtype=np.float64)
    for b in range(B):
        klen = None if kv_len is None else int(kv_len[b])
        for hi, h in enumerate(heads):
            kvh = h // group
            Kb = k[b, :, kvh, :]
            Vb = v[b, :, kvh, :]
            for r0 in range(0, rows.size, _ROW_CHUNK):
                rr = rows[r0:r0 + _ROW_CHUNK]
                S = scale * (q[b, rr, h, :] @ Kb.T)
                allowed = element_mask(Nq, Nk, causal=causal, block_mask=block_mask,
                                       block_q=block_q, block_k=block_k,
                                       kv_len=klen, rows=rr)
                S = np.where(allowed, S, -np.inf)
                m = S.max(axis=1)
                live = allowed.any(axis=1)
                m_safe = np.where(live, m, 0.0)
                P = np.exp(S - m_safe[:, None])
                P = np.where(allowed, P, 0.0)
                l = P.sum(axis=1)
                l_safe = np.where(live, l, 1.0)
                Pn = P / l_safe[:, None]
                fin = np.isfinite(Vb)
                if fin.all():
                    PV = Pn @ Vb
                else:
                    # the sum runs over allowed keys only: a value the row
                    # cannot see is no term of its output (0 * NaN would be).
                    # Finite values through the product (their masked
                    # weights are exact zeros), then each Inf/NaN added to
                    # the rows allowed to see its key
                    PV = Pn @ np.where(fin, Vb, 0.0)
                    for j, dc in zip(*np.nonzero(~fin)):
                        a = allowed[:, j]
                        PV[a, dc] += Pn[a, j] * Vb[j, dc]
                O[b, r0:r0 + rr.size, hi, :] = np.where(live[:, None], PV, 0.0)
                LSE[b, hi, r0:r0 + rr.size] = np.where(live, m_safe + np.log(l_safe), -np.inf)
    return O, LSE


def decode(q, k_cache, v_cache, seqlens, scale, heads=None):
    """One query token per sequence against a contiguous KV cache.

    q: [B, Hq, d]; k_cache, v_cache: [B, max_len, Hkv, d]; seqlens: [B] ints in
    [0, max_len]. The new query attends to every cached key of its sequence and
    nothing past the sequence's length ("Role of KV Cache"; "Two Phases of
    Inference / Decode": Q_new against the cache K_1..K_t). This is attention
    with Nq = 1, no causal rule, and keys limited to seqlens[b].

    Returns (O [B, Hq', d], LSE [B, Hq']).
    """
    q = np.asarray(q, dtype=np.float64)
    O, LSE = attention(q[:, None, :, :], k_cache, v_cache, scale,
                       kv_len=np.asarray(seqlens), heads=heads)
    return O[:, 0, :, :], LSE[:, :, 0]


def logit_bound(q, k, scale, *, centered=False):
    """Upper bound M[b, h, i] on every logit scale * q_i . k_j of a row.

    TPU attention guide, 4단계: by Cauchy-Schwarz, q . k <= |q| |k| <= |q| max_j |k_j|,
    so M_i = scale * |q_i| * max_j |k_j| bounds the row before any key block
    is seen. The max runs over all Nk keys of the (batch, KV head).

    centered=True uses the mean key kbar and R = max_j |k_j - kbar|:
    q . k_j = q . kbar + q . (k_j - kbar) <= q . kbar + |q| R, so
    M_i = scale * (q_i . kbar + |q_i| R) also bounds the raw logits (the guide
    notes centring can tighten the bound and leaves softmax unchanged).
    Assumes scale > 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    group = _check_heads(Hq, Hkv)
    M = np.empty((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            K = k[b, :, h // group, :]
            Q = q[b, :, h, :]
            qn = np.sqrt((Q * Q).sum(axis=1))
            if not centered:
                kmax = np.sqrt((K * K).sum(axis=1)).max()
                M[b, h] = scale * qn * kmax
            else:
                kbar = K.mean(axis=0)
                R = np.sqrt(((K - kbar) ** 2).sum(axis=1)).max()
                M[b, h] = scale * (Q @ kbar + qn * R)
    return M


def round_to_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), as float64.

    The value is first rounded to float32 (nearest even), then to the 8-bit
    significand of bfloat16 by rounding the low 16 bits of its float32 pattern
    to nearest, ties to even. Finite inputs only."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def fixed_max_bounds(q, k, scale, *, centered=False, causal=False, block_mask=None,
                     block_q=None, block_k=None, key_block=256, tau=TAU, min_keys=MIN_KEYS):
    """Per-row fixed reference M_i, its gap and eligibility, from the keys the
    row can see (TPU attention guide, 4단계).

    The guide bounds a row's logits before any key block is read: by
    Cauchy-Schwarz q . k <= |q| |k|, and with a centre c, q . k = q . c +
    q . (k - c) <= q . c + |q| |k - c| (centring tightens the bound and leaves
    the softmax unchanged). It takes one bound per head over all keys; any
    upper bound gives the same exact softmax, and this reading takes the
    bound over the keys the row can see only, so that keys a mask excludes
    never influence the row, and checks eligibility per row (finer than the
    guide's per-head check, equally sound).

    The keys of each (batch, KV head) are cut into blocks: the block mask's
    block_k when there is one, else key_block keys. A block meets row i if the
    row sees at least one of its keys; it is "full" if the row sees all of
    them. With N_j = |k_j|, for each block b meeting the row:

    * full, plain: upper = |q| max_b N_j, lower = -upper;
    * full, centred: c_b = the mean of the block's keys rounded to bfloat16,
      R_b = max_b |k_j - c_b|; upper = q . c_b + |q| R_b, lower = q . c_b - |q| R_b;
    * partial (causal cuts the block): upper = |q| max N_j over the keys the
      row sees, lower = -upper.

    Each key of the row lies in some block b, so every visible logit is at most
    M_i = scale * max_b upper; each block holds a visible key whose logit is at
    least scale * lower, so the row's max logit is at least scale * max_b lower.
    gap_i = M_i - scale * max_b lower bounds how far the row max sits below
    M_i, the row's normaliser against M_i is at least exp(-gap_i), and the row
    is eligible iff gap_i <= tau (then that normaliser stays far above the
    float32 minimum normal exp(-87.3)) and the row sees at least min_keys keys
    (a row with fewer gains nothing from a fixed reference, and with it every
    weight of the row, its largest included, would be rounded to the
    precision of the P V product). Parity unpinned: tau (default 64 nats) and
    min_keys (default 64, one key tile) are chosen here.

    Returns (M, gap, eligible), each [B, Hq, Nq]; rows that see no key get
    M = -inf, gap = nan, eligible = False.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    group = _check_heads(Hq, Hkv)
    kb_size = int(block_k) if block_mask is not None else int(key_block)
    nkb = (Nk + kb_size - 1) // kb_size
    pad = nkb * kb_size - Nk
    exists = np.concatenate([np.ones(Nk, dtype=bool), np.zeros(pad, dtype=bool)])
    exists = exists.reshape(nkb, kb_size)
    M = np.full((B, Hq, Nq), -np.inf)
    gap = np.full((B, Hq, Nq), np.nan)
    elig = np.zeros((B, Hq, Nq), dtype=bool)
    for b in range(B):
        for hk in range(Hkv):
            K = k[b, :, hk, :]
            Kp = np.concatenate([K, np.zeros((pad, d))]).reshape(nkb, kb_size, d)
            N = np.sqrt((Kp * Kp).sum(-1))                      # [nkb, kb]
            cnt = exists.sum(-1)                                # keys per block
            C = round_to_bf16(Kp.sum(1) / cnt[:, None])         # [nkb, d]
            R = np.where(exists, np.sqrt(((Kp - C[:, None, :]) ** 2).sum(-1)), -np.inf).max(-1)
            for h in range(hk * group, (hk + 1) * group):
                for r0 in range(0, Nq, _ROW_CHUNK):
                    rows = np.arange(r0, min(Nq, r0 + _ROW_CHUNK))
                    Q = q[b, rows, h, :]
                    qn = np.sqrt((Q * Q).sum(-1))[:, None]                 # [rows, 1]
                    allowed = element_mask(Nq, Nk, causal=causal, block_mask=block_mask,
                                           block_q=block_q, block_k=block_k, rows=rows)
                    A = np.concatenate([allowed, np.zeros((rows.size, pad), dtype=bool)], 1)
                    A = A.reshape(rows.size, nkb, kb_size)
                    meets = A.any(-1)                                      # [rows, nkb]
                    full = meets & (A | ~exists[None]).all(-1)
                    nvis = np.where(A, N[None], -np.inf).max(-1)           # [rows, nkb]
                    nvis = np.where(meets, nvis, 0.0)
                    if centered:
                        qc = Q @ C.T
                        up_full, lo_full = qc + qn * R[None], qc - qn * R[None]
                    else:
                        up_full, lo_full = qn * nvis, -qn * nvis
                    up = np.where(full, up_full, qn * nvis)
                    lo = np.where(full, lo_full, -qn * nvis)
                    up = np.where(meets, up, -np.inf).max(-1)
                    lo = np.where(meets, lo, -np.inf).max(-1)
                    live = meets.any(-1)
                    nseen = allowed.sum(-1)
                    Mi = np.where(live, scale * up, -np.inf)
                    with np.errstate(invalid="ignore"):
                        gi = np.where(live, scale * (up - lo), np.nan)
                    M[b, h, rows] = Mi
                    gap[b, h, rows] = gi
                    elig[b, h, rows] = (live & (nseen >= min_keys)
                                        & (np.nan_to_num(gi, nan=np.inf) <= tau))
    return M, gap, elig


def fixed_max_attention(q, k, v, scale, M, *, causal=False, block_mask=None,
                        block_q=None, block_k=None):
    """Softmax evaluated against a fixed per-row reference M instead of the max.

    P_ij = exp(S_ij - M_i) / sum_t exp(S_it - M_i). Multiplying numerator and
    denominator by exp(M_i - m_i) shows this equals the max-subtracted softmax
    exactly (the shift invariance the TPU guide's 4단계 relies on). LSE = M + ln l.
    M: [B, Hq, Nq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    group = _check_heads(Hq, Hkv)
    O = np.zeros((B, Nq, Hq, d))
    LSE = np.full((B, Hq, Nq), -np.inf)
    allowed = element_mask(Nq, Nk, causal=causal, block_mask=block_mask,
                           block_q=block_q, block_k=block_k)
    for b in range(B):
        for h in range(Hq):
            S = scale * (q[b, :, h, :] @ k[b, :, h // group, :].T)
            E = np.where(allowed, np.exp(S - M[b, h][:, None]), 0.0)
            l = E.sum(axis=1)
            live = l > 0
            ls = np.where(live, l, 1.0)
            O[b, :, h, :] = np.where(live[:, None], (E / ls[:, None]) @ v[b, :, h // group, :], 0.0)
            LSE[b, h] = np.where(live, M[b, h] + np.log(ls), -np.inf)
    return O, LSE


def online_softmax(x, block_sizes):
    """Running (max, sum) over a row read block by block.

    "Online-Softmax" (LLM inference page): for each new block B_new,
    m_new = max(m_old, max(B_new)) and
    d_new = d_old * exp(m_old - m_new) + sum(exp(B_new - m_new)).
    Returns the list of (m, d) after each block; the last pair gives the row's
    normaliser Z = exp(m) * d.
    """
    x = np.asarray(x, dtype=np.float64)
    if sum(block_sizes) != x.size:
        raise ValueError("blocks must cover the row")
    m, dsum = -np.inf, 0.0
    out = []
    pos = 0
    for n in block_sizes:
        blk = x[pos:pos + n]
        pos += n
        m_new = max(m, blk.max())
        dsum = dsum * np.exp(m - m_new) + np.exp(blk - m_new).sum()
        m = m_new
        out.append((m, dsum))
    return out


def merge_partials(o_parts, lse_parts):
    """Combine results computed over disjoint key sets.

    FlashAttention explainer §2 타일링: with a new overall max, each block's sum
    (and its output) is rescaled by exp(m_block - m_total) and added. With each
    part carrying its normalised output O_c and LSE_c = m_c + ln l_c, that is
    LSE = max_c LSE_c + ln sum_c exp(LSE_c - max) and
    O = sum_c exp(LSE_c - LSE) O_c. Parts with LSE_c = -inf contribute nothing;
    if every part is empty, O = 0 and LSE = -inf.

    o_parts: [C, ..., d]; lse_parts: [C, ...].
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    mx = lse_parts.max(axis=0)
    live = np.isfinite(mx)
    mx_safe = np.where(live, mx, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - mx_safe), 0.0)
    tot = w.sum(axis=0)
    tot_safe = np.where(live, tot, 1.0)
    lse = np.where(live, mx_safe + np.log(tot_safe), -np.inf)
    o = (w[..., None] * o_parts).sum(axis=0) / tot_safe[..., None]
    o = np.where(live[..., None], o, 0.0)
    return o, lse
