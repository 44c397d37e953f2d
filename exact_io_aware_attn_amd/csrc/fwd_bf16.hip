// Prefill attention, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// The method: exact attention evaluated block by block with a running row
// max m and running sum l, so S = Q K^T and P never leave the chip
// ("플래시어텐션: 메모리를 아끼는 정확한 어텐션", §2 타일링 and §3 알고리즘;
// "Attention Mechanism Optimization for Efficient LLM Inference",
// "FlashAttention / Tiling" and "Online-Softmax").
//
// Layout of the work (our design for CDNA4, not the pages' CUDA loop order):
//  * One workgroup = 4 or 8 waves = 128 or 256 query rows of one (batch,
//    query head) (8 when the problem still yields >= 1024 workgroups); the
//    Q tile stays in VGPRs, O accumulates in VGPRs; K/V tiles of 64 keys go
//    HBM -> LDS directly (buffer loads into LDS, no staging registers),
//    double-buffered so the next tile's loads are in flight while the
//    current tile is consumed. Each load instruction fills 1 KiB of LDS in
//    lane order, so every lane fetches the global 16-byte chunk that belongs
//    in its (swizzled) LDS slot.
//  * Small d = 64 problems (fewer than 512 workgroups of 128 rows) take 64
//    rows per 4-wave workgroup and split each row block's keys between two
//    waves (alternate tiles), merging their (m, l, O) at the end with the
//    block-merge rule of the same pages (§2): half the serial tile chain of
//    the longest rows, which is what sets the time there.
//  * Each wave owns 32 query rows and computes S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16, so every lane holds the scores of ONE query
//    for 16 keys of a 32-key block: the row max needs one cross-lane step
//    (lane ^ 32) and the row sum needs none until the end.
//  * P^T feeds O^T = V^T P^T straight from the accumulator registers (the key
//    order inside each 16-key step is permuted so the accumulator layout is
//    the MFMA B-operand layout); V^T comes from the row-major LDS tile through
//    ds_read_b64_tr_b16, so V is never transposed in memory.
//  * Causal: tiles wholly above a wave's rows are skipped, the element rule is
//    applied only on tiles that cross the diagonal. Block mask: the workgroup
//    walks only the union of its rows' live key blocks; every wave lies in
//    one block row (rows are cut into 32-row segments of single block rows
//    when block_q is not a multiple of 32), so a 16-key group is live or dead
//    for the whole wave: dead groups are masked in S and skipped in PV, and a
//    wave whose block row sees the whole union applies no mask at all.
//  * The softmax scale is folded into the exponent argument (one FMA per
//    score: exp2(s * scale*log2(e) - m)), and the running max is used lazily:
//    each 32-key block is exponentiated against the row's current reference
//    m straight away, and m moves (with the O rescale) only for the rows
//    whose sum of 16 values in a lane exceeds kBlkSumMax, so neither the
//    block max nor its cross-lane step is on the common path and P stays
//    <= kBlkSumMax. Any reference gives the same exact result. O is divided
//    by the sum of the bf16-rounded weights that went into PV (a row
//    dominated by one key returns its value row exactly), the LSE uses the
//    fp32 sum of the unrounded ones.
//  * Unmasked dense tiles run as three straight-line stages in a fixed
//    instruction order: S^T of key block 0, then block 1 with block 0's
//    exps interleaved, PV of block 0 with block 1's exps, PV of block 1 --
//    the wave's VALU work issues while its own products occupy the pipe.
//  * Fixed-max softmax (TPU attention guide, 4단계): a per-row upper bound
//    M_i on the logits (Cauchy-Schwarz, over the key blocks the row can see,
//    optionally around per-block centres) replaces the running max, removing
//    the max reduction and the accumulator rescale; a row whose bound could
//    sit more than kTau nats above its max falls back to the running max.
//  * Every decision that shapes a row's arithmetic (its reference, rescales,
//    fixed or running max) is taken from that row's own visible scores and
//    keys, so the values of keys a mask excludes never change its bits.
//  * Workgroup order: heaviest causal tiles first; the query heads sharing a
//    KV head land on the same XCD (blockIdx % 8) so K/V are reused in its L2.

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace miattn {

namespace {

constexpr int BK = 64;   // keys per tile
constexpr float kBlkSumMax = 4096.f;  // lazy rescale: a lane's 16-value block sum above this

// Hardware workgroup id -> (logical tile X, member g of the head group).
// Groups of 8*G consecutive ids keep the G query heads of one KV head on one
// XCD (ids are dealt round-robin over the 8 XCDs).
// The id's divisions take the host's multiplier and shift (FwdParams::dv_*):
// three scalar instructions each instead of an emulated integer division.
__device__ __forceinline__ int fdiv(int n, uint32_t m, uint32_t s) {
  return (int)((__umulhi((uint32_t)n, m) + (uint32_t)n) >> s);
}
__device__ __forceinline__ void map_workgroup(int i, const FwdParams& p, int nX, int& X, int& g) {
  const int G = p.G;
  const int chunk = 8 * G;
  const int full = nX >> 3;
  const int c = fdiv(i, p.dv_8G_m, p.dv_8G_s);
  if (c < full) {
    const int r = i - c * chunk;
    X = c * 8 + (r & 7);
    g = r >> 3;
  } else {
    const int rr = i - full * chunk;
    const int qq = fdiv(rr, p.dv_G_m, p.dv_G_s);
    X = full * 8 + qq;
    g = rr - qq * G;
  }
}

// Exact recompute of one wave's rows (a cold path, taken only when the
// wave's accumulators hold an Inf or NaN, which a value at a key the causal
// rule hides from some of its rows can cause: the matrix product multiplies
// it by a zero weight). Row qc of lane (qc, h) is q0 + qc; the two lanes of a
// row hold halves of d. Keys are visited one at a time with a running max, every
// excluded pair skipped, so a non-finite value reaches exactly the rows that
// see its key; O and the LSE written by the main path are overwritten.
// Not inlined, so its registers do not add to the tile loop's.
template <int D, bool CAUSAL, bool BLOCK>
__device__ __attribute__((noinline)) void exact_rows(
    const __bf16* __restrict__ qb, const __bf16* __restrict__ kb, const __bf16* __restrict__ vb,
    __bf16* __restrict__ ob, float* __restrict__ lse_row, int64_t q_ss, int64_t k_ss,
    int64_t v_ss, int64_t o_ss, int Nq, int Nk, int causal_off, float scale_log2,
    const uint8_t* __restrict__ block_mask, int block_q, int block_k, int nkb, int q0, int nrows) {
  constexpr int DH = D / 2;
  const int lane = threadIdx.x & 63;
  const int qc = lane & 31, h = lane >> 5;
  const int row = q0 + qc;
  const bool ok = qc < nrows && row < Nq;
  const int r = ok ? row : q0;
  float qv[DH], o[DH];
#pragma unroll
  for (int t = 0; t < DH; t += 8) {
    const bf16x8 x = *(const bf16x8*)(qb + (int64_t)r * q_ss + h * DH + t);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[t + e] = bf2f(x[e]);
      o[t + e] = 0.f;
    }
  }
  int last = Nk - 1;
  if (CAUSAL) last = min(last, r + causal_off);
  if (!ok) last = -1;
  int last_w = last;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) last_w = max(last_w, __shfl_xor(last_w, m, 64));
  float mx = kNegInf, l = 0.f;
  for (int j = 0; j <= last_w; ++j) {
    bool vis = j <= last;
    if (BLOCK) vis = vis && block_mask[(int64_t)(r / block_q) * nkb + j / block_k] != 0;
    float dot = 0.f;
#pragma unroll
    for (int t = 0; t < DH; t += 8) {
      const bf16x8 x = *(const bf16x8*)(kb + (int64_t)j * k_ss + h * DH + t);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(qv[t + e], bf2f(x[e]), dot);
    }
    dot += shfl_xor(dot, 32);
    if (vis) {
      const float sc = dot * scale_log2;
      const float m_new = fmaxf(mx, sc);
      const float alpha = ex2(mx - m_new);
      const float pw = ex2(sc - m_new);
      l = l * alpha + pw;
#pragma unroll
      for (int t = 0; t < DH; t += 8) {
        const bf16x8 x = *(const bf16x8*)(vb + (int64_t)j * v_ss + h * DH + t);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[t + e] = __builtin_fmaf(pw, bf2f(x[e]), o[t + e] * alpha);
      }
      mx = m_new;
    }
  }
  if (!ok) return;
  const bool live = last >= 0 && (l > 0.f || l != l);
  const float inv = live ? 1.f / l : 0.f;
#pragma unroll
  for (int t = 0; t < DH; t += 4)
    *(bf16x4*)(ob + (int64_t)row * o_ss + h * DH + t) =
        cvt4(o[t] * inv, o[t + 1] * inv, o[t + 2] * inv, o[t + 3] * inv);
  if (lse_row != nullptr && h == 0) lse_row[row] = live ? (mx + log2f(l)) * kLn2 : kNegInf;
}

// NW waves per workgroup (4 or 8), 32 query rows per wave. KS = 2 splits
// the keys of each 32-row block between two waves (alternate tiles), whose
// partial (m, l, O) are merged at the end: half the serial tile chain per
// row, for problems too small to fill the chip with whole rows.
//
// FX: fixed-max mode compiled in (the bound, the per-row choice and its
// record in the workspace).
// HP: the second half of the causal row blocks (the heavier ones) issues one
// priority step above the first half; used when every workgroup is resident
// at once, so the kernel ends with the heaviest ones.
template <int D, bool CAUSAL, bool BLOCK, int NW, int KS = 1, bool FX = false, bool HP = false>
// waves per SIMD asked of the register allocator. d = 64 with 4 waves and
// whole rows: three (<= 170 VGPRs, 32 KiB of LDS per workgroup, three
// workgroups per CU). d = 64 dense with 8 waves: four (128 VGPRs, two
// workgroups per CU; a few registers spill, off the tile loop). d = 128: two.
__global__ void __launch_bounds__(64 * NW, (D == 64 && NW == 4 && KS == 1) ? 3
                                           : (D == 64 && NW == 8 && !BLOCK) ? 4
                                                                            : 8 / NW)
    fwd_bf16_kernel(const FwdParams p) {
  static_assert(KS == 1 || !BLOCK, "key split: dense masks only");
  constexpr int RW = NW / KS;        // waves per key share (one per 32-row block)
  constexpr int BQ = 32 * RW;        // query rows per workgroup
  constexpr int CH = D / 8;          // 16-byte chunks per K/V row
  constexpr int KSTEPS = D / 16;     // k-steps of the S^T MFMA
  constexpr int MB = D / 32;         // 32-row blocks of O^T
  constexpr int RPI = 1024 / (D * 2);  // tile rows per 1 KiB load instruction
  constexpr int NIW = BK / RPI / NW;   // load instructions per wave per tile

  // K/V tiles: buffer BUF of key share k is [BUF * KS + k]
  __shared__ __attribute__((aligned(16))) __bf16 sKb[2 * KS][BK * D];
  __shared__ __attribute__((aligned(16))) __bf16 sVb[2 * KS][BK * D];
  __shared__ short sLive[BLOCK ? kMaxLiveBlocks : 1];
  // BLOCK: per wave, bit i says whether live-list block i is live for the
  // wave's block row (read per tile from LDS, not from the mask in HBM)
  __shared__ uint32_t sBits[BLOCK ? NW * (kMaxLiveBlocks / 32) : 1];
  __shared__ int sCount;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qc = lane & 31;  // query column of this lane
  const int h = lane >> 5;  // which half of each 8-row group of keys
  const int rw = wave % RW;  // 32-row block of this wave
  const int kp = wave / RW;  // key share of this wave (tiles t with t % KS == kp)

  const int G = p.G;
  int X, g;
  map_workgroup(blockIdx.x, p, p.n_qtiles * p.B * p.Hkv, X, g);
  const int t2 = fdiv(X, p.dv_Hkv_m, p.dv_Hkv_s);
  const int hkv = X - t2 * p.Hkv;
  const int qt_rank = fdiv(t2, p.dv_B_m, p.dv_B_s);
  const int b = t2 - qt_rank * p.B;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - qt_rank) : qt_rank;
  const int hq = hkv * G + g;
  static_assert(!HP || (CAUSAL && !BLOCK && KS == 1), "priority boost: dense causal whole rows");
  const bool prio = HP && 2 * qt >= p.n_qtiles;

  // ---- rows of this wave. A block mask whose block_q is not a multiple of 32
  // cuts the rows into segments of at most 32 rows that never mix block rows
  // whose mask rows differ (from the segment table: runs of identical mask
  // rows, cut into 32-row pieces; lanes past a short segment hold no query),
  // so all rows of a wave see the same keys and the wave can skip the key
  // groups dead for it outright: a dead key is then never multiplied into
  // any of the wave's rows. The grid is sized for the segment count without
  // merging; workgroups past the last segment have nothing to do.
  int q_start, q_end, q0, nrows;
  if (BLOCK && p.block_q % 32 != 0) {
    const int nseg = *p.segs.count;
    const int s0 = qt * NW, sw = s0 + wave;
    if (s0 >= nseg) return;  // the same for every wave of the workgroup
    const int2 sg = sw < nseg ? p.segs.seg[sw] : make_int2(p.Nq, 0);
    q0 = sg.x;
    nrows = sg.y;
    const int2 last = p.segs.seg[min(s0 + NW, nseg) - 1];
    q_start = p.segs.seg[s0].x;
    q_end = last.x + last.y;
  } else {
    q_start = qt * BQ;
    q_end = min(q_start + BQ, p.Nq);
    q0 = q_start + rw * 32;
    nrows = 32;
  }
  const int qrow = q0 + qc;
  const bool row_ok = qc < nrows && qrow < p.Nq;
  const int wave_last = min(q0 + nrows - 1, p.Nq - 1);  // last valid row of the wave

  const __bf16* __restrict__ qg = (const __bf16*)p.q;
  const __bf16* __restrict__ kg = (const __bf16*)p.k + b * p.k_sb + hkv * p.k_sh;
  const __bf16* __restrict__ vg = (const __bf16*)p.v + b * p.v_sb + hkv * p.v_sh;

  // ---- Q fragments: lane (c, h), k-step t holds q[qrow][16t + 8h .. +8]
  bf16x8 qf[KSTEPS];
  {
    const __bf16* qp = qg + b * p.q_sb + (int64_t)qrow * p.q_ss + hq * p.q_sh + 8 * h;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      bf16x8 z = {};
      qf[t] = row_ok ? *(const bf16x8*)(qp + 16 * t) : z;
    }
  }

  // ---- key range of this workgroup
  int kv_end = p.Nk;   // dense: keys [0, kv_end)
  int n_live_keys = 0; // block: number of keys in the live-block list
  if constexpr (!BLOCK) {
    if constexpr (CAUSAL) kv_end = min(p.Nk, max(0, q_end - 1 + p.causal_off + 1));
  } else {
    // union of the live key blocks of the block rows this workgroup covers,
    // compacted in key order into sLive (wave 0, 64 blocks per step)
    if (wave == 0) {
      const int qb0 = q_start / p.block_q;
      const int qb1 = (q_end - 1) / p.block_q;
      int count = 0;
      for (int base = 0; base < p.nkb; base += 64) {
        const int kb = base + lane;
        bool live = false;
        if (kb < p.nkb)
          for (int qb = qb0; qb <= qb1; ++qb) live |= p.block_mask[(int64_t)qb * p.nkb + kb] != 0;
        const uint64_t bal = __ballot(live);
        const int pos = __popcll(bal & ((1ull << lane) - 1ull));
        if (live) sLive[count + pos] = (short)kb;
        count += __popcll(bal);
      }
      if (lane == 0) sCount = count;
    }
    __syncthreads();
    n_live_keys = __builtin_amdgcn_readfirstlane(sCount * p.block_k);
  }
  const int n_keys = BLOCK ? n_live_keys : kv_end;
  const int n_tiles = (n_keys + BK - 1) / BK;

  // BLOCK: which blocks of the union the wave's block row sees (bitmap in
  // LDS), and whether it sees all of them
  bool wave_uniform = true;
  uint32_t* const bits = sBits + (BLOCK ? wave * (kMaxLiveBlocks / 32) : 0);
  if constexpr (BLOCK) {
    if (q0 < p.Nq) {
      const int my_qb = wave_last / p.block_q;  // the wave's one block row
      for (int base = 0; base < sCount; base += 64) {
        const int i = base + lane;
        const bool live = i < sCount && p.block_mask[(int64_t)my_qb * p.nkb + sLive[i]] != 0;
        const uint64_t bal = __ballot(live);
        const int nv = min(64, sCount - base);
        wave_uniform &= bal == (nv == 64 ? ~0ull : ((1ull << nv) - 1ull));
        if (lane == 0) {
          bits[base >> 5] = (uint32_t)bal;
          if (nv > 32) bits[(base >> 5) + 1] = (uint32_t)(bal >> 32);
        }
      }
      wave_lds_sync();
    }
    wave_uniform = __builtin_amdgcn_readfirstlane((int)wave_uniform) != 0;
  }

  // ---- fixed-max bound of this lane's row, from the key blocks the row can
  // see, and the row's choice. A block meets the row if the row sees one of
  // its keys. A block the row sees whole gives upper = |q| max|k| and lower =
  // -upper (or, around the block's centre c with radius R, q.c + |q| R and
  // q.c - |q| R; the dots q.c of 32 blocks at a time on the MFMA, the centres
  // as the A operand); the block the causal rule cuts gives |q| times the
  // prefix max of |k| up to the row's last key. M = scale * max upper bounds
  // every visible logit and scale * max lower lies below the row max, so the
  // row's normaliser against M is at least exp(-gap): the row takes the fixed
  // max iff gap <= kTau and it sees at least kMinFixedKeys keys (below that,
  // the fixed max saves nothing and would round the row's largest weights to
  // bf16 too). Keys the row cannot see enter neither value.
  bool fixed_row = false;
  float m_fix = 0.f;  // bound in log2 units
  if constexpr (FX) {
    float qq = 0.f;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = bf2f(qf[t][e]);
        qq += x * x;
      }
    qq += shfl_xor(qq, 32);
    const float qn = sqrtf(qq);
    const int64_t bh = (int64_t)b * p.Hkv + hkv;
    const int KB = p.ks.kb_size, nkb = p.ks.nkb;
    const int ncand = BLOCK ? sCount : nkb;  // blocks of the live list, or all
    const float* __restrict__ pm = p.ks.pmax + bh * p.Nk;
    // last key seen by this lane's row, and by the wave's first and last rows
    const int ve = CAUSAL ? min(qrow + p.causal_off, p.Nk - 1) : p.Nk - 1;
    const int ve_lo = CAUSAL ? min(q0 + p.causal_off, p.Nk - 1) : p.Nk - 1;
    const int ve_hi = CAUSAL ? min(wave_last + p.causal_off, p.Nk - 1) : p.Nk - 1;
    const int qb = BLOCK ? wave_last / p.block_q : 0;  // the wave's block row
    float up = kNegInf, lo = kNegInf;
    int cnt = 0;  // keys the row sees
    if (p.fixed != 2) {
      // blocks every row of the wave sees whole: one block per lane
      float nmax = kNegInf, nmin = __builtin_inff();
      int call = 0;
      for (int base = 0; base < ncand; base += 64) {
        const int ci = base + lane;
        const bool valid = ci < ncand;
        const int kb = valid ? (BLOCK ? (int)sLive[ci] : ci) : 0;
        bool live = valid;
        if constexpr (BLOCK) live = live && (wave_uniform || ((bits[ci >> 5] >> (ci & 31)) & 1u));
        const int ks0 = kb * KB, ks1 = min(ks0 + KB, p.Nk) - 1;
        const bool whole = live && ks1 <= ve_lo;
        const float n = pm[ks1];
        nmax = whole ? fmaxf(nmax, n) : nmax;
        nmin = whole ? fminf(nmin, n) : nmin;
        call += whole ? ks1 - ks0 + 1 : 0;
      }
      nmax = wave_max(nmax);
      nmin = -wave_max(-nmin);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) call += __shfl_xor(call, m, 64);
      cnt = call;
      if constexpr (CAUSAL) {
        // blocks the wave's rows see differently (at most three): per row,
        // the block max if the row sees it whole, else the prefix max
        const int kb_b = ve_hi / KB;
        for (int kb = max(0, ve_lo + 1) / KB; kb <= kb_b; ++kb) {
          const bool live = !BLOCK || p.block_mask[(int64_t)qb * p.nkb + kb] != 0;
          const int ks0 = kb * KB, ks1 = min(ks0 + KB, p.Nk) - 1;
          if (live && ks0 <= ve) {
            const int last = min(ks1, ve);
            const float n = pm[last];
            nmax = fmaxf(nmax, n);
            nmin = fminf(nmin, n);
            cnt += last - ks0 + 1;
          }
        }
      }
      if (nmax > kNegInf) {
        up = qn * nmax;
        lo = -qn * nmin;
      }
    } else {
      for (int base = 0; base < ncand; base += 32) {
        // lanes L and L + 32 hold candidate base + L (L < 32): its key block
        // (or -1 when dead for the wave), its radius, and its centre as the
        // A operand of the dots
        const int ci = base + qc;
        const bool valid = ci < ncand;
        const int kb = valid ? (BLOCK ? (int)sLive[ci] : ci) : 0;
        bool live = valid;
        if constexpr (BLOCK) live = live && (wave_uniform || ((bits[ci >> 5] >> (ci & 31)) & 1u));
        const float rad = p.ks.radius[bh * nkb + kb];
        const int info = live ? kb : -1;
        const __bf16* cp = p.ks.centre + (bh * nkb + kb) * D + 8 * h;
        f32x16 dots;
#pragma unroll
        for (int r = 0; r < 16; ++r) dots[r] = 0.f;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
          const bf16x8 z = {};
          dots = mfma32(valid ? *(const bf16x8*)(cp + 16 * t) : z, qf[t], dots);
        }
        // register r holds candidate base + 8(r/4) + 4h + r%4 for this row
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int src = 8 * (r >> 2) + 4 * h + (r & 3);
          const int kbr = __shfl(info, src, 64);
          const float rr = __shfl(rad, src, 64);
          const int ks0 = kbr * KB, ks1 = min(ks0 + KB, p.Nk) - 1;
          if (kbr >= 0 && ks1 <= ve) {
            const float rq = qn * rr;
            up = fmaxf(up, dots[r] + rq);
            lo = fmaxf(lo, dots[r] - rq);
            cnt += ks1 - ks0 + 1;
          }
        }
      }
      up = fmaxf(up, shfl_xor(up, 32));
      lo = fmaxf(lo, shfl_xor(lo, 32));
      cnt += __shfl_xor(cnt, 32, 64);
      if (CAUSAL && ve >= 0) {
        // the block the causal rule cuts: the plain bound over its visible keys
        const int kb = ve / KB;
        const int ks0 = kb * KB, ks1 = min(ks0 + KB, p.Nk) - 1;
        const bool live = !BLOCK || p.block_mask[(int64_t)qb * p.nkb + kb] != 0;
        if (live && ks1 > ve) {
          const float u = qn * pm[ve];
          up = fmaxf(up, u);
          lo = fmaxf(lo, -u);
          cnt += ve - ks0 + 1;
        }
      }
    }
    const float gap = p.scale * (up - lo);
    fixed_row = row_ok && cnt >= kMinFixedKeys && up > kNegInf && gap <= kTau;
    m_fix = p.scale * up * kLog2e;
    if (p.ks.flags != nullptr && row_ok && h == 0 && kp == 0)
      p.ks.flags[((int64_t)b * p.Hq + hq) * p.Nq + qrow] = fixed_row ? 1 : 0;
  }

  // ---- staging: instruction j of this wave fills tile rows
  // r = (wave*NIW + j)*RPI + lane/CH, LDS slot lane%CH of the row, which holds
  // the logical chunk kswz(r, slot) (the swizzles are involutions).
  const int dma_row0 = wave * NIW * RPI + lane / CH;
  const int dma_slot = lane % CH;
  uint32_t dko[NIW], dvo[NIW];  // byte offsets within a tile (dense path)
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int r = dma_row0 + j * RPI;
    dko[j] = (uint32_t)(r * p.k_ss + kswz<D>(r, dma_slot) * 8) * 2u;
    dvo[j] = (uint32_t)(r * p.v_ss + vswz<D>(r, dma_slot) * 8) * 2u;
  }
  // bytes covering rows [0, n) of a [rows, stride] view with d elements per row
  auto span = [](int n, int64_t stride) -> uint32_t {
    return n > 0 ? (uint32_t)(((int64_t)(n - 1) * stride + D) * 2) : 0u;
  };
  // BLOCK: one resource over all Nk rows, rows gathered by key index
  const DmaRsrc rk_all = dma_rsrc(kg, span(p.Nk, p.k_ss));
  const DmaRsrc rv_all = dma_rsrc(vg, span(p.Nk, p.v_ss));
  // BLOCK: where this lane's row of load instruction j falls in the live-key
  // list for the next tile to be issued: live block lb_blk[j], row lb_off[j]
  // within it, and that block's id lb_id[j] (read from the list one tile
  // ahead, so the lookup's latency is off the load issue). Tiles are
  // issued in order, one list position BK further each time.
  constexpr int NJB = BLOCK ? NIW : 1;
  int lb_blk[NJB], lb_off[NJB], lb_id[NJB];
  uint32_t lb_ks[NJB], lb_vs[NJB];  // swizzled chunk offsets (bytes) of the row's slot
  int n_live_blocks = 0;
  if constexpr (BLOCK) {
    n_live_blocks = n_live_keys / p.block_k;
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int r = dma_row0 + j * RPI;
      lb_blk[j] = r / p.block_k;
      lb_off[j] = r - lb_blk[j] * p.block_k;
      lb_id[j] = sLive[min(lb_blk[j], max(n_live_blocks - 1, 0))];
      lb_ks[j] = (uint32_t)(kswz<D>(r, dma_slot) * 16);
      lb_vs[j] = (uint32_t)(vswz<D>(r, dma_slot) * 16);
    }
  }
  // step st loads tiles st * KS + k, k < KS (tiles past the end read as
  // zeros: their range is empty)
  auto issue_tile = [&](int st, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    if constexpr (!BLOCK) {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        __bf16* const dk = sKb[BUF * KS + k];
        __bf16* const dv = sVb[BUF * KS + k];
        const int r0 = (st * KS + k) * BK;
        const int nvalid = min(BK, kv_end - r0);
        const DmaRsrc rk = dma_rsrc(kg + (int64_t)r0 * p.k_ss, span(nvalid, p.k_ss));
        const DmaRsrc rv = dma_rsrc(vg + (int64_t)r0 * p.v_ss, span(nvalid, p.v_ss));
#pragma unroll
        for (int j = 0; j < NIW; ++j) {
          const int lds_row = (wave * NIW + j) * RPI;
          buf_load_lds16(rk, dk + lds_row * D, dko[j]);
          buf_load_lds16(rv, dv + lds_row * D, dvo[j]);
        }
      }
    } else {
      const int t = st;
      __bf16* const dk = sKb[BUF];
      __bf16* const dv = sVb[BUF];
#pragma unroll
      for (int j = 0; j < NIW; ++j) {
        const int r = dma_row0 + j * RPI;
        const int L = t * BK + r;
        uint32_t ko = kOutOfRange, vo = kOutOfRange;
        if (L < n_live_keys) {
          const int key = (int)__umul24(lb_id[j], p.block_k) + lb_off[j];
          ko = (uint32_t)(key * p.k_ss) * 2u + lb_ks[j];
          vo = (uint32_t)(key * p.v_ss) * 2u + lb_vs[j];
        }
        const int lds_row = (wave * NIW + j) * RPI;
        buf_load_lds16(rk_all, dk + lds_row * D, ko);
        buf_load_lds16(rv_all, dv + lds_row * D, vo);
        // the same row of the next tile: BK list positions on (block_k >= 16,
        // so at most four blocks further)
        const int off = lb_off[j] + BK;
        const int bk = p.block_k;
        const int q = (off >= bk) + (off >= 2 * bk) + (off >= 3 * bk) + (off >= 4 * bk);
        lb_off[j] = off - q * bk;
        lb_blk[j] += q;
        // the block's id for the next tile, read now and used one tile later
        // (clamped: past the list's end the row is out of range anyway)
        lb_id[j] = sLive[min(lb_blk[j], max(n_live_blocks - 1, 0))];
      }
    }
  };

  // ---- accumulators
  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mb][r] = 0.f;
  // reference of the exponent (log2 units): the row's fixed bound, or the
  // lazy running max (none yet: -FLT_MAX)
  float m_run = fixed_row ? m_fix : -__FLT_MAX__;
  // lanes whose rows keep a running max (all of them outside fixed-max mode)
  const uint64_t online_lanes = FX ? __ballot(!fixed_row) : ~0ull;
  float l_run = 0.f;      // this lane's partial row sum (half of the keys)
  // the same sum over the bf16-rounded weights used in PV, in two partial
  // sums (two independent chains of dot products)
  float l_rnd = 0.f, l_rnd_b = 0.f;
  // add the eight bf16 weights of a PV operand to the partial sums
  auto sum_rounded = [&](const bf16x8& pf) __attribute__((always_inline)) {
    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
    l_rnd = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 0, 1), one2, l_rnd, false);
    l_rnd_b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 2, 3), one2, l_rnd_b, false);
    l_rnd = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 4, 5), one2, l_rnd, false);
    l_rnd_b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 6, 7), one2, l_rnd_b, false);
  };
  const float c = p.scale_log2;

  // per-lane address pieces for the V^T transpose reads (see PV below)
  const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_ch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_half = 4 * (lane & 1);

  // one tile of keys from LDS buffer BUF (compile-time)
  auto tile_body = [&](int st, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int t = st * KS + kp;
    const __bf16* const sk = sKb[BUF * KS + kp];
    const __bf16* const sv = sVb[BUF * KS + kp];
    // ---- what this wave has to do with this tile
    // state 0: nothing visible, 1: everything visible, 2: apply the mask
    int state = 1;
    bool grp_live[4] = {true, true, true, true};  // BLOCK, per 16-key group
    const int tile_k0 = t * BK;
    if (q0 >= p.Nq || tile_k0 >= n_keys) {
      state = 0;
    } else if constexpr (!BLOCK) {
      if (CAUSAL) {
        if (tile_k0 > wave_last + p.causal_off) state = 0;
        else if (tile_k0 + BK - 1 > q0 + p.causal_off) state = 2;
      }
      if (state == 1 && tile_k0 + BK > p.Nk) state = 2;
    } else {
      // 16-key groups live for the wave (the same for every lane). A wave
      // whose block row sees the whole union has only the list's tail to
      // mask (tile_k0 < n_keys here).
      if (wave_uniform) {
        const int nl = n_live_keys - tile_k0;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) grp_live[gi] = 16 * gi < nl;
        state = (nl >= BK && !CAUSAL) ? 1 : 2;
      } else {
        bool any = false, all = true;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const int L = tile_k0 + 16 * gi;
          bool live = L < n_live_keys;
          if (live) {
            const int j = L / p.block_k;
            live = (bits[j >> 5] >> (j & 31)) & 1u;
          }
          grp_live[gi] = live;
          any |= live;
          all &= live;
        }
        state = !any ? 0 : (all && !CAUSAL) ? 1 : 2;
      }
    }

    // ---- S^T = K Q^T for the tile's two 32-key blocks (generic path)
    f32x16 s[2];
    // K fragment of block kb, k-step ks: row 32kb + qc, chunk 2ks + h
    auto kfrag = [&](int kb, int ks) {
      const int row = 32 * kb + qc;
      return *(const bf16x8*)(sk + row * D + kswz<D>(row, 2 * ks + h) * 8);
    };
    auto qk = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      bf16x8 k0 = kfrag(0, 0), k1 = kfrag(0, 1);
#pragma unroll
      for (int i = 0; i < 2 * KSTEPS; ++i) {
        bf16x8 nx = k1;
        if (i + 2 < 2 * KSTEPS) nx = kfrag((i + 2) / KSTEPS, (i + 2) % KSTEPS);
        s[i / KSTEPS] = mfma32(k0, qf[i % KSTEPS], s[i / KSTEPS]);
        k0 = k1;
        k1 = nx;
      }
    };

    // ---- mask of block kb (raw scores), without branches. Lane (qc, h),
    // register r of block kb holds key 32kb + 8(r/4) + 4h + r%4 of the tile,
    // query qrow; key group 2kb + r/8 in every lane.
    auto mask_block = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);  // key within tile
        bool ok;
        if constexpr (!BLOCK) {
          const int key = tile_k0 + kk;
          ok = key < p.Nk;
          if (CAUSAL) ok = ok && key <= qrow + p.causal_off;
        } else if constexpr (!CAUSAL) {
          ok = grp_live[kk >> 4];  // dead tail groups are not live either
        } else {
          const int L = tile_k0 + kk;
          ok = L < n_live_keys && grp_live[kk >> 4];
          if (ok) {
            const int blk = L / p.block_k;
            const int key = (int)sLive[blk] * p.block_k + (L - blk * p.block_k);
            ok = key <= qrow + p.causal_off;
          }
        }
        s[kb][r] = ok ? s[kb][r] : kNegInf;
      }
    };

    auto exps = [&](const f32x16& sb, f32x16& e, float m) __attribute__((always_inline)) {
      e[0] = ex2(__builtin_fmaf(sb[0], c, -m));
      e[1] = ex2(__builtin_fmaf(sb[1], c, -m));
      float l0 = e[0], l1 = e[1];
#pragma unroll
      for (int r = 2; r < 16; r += 2) {
        e[r] = ex2(__builtin_fmaf(sb[r], c, -m));
        e[r + 1] = ex2(__builtin_fmaf(sb[r + 1], c, -m));
        l0 += e[r];
        l1 += e[r + 1];
      }
      return l0 + l1;
    };
    // Lazy reference max: the exps of a 32-key block are taken against the
    // row's current reference m without moving it first. Only when some
    // lane's sum of its 16 values exceeds kBlkSumMax (a value above
    // kBlkSumMax/16 appeared, or the row has no reference yet: m = -FLT_MAX
    // sends every finite score to inf) does the wave take the block's exact
    // max and evaluate the block again; the rows whose own sums exceeded move
    // m and rescale O and l, the others keep m (alpha = 1, the same exps), so
    // a row's reference depends on its own scores only. Any reference gives
    // the same exact result, and P stays <= kBlkSumMax. Rows on the fixed max
    // never move.
    auto settle = [&](const f32x16& sb, f32x16& e, float& lb) __attribute__((always_inline)) {
      if (__ballot(lb > kBlkSumMax) & online_lanes) {
        const int over = lb > kBlkSumMax;
        const bool need = !fixed_row && (over | __shfl_xor(over, 32, 64)) != 0;
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sb[r]);
        mx = fmaxf(mx, shfl_xor(mx, 32)) * c;
        const float m_new = need ? fmaxf(m_run, mx) : m_run;
        const float alpha = need ? ex2(m_run - m_new) : 1.f;
        m_run = m_new;
        l_run *= alpha;
        l_rnd *= alpha;
        l_rnd_b *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
        lb = exps(sb, e, m_new);
      }
      l_run += lb;
    };

    // one 32-key block of the generic path: exps, lazy check, P in place
    auto softmax_block = [&](int kb) __attribute__((always_inline)) {
      f32x16 e;
      float lb = exps(s[kb], e, m_run);
      settle(s[kb], e, lb);
      s[kb] = e;
    };

    // ---- O^T += V^T P^T, four 16-key steps. Step u uses registers
    // 8(u%2) .. +7 of block u/2: keys 16u + 4h + e (e < 4) and
    // 16u + 8 + 4h + (e - 4) (e >= 4) for query c -- the B operand as is.
    // A operand of step u, block mb (V^T rows 32mb..+31, the step's 16
    // keys): two transpose reads, keys 16u + 8rr + 4h' + j of the groups
    auto vfrag = [&](int u, int mb) {
      const int ch = 4 * mb + tr_ch;
      const int r0 = 16 * u + tr_row, r1 = 16 * u + 8 + tr_row;
      const s16x4 lo = lds_tr16(sv + r0 * D + vswz<D>(r0, ch) * 8 + tr_half);
      const s16x4 hi = lds_tr16(sv + r1 * D + vswz<D>(r1, ch) * 8 + tr_half);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // PV of the 32-key block kb (steps 2kb, 2kb+1)
    auto pv_block = [&](int kb) __attribute__((always_inline)) {
      const f32x16& sb = s[kb];
      if constexpr (BLOCK) {
        // key group u is live or dead for the whole wave (one block row):
        // dead groups are skipped, so their V rows never meet the wave's P
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          const int u = 2 * kb + uu;
          if (!grp_live[u]) continue;
          const int o8 = 8 * uu;
          const bf16x8 pf = cvt8(sb[o8 + 0], sb[o8 + 1], sb[o8 + 2], sb[o8 + 3], sb[o8 + 4],
                                 sb[o8 + 5], sb[o8 + 6], sb[o8 + 7]);
          sum_rounded(pf);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) oacc[mb] = mfma32(vfrag(u, mb), pf, oacc[mb]);
        }
      } else {
        bf16x8 vcur = vfrag(2 * kb, 0);
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          const int o8 = 8 * uu;
          const bf16x8 pf = cvt8(sb[o8 + 0], sb[o8 + 1], sb[o8 + 2], sb[o8 + 3], sb[o8 + 4],
                                 sb[o8 + 5], sb[o8 + 6], sb[o8 + 7]);
          sum_rounded(pf);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const int nxt = uu * MB + mb + 1;
            bf16x8 vnext = vcur;
            if (nxt < 2 * MB) vnext = vfrag(2 * kb + nxt / MB, nxt % MB);
            oacc[mb] = mfma32(vcur, pf, oacc[mb]);
            vcur = vnext;
          }
        }
      }
    };
    auto body = [&](auto maskc) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(maskc)::value;
      qk();
      if constexpr (MASK) mask_block(0);
      softmax_block(0);
      pv_block(0);
      if constexpr (MASK) mask_block(1);
      softmax_block(1);
      pv_block(1);
    };
    // ---- the unmasked dense tile as three straight-line stages with a fixed
    // instruction order (sched_barrier between steps), so the wave's own
    // exp2 work issues while its products run in the matrix pipe:
    //   1. S^T of key block 0, then of block 1 interleaved with block 0's exps
    //   2. PV of block 0 interleaved with block 1's exps
    //   3. PV of block 1
    // with each block's (rare) rescale between the stages.
    constexpr int NPV = 2 * MB;  // PV MFMAs per 32-key block
    // Softmax of one 16-value block as a software pipeline over NC chunks:
    // chunk j issues the FMAs of values 2j, 2j+1, the exp2 of 2j-2, 2j-1 and
    // the sums of 2j-4, 2j-3 (the lags cover the exp latency).
    struct SmPipe {
      f32x16 x, e;
      float l0, l1;
    };
    // MK: the element rule on this tile (causal diagonal or key tail): value i
    // of a lane's block sits at key 8(i/4) + i%4 past the lane's first key of
    // the block and is kept iff that offset is <= lim; otherwise the score
    // itself becomes -inf (in place, so the rare rescale, which takes the
    // block max and evaluates the block again from the scores, sees it too)
    auto sm_chunk = [&](SmPipe& P, f32x16& sb, float m, int j, auto mkc, int lim)
                        __attribute__((always_inline)) {
      constexpr bool MK = decltype(mkc)::value;
      if (j < 8) {
        if constexpr (MK) {
          const int k0 = 8 * ((2 * j) >> 2) + ((2 * j) & 3);
          const int k1 = 8 * ((2 * j + 1) >> 2) + ((2 * j + 1) & 3);
          sb[2 * j] = k0 <= lim ? sb[2 * j] : kNegInf;
          sb[2 * j + 1] = k1 <= lim ? sb[2 * j + 1] : kNegInf;
        }
        P.x[2 * j] = __builtin_fmaf(sb[2 * j], c, -m);
        P.x[2 * j + 1] = __builtin_fmaf(sb[2 * j + 1], c, -m);
      }
      if (j >= 1 && j <= 8) {
        P.e[2 * j - 2] = ex2(P.x[2 * j - 2]);
        P.e[2 * j - 1] = ex2(P.x[2 * j - 1]);
      }
      if (j == 2) {
        P.l0 = P.e[0];
        P.l1 = P.e[1];
      } else if (j >= 3 && j <= 9) {
        P.l0 += P.e[2 * j - 4];
        P.l1 += P.e[2 * j - 3];
      }
    };
    auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
    // The wave's issue priority falls as it moves through the tile (2, 1, 0
    // by stage): of the two waves sharing a SIMD, the one further behind is
    // served first, so they reach the tile's barrier closer together.
    auto body_fast = [&](auto mkc) __attribute__((always_inline)) {
      // masked tiles (dense masks only): the last key this lane's row may
      // see, as an offset from the lane's first key of block 0
      int lim0 = 0;
      if constexpr (decltype(mkc)::value && !BLOCK) {
        int last = p.Nk - 1;
        if (CAUSAL) last = min(last, qrow + p.causal_off);
        lim0 = last - tile_k0 - 4 * h;
      }
      const int lim1 = lim0 - 32;
      if (HP && prio) __builtin_amdgcn_s_setprio(3);
      else __builtin_amdgcn_s_setprio(2);
      // ---- stage 1: S^T block 0, then block 1 with block 0's softmax
      constexpr int NK = 2 * KSTEPS;   // K fragments per tile
      constexpr int LEAD = 3;          // K fragments in flight
      bf16x8 kf[NK];
#pragma unroll
      for (int i = 0; i < LEAD; ++i) kf[i] = kfrag(i / KSTEPS, i % KSTEPS);
      fence();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const float m0 = m_run;
      SmPipe P0;
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        s[i / KSTEPS] = mfma32(kf[i], qf[i % KSTEPS], s[i / KSTEPS]);
        if (i + LEAD < NK) kf[i + LEAD] = kfrag((i + LEAD) / KSTEPS, (i + LEAD) % KSTEPS);
        // block 0's softmax starts one product after block 0 is complete
        const int j0 = i - KSTEPS - 1;
        if (j0 >= 0) {
          if constexpr (KSTEPS == 8) {
            sm_chunk(P0, s[0], m0, j0, mkc, lim0);
          } else {
            sm_chunk(P0, s[0], m0, 2 * j0, mkc, lim0);
            sm_chunk(P0, s[0], m0, 2 * j0 + 1, mkc, lim0);
          }
        }
        fence();
      }
      // rest of block 0's softmax, then the first V fragments of stage 2
      {
        constexpr int done = KSTEPS == 8 ? KSTEPS - 1 : 2 * (KSTEPS - 1);
#pragma unroll
        for (int j = done; j < 10; ++j) sm_chunk(P0, s[0], m0, j, mkc, lim0);
      }
      constexpr int VLEAD = 3;  // V fragments in flight
      bf16x8 vf[NPV];
#pragma unroll
      for (int j = 0; j < VLEAD; ++j) vf[j] = vfrag(j / MB, j % MB);
      float lb0 = P0.l0 + P0.l1;
      f32x16 e0 = P0.e;
      fence();
      if (HP && prio) __builtin_amdgcn_s_setprio(2);
      else __builtin_amdgcn_s_setprio(1);
      settle(s[0], e0, lb0);
      // ---- stage 2: PV of block 0 with block 1's softmax
      const float m1 = m_run;
      SmPipe P1;
      bf16x8 pf[2];
      pf[0] = cvt8(e0[0], e0[1], e0[2], e0[3], e0[4], e0[5], e0[6], e0[7]);
      sum_rounded(pf[0]);
      fence();
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        if (j == 1) {
          pf[1] = cvt8(e0[8], e0[9], e0[10], e0[11], e0[12], e0[13], e0[14], e0[15]);
          sum_rounded(pf[1]);
        }
        oacc[j % MB] = mfma32(vf[j], pf[j / MB], oacc[j % MB]);
        if (j + VLEAD < NPV) vf[j + VLEAD] = vfrag((j + VLEAD) / MB, (j + VLEAD) % MB);
        if constexpr (NPV == 8) {
          sm_chunk(P1, s[1], m1, j, mkc, lim1);
        } else {
          sm_chunk(P1, s[1], m1, 2 * j, mkc, lim1);
          sm_chunk(P1, s[1], m1, 2 * j + 1, mkc, lim1);
        }
        fence();
      }
      {
        constexpr int done = NPV == 8 ? NPV : 2 * NPV;
#pragma unroll
        for (int j = done; j < 10; ++j) sm_chunk(P1, s[1], m1, j, mkc, lim1);
      }
#pragma unroll
      for (int j = 0; j < VLEAD; ++j) vf[j] = vfrag(2 + j / MB, j % MB);
      float lb1 = P1.l0 + P1.l1;
      f32x16 e1 = P1.e;
      fence();
      if (HP && prio) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
      settle(s[1], e1, lb1);
      // ---- stage 3: PV of block 1
      pf[0] = cvt8(e1[0], e1[1], e1[2], e1[3], e1[4], e1[5], e1[6], e1[7]);
      sum_rounded(pf[0]);
      fence();
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        if (j == 1) {
          pf[1] = cvt8(e1[8], e1[9], e1[10], e1[11], e1[12], e1[13], e1[14], e1[15]);
          sum_rounded(pf[1]);
        }
        oacc[j % MB] = mfma32(vf[j], pf[j / MB], oacc[j % MB]);
        if (j + VLEAD < NPV) vf[j + VLEAD] = vfrag(2 + (j + VLEAD) / MB, (j + VLEAD) % MB);
        fence();
      }
    };
    // state 1 has every key group live (and no causal rule), dense or block
    // dense masks: tiles that cross the causal diagonal or hold the key tail
    // take the same fixed-order body with the element rule folded into the
    // exponent step; block masks with partly live tiles take the plain path
    if (state == 1) body_fast(std::false_type());
    else if (state == 2) {
      if constexpr (!BLOCK) body_fast(std::true_type());
      else body(std::true_type());
    }
  };

  const int n_steps = (n_tiles + KS - 1) / KS;
  // each wave waits for its own tile loads, then the barrier publishes the
  // tile to all waves (and frees the half that was just read)
  if (n_steps > 0) issue_tile(0, std::integral_constant<int, 0>());
  wait_all_loads();
  __syncthreads();
  for (int st = 0; st < n_steps; st += 2) {
    if (st + 1 < n_steps) issue_tile(st + 1, std::integral_constant<int, 1>());
    tile_body(st, std::integral_constant<int, 0>());
    wait_all_loads();
    __syncthreads();  // buffer set 0 free; step st+1 landed in set 1
    if (st + 1 < n_steps) {
      if (st + 2 < n_steps) issue_tile(st + 2, std::integral_constant<int, 0>());
      tile_body(st + 1, std::integral_constant<int, 1>());
      wait_all_loads();
      __syncthreads();
    }
  }

  l_rnd += l_rnd_b;
  float m_ref = m_run;
  if constexpr (KS > 1) {
    // ---- merge the key shares of each row block: wave rw + RW hands its
    // (m, l, O) to wave rw through LDS (the K/V buffers are free now); the
    // pages' block-merge rule, O = sum_s 2^(m_s - m) O_s, l likewise
    static_assert(KS == 2, "two key shares");
    constexpr int NX = MB * 16 + 3;  // floats per lane handed over
    static_assert(RW * NX * 64 * 4 <= (int)sizeof(sKb), "merge area");
    float* const xch = reinterpret_cast<float*>(&sKb[0][0]) + rw * NX * 64 + lane;
    if (kp == 1) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(mb * 16 + r) * 64] = oacc[mb][r];
      xch[(MB * 16) * 64] = m_ref;
      xch[(MB * 16 + 1) * 64] = l_run;
      xch[(MB * 16 + 2) * 64] = l_rnd;
    }
    __syncthreads();
    if (kp != 0) return;
    const float m1 = xch[(MB * 16) * 64];
    const float l1 = xch[(MB * 16 + 1) * 64];
    const float m = fmaxf(m_ref, m1);
    const float a0 = ex2(m_ref - m), a1 = ex2(m1 - m);
    l_run = l_run * a0 + l1 * a1;
    l_rnd = l_rnd * a0 + xch[(MB * 16 + 2) * 64] * a1;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[mb][r] = oacc[mb][r] * a0 + xch[(mb * 16 + r) * 64] * a1;
    m_ref = m;
  }

  // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) * ln 2
  const float l_tot = l_run + shfl_xor(l_run, 32);
  const bool live = l_tot > 0.f;
  // O is divided by the sum of the bf16 weights it was accumulated with (a
  // row dominated by one key then returns that key's value row exactly, the
  // weight's own rounding cancelling), the LSE uses the fp32 sum
  const float r_tot = l_rnd + shfl_xor(l_rnd, 32);
  const float inv = live && r_tot > 0.f ? 1.f / r_tot : 0.f;
  if (row_ok) {
    __bf16* op = (__bf16*)p.o + b * p.o_sb + (int64_t)qrow * p.o_ss + hq * p.o_sh;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const bf16x4 v4 = cvt4(oacc[mb][4 * jj + 0] * inv, oacc[mb][4 * jj + 1] * inv,
                               oacc[mb][4 * jj + 2] * inv, oacc[mb][4 * jj + 3] * inv);
        *(bf16x4*)(op + 32 * mb + 8 * jj + 4 * h) = v4;
      }
    if (p.lse != nullptr && h == 0)
      p.lse[((int64_t)b * p.Hq + hq) * p.Nq + qrow] = live ? (m_ref + log2f(l_tot)) * kLn2 : kNegInf;
  }
  // Under the causal rule one product serves rows that see a key and rows
  // that do not, so an Inf or NaN in V at such a key reaches the latter
  // through a zero weight. A non-finite accumulator is the only trace it can
  // leave: such a wave recomputes its rows exactly (a cold path, also taken
  // by rows whose own visible keys hold Inf or NaN, with the same result).
  if constexpr (CAUSAL) {
    bool nonfinite = false;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) nonfinite |= !__builtin_isfinite(oacc[mb][r]);
    if (__ballot(nonfinite) != 0)
      exact_rows<D, CAUSAL, BLOCK>(
          qg + b * p.q_sb + hq * p.q_sh, kg, vg, (__bf16*)p.o + b * p.o_sb + hq * p.o_sh,
          p.lse != nullptr ? p.lse + ((int64_t)b * p.Hq + hq) * p.Nq : nullptr, p.q_ss, p.k_ss,
          p.v_ss, p.o_ss, p.Nq, p.Nk, p.causal_off, p.scale_log2, p.block_mask, p.block_q,
          p.block_k, p.nkb, q0, nrows);
  }
}

// the key split is used for d = 64 dense problems with at least four key
// tiles whose 128-row workgroups would be fewer than two per CU (512): there
// the serial tile chain of the longest rows sets the time; with more
// workgroups the doubled K/V staging per row costs more than it saves
template <int D, bool BLOCK>
bool key_split(const FwdParams& p) {
  const int64_t wg128 = (int64_t)((p.Nq + 127) / 128) * p.B * p.Hq;
  return !BLOCK && D == 64 && (p.Nk + BK - 1) / BK >= 4 && wg128 < 512;
}

// multiplier and shift of the division by d (1 <= d < 2^31) used in the kernel;
// d = 0 (an empty problem, nothing launched) gives a harmless pair
static void fast_div(uint32_t d, uint32_t& m, uint32_t& s) {
  if (d == 0) {
    m = 0;
    s = 0;
    return;
  }
  uint32_t sh = 0;
  while ((1ull << sh) < d) ++sh;
  s = sh;
  m = (uint32_t)(((1ull << 32) * ((1ull << sh) - d)) / d + 1);
}

template <int D, bool CAUSAL, bool BLOCK, bool FX>
hipError_t launch_one(const FwdParams& p0, hipStream_t s) {
  // 8 waves (256 rows) per workgroup share each K/V tile when that still
  // leaves >= 1024 workgroups; smaller problems use 4 waves (128 rows). Dense
  // causal d = 64 always uses 4 waves: on the diagonal of a 256-row workgroup
  // the waves of its first rows sit idle for up to three of the tiles the
  // last rows need, which at d = 64 (three 4-wave workgroups per CU) costs
  // more than sharing each K/V tile among 8 waves saves
  FwdParams p = p0;
  p.G = p.Hq / p.Hkv;
  fast_div((uint32_t)p.G, p.dv_G_m, p.dv_G_s);
  fast_div(8u * (uint32_t)p.G, p.dv_8G_m, p.dv_8G_s);
  fast_div((uint32_t)p.Hkv, p.dv_Hkv_m, p.dv_Hkv_s);
  fast_div((uint32_t)p.B, p.dv_B_m, p.dv_B_s);
  const int64_t big = (int64_t)((p.Nq + 255) / 256) * p.B * p.Hq;
  const bool wide = big >= 1024 && !(D == 64 && CAUSAL && !BLOCK);
  // rows are cut into 32-row segments of single block rows when block_q is
  // not a multiple of 32 (see the kernel)
  const bool seg = BLOCK && p.block_q % 32 != 0;
  const int nseg = seg ? (p.Nq / p.block_q) * ((p.block_q + 31) / 32) : 0;
  if (wide) {
    p.n_qtiles = seg ? (nseg + 7) / 8 : (p.Nq + 255) / 256;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, BLOCK, 8, 1, FX>),
                       dim3(p.n_qtiles * p.B * p.Hq), dim3(512), 0, s, p);
  } else if (key_split<D, BLOCK>(p)) {
    // few workgroups of whole rows: 64 rows per workgroup, keys split in two
    p.n_qtiles = (p.Nq + 63) / 64;
    if constexpr (!BLOCK && D == 64)
      hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false, 4, 2, FX>),
                         dim3(p.n_qtiles * p.B * p.Hq), dim3(256), 0, s, p);
  } else {
    p.n_qtiles = seg ? (nseg + 3) / 4 : (p.Nq + 127) / 128;
    const int64_t nwg = (int64_t)p.n_qtiles * p.B * p.Hq;
    if constexpr (D == 64 && CAUSAL && !BLOCK) {
      // all workgroups resident at once (three per CU): boost the heavy half
      int dev = 0, ncu = 0;
      if (hipGetDevice(&dev) == hipSuccess &&
          hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
          nwg <= 3 * (int64_t)ncu) {
        hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, BLOCK, 4, 1, FX, true>), dim3(nwg), dim3(256), 0, s, p);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, BLOCK, 4, 1, FX>), dim3(nwg), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool BLOCK>
hipError_t launch_mode(const FwdParams& p, hipStream_t s) {
  return p.fixed ? launch_one<D, CAUSAL, BLOCK, true>(p, s) : launch_one<D, CAUSAL, BLOCK, false>(p, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, bool block, hipStream_t s) {
  if (p.Nq == 0 || p.B == 0) return hipSuccess;
#define MIATTN_DISPATCH(DD)                                                     \
  if (causal && block) return launch_mode<DD, true, true>(p, s);               \
  if (causal) return launch_mode<DD, true, false>(p, s);                       \
  if (block) return launch_mode<DD, false, true>(p, s);                        \
  return launch_mode<DD, false, false>(p, s);
  if (d == 64) { MIATTN_DISPATCH(64) }
  MIATTN_DISPATCH(128)
#undef MIATTN_DISPATCH
}

}  // namespace miattn
