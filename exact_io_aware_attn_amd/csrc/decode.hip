// Decode attention: one new query token per sequence (or nt <= 16/G new
// tokens, causal among themselves) against a KV cache, split over the cache
// ("split-K") and merged with the block rule.
//
// Decode reads every cached key and value once per generated token and does
// O(1) FLOPs per byte, so it is bound by HBM bandwidth ("Attention Mechanism
// Optimization for Efficient LLM Inference", "Why Decode is Memory-bound").
// The design aims at keeping every CU streaming until the end:
//  * the cached keys of all sequences are laid end to end (sum of the
//    lengths T) and cut into `splits` equal contiguous ranges, one per
//    workgroup, so every workgroup streams the same number of cache rows
//    whatever the length mix; a range that crosses a sequence boundary
//    yields one partial result per sequence it touches;
//  * a workgroup has NW waves, one per KV head of its head group; wave w
//    serves all G = Hq/Hkv query heads of its KV head, so each cache byte is
//    read once, and the waves walk the same cache rows together, so the rows
//    ([Hkv, d] contiguous per key) stream whole;
//  * each wave streams 32-key slices. Every load instruction reads whole
//    rows of its KV head (16 lanes x 16 bytes per 256-byte row), so each
//    cache line is fetched by one instruction and the loads can carry the
//    nontemporal hint (the cache is read once). K and V land in registers,
//    are written to an LDS slice private to the wave and read back in the
//    MFMA operand layouts (K: 16-byte reads; V: transposed,
//    ds_read_b64_tr_b16, for O^T = V^T P^T); the next slice's loads are in
//    flight while the current one is consumed, and no workgroup barrier sits
//    in the key loop;
//  * S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_16x16x32_bf16 with the
//    query rows of the group -- nt new tokens x G query heads, row t*G + g --
//    as the 16-wide N dimension (zero-padded). The new tokens' own keys are
//    the last nt cached rows: token t sees cache rows below len - nt + t + 1
//    (the causal rule aligned at the end), so several tokens verified or
//    generated at once share one read of the cache;
//  * rows at or past seqlens[b] are never read;
//  * a paged cache changes only the address of a row: each lane looks up its
//    row's page in the sequence's block table (a small, hot array) and reads
//    the row there; ranges, slices and the merge are the same;
//  * partial (range i, sequence b) is stored in slot i + b: the (i, b) pairs
//    that meet form a monotone staircase, so i + b is unique. A second kernel
//    merges the partials of each sequence with weights exp(LSE_c - LSE)
//    ("플래시어텐션: 메모리를 아끼는 정확한 어텐션", §2 타일링: rescale each block by
//    exp(m_block - m_total) and add).

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace miattn {

namespace {

constexpr int SL = 32;  // keys per wave slice

// Ranges: workgroup i covers flattened rows [floor(i*T/S), floor((i+1)*T/S))
// with S = min(splits, T) so that no range is empty. owner(x) is the range
// holding row x.
__device__ __forceinline__ int64_t range_lo(int64_t i, int64_t T, int64_t S) { return i * T / S; }
__device__ __forceinline__ int64_t owner(int64_t x, int64_t T, int64_t S) {
  return ((x + 1) * S - 1) / T;
}

// The lengths live on the device and cannot be checked on the host: each is
// read through this clamp to [0, max_len], so a length outside that range
// reads no row outside the sequence's cache (a longer one acts as max_len, a
// negative one as 0). Both kernels see the same clamped lengths.
__device__ __forceinline__ int seq_len(const int32_t* seqlens, int b, int max_len) {
  return min(max(seqlens[b], 0), max_len);
}

// Sum of the clamped lengths of sequences [0, n) by one wave (every lane gets
// the result).
__device__ int64_t wave_sum_lens(const int32_t* seqlens, int n, int max_len, int lane) {
  int64_t s = 0;
  for (int i = lane; i < n; i += 64) s += seq_len(seqlens, i, max_len);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  return s;
}

// NW: waves per workgroup = KV heads per workgroup (a divisor of Hkv)
template <int D, int NW, bool PAGED>
__global__ void __launch_bounds__(NW * 64, NW >= 4 ? 8 / NW : 1) decode_split_kernel(const DecodeParams p) {
  constexpr int KST = D / 32;  // k-steps (32 d each) of S^T
  constexpr int MB = D / 16;   // 16-row blocks of O^T
  constexpr int VCH = D / 8;   // 16-byte chunks per row
  constexpr int RPL = 64 / VCH;  // cache rows per load instruction
  constexpr int NL = SL / RPL;   // load instructions per slice, K and V each
  // per-wave K and V slices, row-major [SL][D] bf16 with 16-byte chunks
  // swizzled (K: the 16 rows of an operand read hit distinct banks; V: the
  // transpose reads of 4 rows x 2 chunks do). One buffer per wave suffices: a
  // wave's LDS instructions execute in order.
  __shared__ __attribute__((aligned(16))) __bf16 sKall[NW * SL * D];
  __shared__ __attribute__((aligned(16))) __bf16 sVall[NW * SL * D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;    // query row (column) of this lane: token n / G, head n % G
  const int g4 = lane >> 4;   // lane group
  const int hkv = blockIdx.y * NW + wave;
  const int G = p.Hq / p.Hkv;
  __bf16* const sk = sKall + wave * SL * D;
  __bf16* const sv = sVall + wave * SL * D;

  const int64_t T = wave_sum_lens(p.seqlens, p.B, p.max_len, lane);
  if (T == 0) return;
  const int64_t S = p.n_splits < T ? p.n_splits : T;
  const int64_t wg = blockIdx.x;
  if (wg >= S) return;
  const int64_t lo = range_lo(wg, T, S), hi = range_lo(wg + 1, T, S);

  const __bf16* __restrict__ kbase = (const __bf16*)p.kc + hkv * p.k_sh;
  const __bf16* __restrict__ vbase = (const __bf16*)p.vc + hkv * p.v_sh;
  auto vsw = [](int r, int ch) { return ch ^ ((r & 3) << 1); };
  auto ksw = [](int r, int ch) { return D == 128 ? (ch ^ (r & 15)) : (ch ^ ((r >> 1) & 7)); };
  // transpose-read addressing (see common.hpp): source lane s supplies
  // row 4*(s>>4) + ((s&15)>>2) (+16 for the second read), d 16mb + 4*(s&3)
  const int tr_row = 4 * g4 + ((lane & 15) >> 2);
  const int tr_d = 4 * (lane & 3);
  const int lrow = lane / VCH;   // row (within a load instruction's rows) of this lane
  const int lch = lane % VCH;    // its 16-byte chunk

  // walk the sequences in order; [start, start + len) is sequence b's rows
  int64_t start = 0;
  for (int b = 0; b < p.B && start < hi; ++b) {
    const int len = seq_len(p.seqlens, b, p.max_len);
    const int64_t end = start + len;
    if (len > 0 && end > lo) {
      const int k_begin = (int)((lo > start ? lo : start) - start);
      const int k_end = (int)((hi < end ? hi : end) - start);
      const __bf16* kg = kbase + (PAGED ? 0 : b * p.k_sb) + lch * 8;
      const __bf16* vg = vbase + (PAGED ? 0 : b * p.v_sb) + lch * 8;
      const int32_t* tab = PAGED ? p.table + (int64_t)b * p.max_pages : nullptr;
      const int pmask = (1 << p.page_shift) - 1;

      // Q^T as B operand: lane (n, g4), k-step t holds q[row n][32t + 8g4 .. +8]
      const int tok = n / G, hg = n - tok * G;
      // keys this row may see: cache rows below len - nt + tok + 1
      const int k_lim = len - p.nt + tok + 1;
      bf16x8 qf[KST];
      {
        const bool ok = n < G * p.nt;
        const __bf16* qp = (const __bf16*)p.q +
                           (((int64_t)b * p.nt + (ok ? tok : 0)) * p.Hq + hkv * G + (ok ? hg : 0)) * D +
                           8 * g4;
#pragma unroll
        for (int t = 0; t < KST; ++t) {
          bf16x8 z = {};
          qf[t] = ok ? *(const bf16x8*)(qp + 32 * t) : z;
        }
      }

      const int n_iter = (k_end - k_begin + SL - 1) / SL;
      // load instruction i of a slice: rows RPL*i + lrow, chunk lch
      u32x4 kreg[2][NL], vreg[2][NL];
      // paged: page of each row the lane loads for the next slice, read one
      // slice ahead of the rows themselves (so a row load never waits for its
      // table entry, and with it for the loads issued before)
      int tpg[NL];
      auto load_pages = [&](int it) {
        if constexpr (PAGED) {
          const int s0 = k_begin + it * SL + lrow;
#pragma unroll
          for (int i = 0; i < NL; ++i) {
            const int key = s0 + RPL * i;
            tpg[i] = key < k_end ? tab[key >> p.page_shift] : 0;
          }
        }
      };
      auto load_set = [&](int it, auto setc) {
        constexpr int set = decltype(setc)::value;
        const int s0 = k_begin + it * SL + lrow;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int key = s0 + RPL * i;
          const bool ok = key < k_end;
          u32x4 z = {0u, 0u, 0u, 0u};
          int64_t ko = (int64_t)key * p.k_ss, vo = (int64_t)key * p.v_ss;
          if constexpr (PAGED) {
            const int64_t page = tpg[i];
            const int64_t r = key & pmask;
            ko = page * p.k_sb + r * p.k_ss;
            vo = page * p.v_sb + r * p.v_ss;
          }
          kreg[set][i] = ok ? __builtin_nontemporal_load((const u32x4*)(kg + ko)) : z;
          vreg[set][i] = ok ? __builtin_nontemporal_load((const u32x4*)(vg + vo)) : z;
        }
      };

      f32x4 oacc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      float m_run = kNegInf, l_run = 0.f;

      // one slice: stage V, prefetch the next slice into the other register
      // set, then S^T, softmax update and O^T += V^T P^T. SET is a
      // compile-time constant so both register sets stay in registers.
      auto step = [&](int it, auto setc) {
        constexpr int SET = decltype(setc)::value;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int r = RPL * i + lrow;
          *(u32x4*)(sk + r * D + ksw(r, lch) * 8) = kreg[SET][i];
          *(u32x4*)(sv + r * D + vsw(r, lch) * 8) = vreg[SET][i];
        }
        if (it + 1 < n_iter) {
          load_set(it + 1, std::integral_constant<int, 1 - SET>());
          if (PAGED && it + 2 < n_iter) load_pages(it + 2);
        }
        wave_lds_sync();

        const int s0 = k_begin + it * SL;
        f32x4 s[2];
#pragma unroll
        for (int mb2 = 0; mb2 < 2; ++mb2) {
          s[mb2] = f32x4{0.f, 0.f, 0.f, 0.f};
          // K A operand: slice row 16mb2 + (lane&15), d 32t + 8g4 .. +8
          const int r = 16 * mb2 + (lane & 15);
#pragma unroll
          for (int t = 0; t < KST; ++t) {
            const bf16x8 ka = *(const bf16x8*)(sk + r * D + ksw(r, 4 * t + g4) * 8);
            s[mb2] = mfma16k32(ka, qf[t], s[mb2]);
          }
        }
        // lane (n, g4), register r of half mb2: key s0 + 16mb2 + 4g4 + r, head n
        float mx = kNegInf;
#pragma unroll
        for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = s0 + 16 * mb2 + 4 * g4 + r;
            float x = s[mb2][r] * p.scale_log2;
            if (key >= k_end || key >= k_lim) x = kNegInf;
            s[mb2][r] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = ex2(m_run - m_use);
        m_run = m_new;
        if (__ballot(alpha != 1.f)) {
          l_run *= alpha;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
        }
        float e[8];
#pragma unroll
        for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            e[4 * mb2 + r] = ex2(s[mb2][r] - m_use);
            l_run += e[4 * mb2 + r];
          }
        // P^T B operand: element j < 4 -> key 4g4 + j, j >= 4 -> key 16 + 4g4 + j-4
        const bf16x8 pf = cvt8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int dd = 16 * mb + tr_d;
          const s16x4 lo4 = lds_tr16(sv + tr_row * D + vsw(tr_row, dd >> 3) * 8 + (dd & 7));
          const s16x4 hi4 =
              lds_tr16(sv + (16 + tr_row) * D + vsw(16 + tr_row, dd >> 3) * 8 + (dd & 7));
          const s16x8 a16 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[mb] = mfma16k32(__builtin_bit_cast(bf16x8, a16), pf, oacc[mb]);
        }
        wave_lds_sync();
      };

      if (n_iter > 0) {
        load_pages(0);
        load_set(0, std::integral_constant<int, 0>());
        if (PAGED && n_iter > 1) load_pages(1);
      }
      for (int it = 0; it < n_iter; it += 2) {
        step(it, std::integral_constant<int, 0>());
        if (it + 1 < n_iter) step(it + 1, std::integral_constant<int, 1>());
      }

      // this range's result for sequence b: lane (n, g4) holds
      // O^T[d = 16mb + 4g4 + r][head n]; stored normalised with its LSE
      float l_tot = l_run;
      l_tot += shfl_xor(l_tot, 16);
      l_tot += shfl_xor(l_tot, 32);
      // several new tokens: the product for a slice serves tokens that see a
      // key and tokens that do not, so an Inf or NaN at such a key can reach
      // the latter through a zero weight. A row whose accumulators are not all
      // finite hands the merge a NaN LSE instead, and the merge recomputes it
      int nf = 0;
      if (p.nt > 1) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) nf |= !__builtin_isfinite(oacc[mb][r]);
        nf |= __shfl_xor(nf, 16, 64);  // the row's four lanes: n + 16 g4
        nf |= __shfl_xor(nf, 32, 64);
      }
      if (n < G * p.nt) {
        const int64_t row = ((wg + b) * p.nt + tok) * p.Hq + hkv * G + hg;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* po = p.part_o + row * D + 4 * g4;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) *(f32x4*)(po + 16 * mb) = oacc[mb] * inv;
        if (g4 == 0)
          p.part_lse[row] = nf ? __builtin_nanf("") : l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
      }
    }
    start = end;
  }
}

// Exact recompute of one row (batch b, token and query head th) over all its
// visible cache rows, for rows a range flagged (see the split kernel): keys
// one at a time with a running max, lanes holding d / 64 columns each, every
// excluded key skipped. A cold path.
template <int D>
__device__ __forceinline__ void merge_exact_row(const DecodeParams& p, int b, int th,
                                                          int len) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const int tok = th / p.Hq, hq = th - tok * p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);
  const int k_lim = min(len, len - p.nt + tok + 1);
  const int64_t bh = ((int64_t)b * p.nt + tok) * p.Hq + hq;
  const __bf16* qr = (const __bf16*)p.q + bh * D;
  const __bf16* kb = (const __bf16*)p.kc + hkv * p.k_sh;
  const __bf16* vb = (const __bf16*)p.vc + hkv * p.v_sh;
  const int pmask = (1 << p.page_shift) - 1;
  float qv[PER], acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    qv[j] = bf2f(qr[lane + 64 * j]);
    acc[j] = 0.f;
  }
  float mx = kNegInf, l = 0.f;
  for (int key = 0; key < k_lim; ++key) {
    int64_t ko = (int64_t)b * p.k_sb + (int64_t)key * p.k_ss;
    int64_t vo = (int64_t)b * p.v_sb + (int64_t)key * p.v_ss;
    if (p.table != nullptr) {
      const int64_t page = p.table[(int64_t)b * p.max_pages + (key >> p.page_shift)];
      ko = page * p.k_sb + (int64_t)(key & pmask) * p.k_ss;
      vo = page * p.v_sb + (int64_t)(key & pmask) * p.v_ss;
    }
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) dot = __builtin_fmaf(qv[j], bf2f(kb[ko + lane + 64 * j]), dot);
    const float sc = wave_sum(dot) * p.scale_log2;
    const float m_new = fmaxf(mx, sc);
    const float alpha = ex2(mx - m_new);
    const float pw = ex2(sc - m_new);
    l = l * alpha + pw;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = __builtin_fmaf(pw, bf2f(vb[vo + lane + 64 * j]), acc[j] * alpha);
    mx = m_new;
  }
  const bool live = k_lim > 0;
  __bf16* o = (__bf16*)p.o + bh * D;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[lane + 64 * j] = (__bf16)(live ? acc[j] / l : 0.f);
  if (p.lse != nullptr && lane == 0) p.lse[bh] = live ? (mx + log2f(l)) * kLn2 : kNegInf;
}

// One workgroup (a single wave) per (batch, new token, query head): merge the
// partials of the ranges that met the sequence. Each lane owns d / 64 columns.
template <int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(const DecodeParams p) {
  constexpr int PER = D / 64;
  const int bh = blockIdx.x;  // (b * nt + token) * Hq + hq
  const int rows = p.nt * p.Hq;
  const int b = bh / rows, th = bh - b * rows;
  const int lane = threadIdx.x;
  const int64_t T = wave_sum_lens(p.seqlens, p.B, p.max_len, lane);
  const int64_t start = wave_sum_lens(p.seqlens, b, p.max_len, lane);
  const int len = seq_len(p.seqlens, b, p.max_len);
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float W = 0.f, M = kNegInf;
  if (len > 0) {
    const int64_t S = p.n_splits < T ? p.n_splits : T;
    const int64_t i0 = owner(start, T, S), i1 = owner(start + len - 1, T, S);
    bool redo = false;  // a partial flagged non-finite (NaN LSE)
    for (int64_t i = i0; i <= i1; ++i) {
      const float x = p.part_lse[(i + b) * rows + th];
      redo |= x != x;
      M = fmaxf(M, x);
    }
    if (redo) {
      merge_exact_row<D>(p, b, th, len);
      return;
    }
    const float Mu = M == kNegInf ? 0.f : M;
    for (int64_t i = i0; i <= i1; ++i) {
      const int64_t row = (i + b) * rows + th;
      const float w = __expf(p.part_lse[row] - Mu);
      W += w;
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] += w * p.part_o[row * D + lane + 64 * j];
    }
    M = Mu;
  }
  __bf16* o = (__bf16*)p.o + (int64_t)bh * D;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[lane + 64 * j] = (__bf16)(W > 0.f ? acc[j] / W : 0.f);
  if (p.lse != nullptr && lane == 0) p.lse[bh] = W > 0.f ? M + logf(W) : kNegInf;
}

}  // namespace

int decode_waves_per_group(int Hkv) {
  int nw = 8;
  while (Hkv % nw) nw >>= 1;
  return nw;
}

hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  const int nw = decode_waves_per_group(p.Hkv);
  const dim3 grid(p.n_splits, p.Hkv / nw);
#define MIATTN_DECODE(DD, NWV)                                                              \
  case NWV:                                                                                 \
    if (p.table != nullptr)                                                                 \
      hipLaunchKernelGGL((decode_split_kernel<DD, NWV, true>), grid, dim3(NWV * 64), 0, s, p); \
    else                                                                                    \
      hipLaunchKernelGGL((decode_split_kernel<DD, NWV, false>), grid, dim3(NWV * 64), 0, s, p); \
    break;
  if (d == 64) {
    switch (nw) { MIATTN_DECODE(64, 8) MIATTN_DECODE(64, 4) MIATTN_DECODE(64, 2) MIATTN_DECODE(64, 1) }
  } else {
    switch (nw) { MIATTN_DECODE(128, 8) MIATTN_DECODE(128, 4) MIATTN_DECODE(128, 2) MIATTN_DECODE(128, 1) }
  }
#undef MIATTN_DECODE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d == 64)
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(p.B * p.nt * p.Hq), dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(p.B * p.nt * p.Hq), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace miattn
