// Backward pass of exact attention by recomputation, bf16 in and out, fp32
// accumulation, gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// FlashAttention explainer (base.kaita.kr), §4 재계산: the forward pass keeps
// only O and the row statistics; the backward pass rebuilds S and P tile by
// tile from Q, K, V in on-chip memory instead of reading an N x N matrix. Per
// (query i, key j) pair, with P_ij = exp(scale * q_i . k_j - LSE_i):
//   dV_j += P_ij dO_i,   dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - D_i),
//   dQ_i += scale dS_ij k_j,   dK_j += scale dS_ij q_i,
// where D_i = dO_i . O_i equals sum_j P_ij dP_ij (the row term of the softmax
// Jacobian). Three kernels, no atomics (outputs are bitwise repeatable):
//  * bwd_prep_kernel: D_i and LSE_i * log2(e) per row into the workspace.
//  * dK and dV: keys stationary (32 per key block, 128 per workgroup), K and
//    V in registers; Q and dO tiles of 64 rows stream through LDS for every
//    query head of the group, so dK and dV sum the group in registers. At
//    d = 64 one wave holds a key block (bwd_dkdv_kernel); at d = 128 two
//    waves share it, one holding K and dV, the other V and dK
//    (bwd_dkdv_split_kernel).
//  * bwd_dq_kernel: queries stationary (32 per wave), Q and dO in registers;
//    K and V tiles of 64 keys stream through LDS.
// The main kernels stage tiles HBM -> LDS with the LDS-DMA loads the forward
// kernel uses (rows past the end read as zeros), with one barrier per tile,
// and skip tiles the causal rule hides entirely.

#include "common.hpp"
#include "internal.hpp"

namespace miattn {

namespace {

constexpr int BT = 64;  // rows of a streamed tile (queries or keys)
constexpr int NW = 4;   // waves per workgroup, 32 stationary rows each

// LDS swizzle (row r, logical 16-byte chunk ch -> slot) for the tiles this
// pass reads both as rows and through the transpose load (Q and dO in dK/dV,
// K in dQ). A row read serves 16 lanes with 16 consecutive rows of one chunk;
// a transpose read serves 32 lanes with 4 consecutive rows (aligned to 4) of 4
// consecutive chunks. The row term is a permutation over each aligned run of
// 16 rows (d = 128; over each parity class of them at d = 64, where two rows
// share the 256 bytes of the banks) whose high bits differ within every
// aligned run of 4 rows, so neither read meets a bank twice. An involution.
template <int D>
__device__ __forceinline__ int bswz(int r, int ch) {
  if constexpr (D == 128) return ch ^ (((r & 3) << 2) | ((r >> 2) & 3));
  else return ch ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// The layout of a streamed tile: kswz (read as rows only), vswz (read both
// ways; the dQ kernel's K tile, where the extra address registers of bswz
// would spill) or bswz.
enum { SW_K = 0, SW_V = 1, SW_B = 2 };
template <int D, int SW>
__device__ __forceinline__ int swz(int r, int ch) {
  if constexpr (SW == SW_K) return kswz<D>(r, ch);
  else if constexpr (SW == SW_V) return vswz<D>(r, ch);
  else return bswz<D>(r, ch);
}

// A-operand fragment of a [BT][D] LDS tile read as rows: lane (i, h) gets row
// 32*blk + i, elements 16*ks + 8*h .. +8.
template <int D, int SW>
__device__ __forceinline__ bf16x8 row_frag(const __bf16* t, int blk, int ks, int qc, int h) {
  const int row = 32 * blk + qc;
  const int ch = 2 * ks + h;
  const int slot = swz<D, SW>(row, ch);
  return *(const bf16x8*)(t + row * D + slot * 8);
}

// A-operand fragment of the transposed tile for the 16-row step u and the
// 32-column block mb: lane (i, h') gets columns 32*mb + i of rows
// 16u + 8*(e/4) + 4h' + e%4, e = 0..7 -- the row order in which the 32x32
// accumulator holds them, so the accumulator serves as the B operand as is.
template <int D, int SW>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* t, int u, int mb, int tr_row, int tr_ch,
                                          int tr_half) {
  const int ch = 4 * mb + tr_ch;
  const int r0 = 16 * u + tr_row, r1 = 16 * u + 8 + tr_row;
  const s16x4 lo = lds_tr16(t + r0 * D + swz<D, SW>(r0, ch) * 8 + tr_half);
  const s16x4 hi = lds_tr16(t + r1 * D + swz<D, SW>(r1, ch) * 8 + tr_half);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// bytes covering rows [0, n) of a [rows, stride] view with D elements per row
template <int D>
__device__ __forceinline__ uint32_t span(int n, int64_t stride) {
  return n > 0 ? (uint32_t)(((int64_t)(n - 1) * stride + D) * 2) : 0u;
}

// Block mask over rows [q_lo, q_hi] x keys [k_lo, k_hi] (inside Nq x Nk):
// 0 every pair excluded, 1 every pair included, 2 mixed. Uniform per wave.
__device__ __forceinline__ int block_state(const BwdParams& p, int q_lo, int q_hi, int k_lo,
                                           int k_hi) {
  bool any = false, all = true;
  for (int qb = q_lo / p.block_q; qb <= q_hi / p.block_q; ++qb)
    for (int kb = k_lo / p.block_k; kb <= k_hi / p.block_k; ++kb) {
      const bool live = p.block_mask[(int64_t)qb * p.nkb + kb] != 0;
      any |= live;
      all &= live;
    }
  return !any ? 0 : all ? 1 : 2;
}

// Block mask: the streamed tiles (64 rows of queries or keys) that meet a live
// block of the workgroup's stationary range, compacted in order into list[]
// by one wave (64 candidate tiles per step); returns their count. The
// stationary range is block rows [s0, s1] (QSIDE: query blocks, the tiles are
// key tiles) or block columns [s0, s1] (key blocks, the tiles are query
// tiles); tile_range(t, a, b) gives the other axis's blocks [a, b] of tile t.
template <bool QSIDE, typename Range>
__device__ int live_tiles(const BwdParams& p, int t_begin, int t_end, int s0, int s1, Range tile_range,
                          short* list, int lane) {
  int count = 0;
  for (int base = t_begin; base < t_end; base += 64) {
    const int t = base + lane;
    bool live = false;
    if (t < t_end) {
      int a, b;
      tile_range(t, a, b);
      for (int x = s0; x <= s1 && !live; ++x)
        for (int y = a; y <= b && !live; ++y)
          live = (QSIDE ? p.block_mask[(int64_t)x * p.nkb + y] : p.block_mask[(int64_t)y * p.nkb + x]) != 0;
    }
    const uint64_t bal = __ballot(live);
    if (live) list[count + __popcll(bal & ((1ull << lane) - 1ull))] = (short)t;
    count += __popcll(bal);
  }
  return count;
}

// ---- Exact recomputation of gradient rows that turned non-finite. In a
// tile the masks cut, an excluded pair has weight 0, and 0 times an Inf or
// NaN operand (Q or dO of a row a key cannot reach, K of a key a row cannot
// see) is NaN in the matrix products. The main kernels raise a flag in the
// workspace when a wave's accumulators are non-finite; bwd_fix_kernel then
// recomputes every gradient row holding an Inf or NaN with sums over the
// visible pairs only, so such a value is no term of any gradient and values
// at visible pairs propagate as IEEE arithmetic does. Lanes split the head
// dimension (D / 64 elements each); each dot product is summed over the wave.

// dK and dV of one key of one (batch, KV head)
template <int D, bool CAUSAL, bool BLOCK>
__device__ void exact_key_row(const BwdParams& p, int b, int hkv, int key) {
  constexpr int DL = D / 64;
  const int e0 = DL * (threadIdx.x & 63);
  const int G = p.Hq / p.Hkv;
  const int64_t nstat = (int64_t)p.B * p.Hq * p.npad;
  const __bf16* kr = (const __bf16*)p.k + b * p.k_sb + (int64_t)key * p.k_ss + hkv * p.k_sh + e0;
  const __bf16* vr = (const __bf16*)p.v + b * p.v_sb + (int64_t)key * p.v_ss + hkv * p.v_sh + e0;
  float kv[DL], vv[DL], ak[DL], av[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    kv[e] = bf2f(kr[e]);
    vv[e] = bf2f(vr[e]);
    ak[e] = av[e] = 0.f;
  }
  const int q_lo = CAUSAL ? max(0, key - p.causal_off) : 0;
  for (int g = 0; g < G; ++g) {
    const int hq = hkv * G + g;
    const float* st = p.stats + ((int64_t)b * p.Hq + hq) * p.npad;
    const __bf16* qh = (const __bf16*)p.q + b * p.q_sb + hq * p.q_sh + e0;
    const __bf16* gh = (const __bf16*)p.dout + b * p.do_sb + hq * p.do_sh + e0;
    for (int q = q_lo; q < p.Nq; ++q) {
      if (BLOCK && p.block_mask[(int64_t)(q / p.block_q) * p.nkb + key / p.block_k] == 0) continue;
      float qv[DL], gv[DL], sd = 0.f, dd = 0.f;
#pragma unroll
      for (int e = 0; e < DL; ++e) {
        qv[e] = bf2f(qh[(int64_t)q * p.q_ss + e]);
        gv[e] = bf2f(gh[(int64_t)q * p.do_ss + e]);
        sd = __builtin_fmaf(qv[e], kv[e], sd);
        dd = __builtin_fmaf(gv[e], vv[e], dd);
      }
      sd = wave_sum(sd);
      dd = wave_sum(dd);
      const float pr = ex2(__builtin_fmaf(sd, p.scale_log2, -st[q]));
      const float ds = pr * (dd - st[nstat + q]);
#pragma unroll
      for (int e = 0; e < DL; ++e) {
        av[e] = __builtin_fmaf(pr, gv[e], av[e]);
        ak[e] = __builtin_fmaf(ds, qv[e], ak[e]);
      }
    }
  }
  __bf16* dkr = (__bf16*)p.dk + b * p.dk_sb + (int64_t)key * p.dk_ss + hkv * p.dk_sh + e0;
  __bf16* dvr = (__bf16*)p.dv + b * p.dv_sb + (int64_t)key * p.dv_ss + hkv * p.dv_sh + e0;
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    dkr[e] = (__bf16)(ak[e] * p.scale);
    dvr[e] = (__bf16)av[e];
  }
}

// dQ of one query row of one (batch, query head)
template <int D, bool CAUSAL, bool BLOCK>
__device__ void exact_q_row(const BwdParams& p, int b, int hq, int q) {
  constexpr int DL = D / 64;
  const int e0 = DL * (threadIdx.x & 63);
  const int hkv = hq / (p.Hq / p.Hkv);
  const int64_t nstat = (int64_t)p.B * p.Hq * p.npad;
  const int64_t srow = ((int64_t)b * p.Hq + hq) * p.npad + q;
  const __bf16* qr = (const __bf16*)p.q + b * p.q_sb + (int64_t)q * p.q_ss + hq * p.q_sh + e0;
  const __bf16* gr = (const __bf16*)p.dout + b * p.do_sb + (int64_t)q * p.do_ss + hq * p.do_sh + e0;
  const __bf16* kh = (const __bf16*)p.k + b * p.k_sb + hkv * p.k_sh + e0;
  const __bf16* vh = (const __bf16*)p.v + b * p.v_sb + hkv * p.v_sh + e0;
  float qv[DL], gv[DL], aq[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    qv[e] = bf2f(qr[e]);
    gv[e] = bf2f(gr[e]);
    aq[e] = 0.f;
  }
  const float lse2 = p.stats[srow], dsum = p.stats[nstat + srow];
  const int k_hi = CAUSAL ? min(p.Nk, q + p.causal_off + 1) : p.Nk;
  for (int key = 0; key < k_hi; ++key) {
    if (BLOCK && p.block_mask[(int64_t)(q / p.block_q) * p.nkb + key / p.block_k] == 0) continue;
    float kv[DL], sd = 0.f, dd = 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) {
      kv[e] = bf2f(kh[(int64_t)key * p.k_ss + e]);
      sd = __builtin_fmaf(qv[e], kv[e], sd);
      dd = __builtin_fmaf(gv[e], bf2f(vh[(int64_t)key * p.v_ss + e]), dd);
    }
    sd = wave_sum(sd);
    dd = wave_sum(dd);
    const float ds = ex2(__builtin_fmaf(sd, p.scale_log2, -lse2)) * (dd - dsum);
#pragma unroll
    for (int e = 0; e < DL; ++e) aq[e] = __builtin_fmaf(ds, kv[e], aq[e]);
  }
  __bf16* dqr = (__bf16*)p.dq + b * p.dq_sb + (int64_t)q * p.dq_ss + hq * p.dq_sh + e0;
#pragma unroll
  for (int e = 0; e < DL; ++e) dqr[e] = (__bf16)(aq[e] * p.scale);
}

// A gradient row (D / 64 elements per lane) holds an Inf or NaN.
template <int D>
__device__ __forceinline__ bool row_nonfinite(const __bf16* r) {
  constexpr int DL = D / 64;
  bool bad = false;
#pragma unroll
  for (int e = 0; e < DL; ++e) bad |= !__builtin_isfinite(bf2f(r[DL * (threadIdx.x & 63) + e]));
  return __ballot(bad) != 0;
}

// Raised by each lane that wrote an Inf or NaN (a vector store under the
// lanes' own condition; a ballot first cost the d = 64 dK/dV kernel ten
// registers and its third wave per SIMD)
__device__ __forceinline__ void raise_flag(const BwdParams& p, bool nonfinite) {
  if (nonfinite) *p.flag = 1;
}

// ---- D_i = dO_i . O_i (fp32) and LSE_i * log2(e), per (batch, head, row);
// rows Nq .. npad-1 get D = 0 and +inf (their weights exp2(s - inf) are 0).
// D/8 lanes per row, 16 bytes each.
template <int D>
__global__ void __launch_bounds__(256) bwd_prep_kernel(const BwdParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int64_t total = (int64_t)p.B * p.Hq * p.npad;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int ch = threadIdx.x % LPR;
  if (blockIdx.x == 0 && threadIdx.x == 0) *p.flag = 0;
  if (row >= total) return;  // whole groups of LPR lanes leave together
  const int i = (int)(row % p.npad);
  const int64_t bh = row / p.npad;
  const int hq = (int)(bh % p.Hq);
  const int b = (int)(bh / p.Hq);
  float acc = 0.f;
  if (i < p.Nq) {
    const bf16x8 o = *(const bf16x8*)((const __bf16*)p.o + b * p.o_sb + (int64_t)i * p.o_ss +
                                      hq * p.o_sh + 8 * ch);
    const bf16x8 g = *(const bf16x8*)((const __bf16*)p.dout + b * p.do_sb +
                                      (int64_t)i * p.do_ss + hq * p.do_sh + 8 * ch);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(bf2f(o[e]), bf2f(g[e]), acc);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += shfl_xor(acc, m);
  if (ch == 0) {
    p.stats[row] = i < p.Nq ? p.lse[bh * p.Nq + i] * kLog2e : __builtin_inff();
    p.stats[total + row] = acc;
  }
}

// ---- dK and dV. Workgroup: 128 keys of one (batch, KV head); wave w holds
// keys 32w .. 32w+31 as B operands (lane (c, h): key c, elements 16t + 8h).
// S[q][key] = Q K^T and dP[q][key] = dO V^T come out with lane (c, h)
// holding key c for the 16 query rows 8*(r/4) + 4h + r%4 of a 32-row block;
// P and dS in that layout are the B operands of dV^T += dO^T P and
// dK^T += Q^T dS, whose A operands are transposed reads of the dO and Q tiles.
// Used at d = 64, where K, V and both accumulators (96 registers) leave room
// for two waves per SIMD; d = 128 splits each key block over two waves
// (bwd_dkdv_split_kernel below).
template <int D, bool CAUSAL, bool BLOCK>
__global__ void __launch_bounds__(64 * NW, 2) bwd_dkdv_kernel(const BwdParams p) {
  static_assert(D == 64, "d = 128 runs bwd_dkdv_split_kernel");
  constexpr int CH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int MB = D / 32;
  constexpr int RPI = 1024 / (D * 2);  // tile rows per 1 KiB load instruction
  constexpr int NIW = BT / RPI / NW;   // load instructions per wave per tile and tensor
  // Q and dO layout: vswz; bswz's extra address arithmetic measured slower
  // here than the row reads' bank conflicts
  constexpr int SWT = SW_V;

  __shared__ __attribute__((aligned(16))) __bf16 sQ[2][BT * D];
  __shared__ __attribute__((aligned(16))) __bf16 sG[2][BT * D];    // dO
  __shared__ __attribute__((aligned(16))) float sSt[2][2 * BT];   // lse2 then dsum
  __shared__ short sTile[BLOCK ? kMaxBwdTiles : 1];  // live query tiles (block mask)
  __shared__ int sNT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qc = lane & 31;
  const int h = lane >> 5;

  const int nbh = p.B * p.Hkv;
  const int bh = blockIdx.x % nbh;
  const int kt = blockIdx.x / nbh;  // key tiles in order: causal ones with most queries first
  const int b = bh / p.Hkv;
  const int hkv = bh % p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int k0w = kt * 128 + 32 * wave;  // first key of this wave
  const int key = k0w + qc;
  const bool key_ok = key < p.Nk;

  // stationary K and V fragments
  bf16x8 kf[KSTEPS], vf[KSTEPS];
  {
    const __bf16* kp = (const __bf16*)p.k + b * p.k_sb + (int64_t)key * p.k_ss + hkv * p.k_sh + 8 * h;
    const __bf16* vp = (const __bf16*)p.v + b * p.v_sb + (int64_t)key * p.v_ss + hkv * p.v_sh + 8 * h;
    const bf16x8 z = {};
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      kf[t] = key_ok ? *(const bf16x8*)(kp + 16 * t) : z;
      vf[t] = key_ok ? *(const bf16x8*)(vp + 16 * t) : z;
    }
  }

  // queries that can see the workgroup's keys: q >= key - causal_off
  int qb0 = 0;
  if constexpr (CAUSAL) qb0 = max(0, kt * 128 - p.causal_off) / BT * BT;
  int n_qt = p.Nq > qb0 ? (p.Nq - qb0 + BT - 1) / BT : 0;
  if constexpr (BLOCK) {
    // query tiles meeting a live block of the workgroup's key blocks
    if (wave == 0) {
      const int kb0 = kt * 128 / p.block_k, kb1 = (min(kt * 128 + 128, p.Nk) - 1) / p.block_k;
      const int n = live_tiles<false>(
          p, qb0 / BT, (p.Nq + BT - 1) / BT, kb0, kb1,
          [&](int t, int& a, int& b) {
            a = t * BT / p.block_q;
            b = (min(t * BT + BT, p.Nq) - 1) / p.block_q;
          },
          sTile, lane);
      if (lane == 0) sNT = n;
    }
    __syncthreads();
    n_qt = sNT;
  }
  // first row of the workgroup's i-th query tile
  auto tile_row = [&](int i) { return BLOCK ? (int)sTile[i] * BT : qb0 + i * BT; };
  const int n_steps = G * n_qt;  // step s: query head hkv*G + s / n_qt, tile s % n_qt

  // ---- staging: instruction j of this wave fills tile rows
  // (wave*NIW + j)*RPI + lane/CH, LDS slot lane%CH holding chunk swz(r, slot)
  const int dma_row0 = wave * NIW * RPI + lane / CH;
  const int dma_slot = lane % CH;
  uint32_t qo[NIW], go[NIW];
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int r = dma_row0 + j * RPI;
    qo[j] = (uint32_t)(r * p.q_ss + swz<D, SWT>(r, dma_slot) * 8) * 2u;
    go[j] = (uint32_t)(r * p.do_ss + swz<D, SWT>(r, dma_slot) * 8) * 2u;
  }
  const int64_t nstat = (int64_t)p.B * p.Hq * p.npad;
  const DmaRsrc rst = dma_rsrc(p.stats, (uint32_t)(2 * nstat * 4));
  auto issue = [&](int st, int buf) {
    const int g = st / n_qt;
    const int r0 = tile_row(st - g * n_qt);
    const int hq = hkv * G + g;
    const int nvalid = min(BT, p.Nq - r0);
    const __bf16* qb = (const __bf16*)p.q + b * p.q_sb + (int64_t)r0 * p.q_ss + hq * p.q_sh;
    const __bf16* gb = (const __bf16*)p.dout + b * p.do_sb + (int64_t)r0 * p.do_ss + hq * p.do_sh;
    const DmaRsrc rq = dma_rsrc(qb, span<D>(nvalid, p.q_ss));
    const DmaRsrc rg = dma_rsrc(gb, span<D>(nvalid, p.do_ss));
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int lds_row = (wave * NIW + j) * RPI;
      buf_load_lds16(rq, sQ[buf] + lds_row * D, qo[j]);
      buf_load_lds16(rg, sG[buf] + lds_row * D, go[j]);
    }
    // statistics of the tile's 64 rows (always inside the padded rows):
    // lanes 0-15 the lse2 row, lanes 16-31 the dsum row, 16 bytes each
    if (wave == 0 && lane < 32) {
      const int64_t srow = ((int64_t)b * p.Hq + hq) * p.npad + r0;
      const uint32_t off = (uint32_t)((srow + (lane >= 16 ? nstat : 0)) * 4 + 16 * (lane & 15));
      buf_load_lds16(rst, sSt[buf], off);
    }
  };

  f32x16 dkacc[MB], dvacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkacc[mb][r] = dvacc[mb][r] = 0.f;
  const float c = p.scale_log2;
  const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_ch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_half = 4 * (lane & 1);

  // one 32-query block qb of the tile: products, softmax, gradient products
  auto scores = [&](const __bf16* sq, const __bf16* sg, int qb, f32x16& s, f32x16& dp)
      __attribute__((always_inline)) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      s = mfma32(row_frag<D, SWT>(sq, qb, t, qc, h), kf[t], s);
      dp = mfma32(row_frag<D, SWT>(sg, qb, t, qc, h), vf[t], dp);
    }
  };
  // P = exp2(c s - lse2) into s and dS = P (dP - D) into dp, rows 8j + 4h + i
  const int key_blk = (BLOCK && key_ok) ? key / p.block_k : 0;  // this lane's mask column
  auto softmax = [&](const float* ss, int qb, int qs, bool masked, f32x16& s, f32x16& dp)
      __attribute__((always_inline)) {
    // block mask, mixed region: the 32 rows span at most three block rows;
    // their flags for this lane's key block are read once, and each row picks
    // one by comparing with the block-row boundaries
    bool fl0 = false, fl1 = false, fl2 = false;
    int qbb1 = 0, qbb2 = 0;
    if (BLOCK && masked) {
      const int qb0 = qs / p.block_q, nqb = p.Nq / p.block_q;
      qbb1 = (qb0 + 1) * p.block_q;
      qbb2 = (qb0 + 2) * p.block_q;
      const uint8_t* col = p.block_mask + key_blk;
      if (key_ok) {
        fl0 = col[(int64_t)qb0 * p.nkb] != 0;
        fl1 = qb0 + 1 < nqb && col[(int64_t)(qb0 + 1) * p.nkb] != 0;
        fl2 = qb0 + 2 < nqb && col[(int64_t)(qb0 + 2) * p.nkb] != 0;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 l4 = *(const f32x4*)(ss + 32 * qb + 8 * j + 4 * h);
      const f32x4 d4 = *(const f32x4*)(ss + BT + 32 * qb + 8 * j + 4 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * j + i;
        float pr = ex2(__builtin_fmaf(s[r], c, -l4[i]));
        if ((CAUSAL || BLOCK) && masked) {
          const int q = qs + 8 * j + 4 * h + i;
          bool ok = true;
          if (CAUSAL) ok = key <= q + p.causal_off;
          if (BLOCK) ok = ok && q < p.Nq && (q >= qbb2 ? fl2 : q >= qbb1 ? fl1 : fl0);
          pr = ok ? pr : 0.f;
        }
        s[r] = pr;
        dp[r] = pr * (dp[r] - d4[i]);
      }
    }
  };
  auto grads = [&](const __bf16* sq, const __bf16* sg, int qb, const f32x16& s, const f32x16& dp)
      __attribute__((always_inline)) {
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int u = 2 * qb + uu;
      const int o8 = 8 * uu;
      const bf16x8 pf = cvt8(s[o8 + 0], s[o8 + 1], s[o8 + 2], s[o8 + 3], s[o8 + 4], s[o8 + 5],
                             s[o8 + 6], s[o8 + 7]);
      const bf16x8 df = cvt8(dp[o8 + 0], dp[o8 + 1], dp[o8 + 2], dp[o8 + 3], dp[o8 + 4],
                             dp[o8 + 5], dp[o8 + 6], dp[o8 + 7]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        dvacc[mb] = mfma32(tr_frag<D, SWT>(sg, u, mb, tr_row, tr_ch, tr_half), pf, dvacc[mb]);
        dkacc[mb] = mfma32(tr_frag<D, SWT>(sq, u, mb, tr_row, tr_ch, tr_half), df, dkacc[mb]);
      }
    }
  };

  auto body = [&](int st, int buf) {
    const int g = st / n_qt;
    const int r0 = tile_row(st - g * n_qt);
    const __bf16* sq = sQ[buf];
    const __bf16* sg = sG[buf];
    const float* ss = sSt[buf];
    // per 32-query block: 0 no pair visible, 1 all visible, 2 apply the causal rule
    int state[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qs = r0 + 32 * qb;
      state[qb] = 1;
      if (qs >= p.Nq || k0w >= p.Nk) state[qb] = 0;
      else if (CAUSAL) {
        if (qs + 31 + p.causal_off < k0w) state[qb] = 0;
        else if (qs + p.causal_off < k0w + 31) state[qb] = 2;
      }
      if (BLOCK && state[qb] != 0) {
        const int bs = block_state(p, qs, min(qs + 31, p.Nq - 1), k0w, min(k0w + 31, p.Nk - 1));
        state[qb] = bs == 0 ? 0 : (bs == 2 ? 2 : state[qb]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (state[qb] == 0) continue;
      f32x16 s, dp;
      scores(sq, sg, qb, s, dp);
      softmax(ss, qb, r0 + 32 * qb, state[qb] == 2, s, dp);
      grads(sq, sg, qb, s, dp);
    }
  };

  if (n_steps > 0) issue(0, 0);
  wait_all_loads();
  __syncthreads();
  for (int st = 0; st < n_steps; ++st) {
    const int buf = st & 1;
    if (st + 1 < n_steps) issue(st + 1, buf ^ 1);
    body(st, buf);
    wait_all_loads();
    __syncthreads();  // buffer buf free; step st+1 landed in buf^1
  }

  // ---- epilogue: dK = scale * acc, dV = acc; lane (c, h) holds dims
  // 32mb + 8jj + 4h .. +3 of key c
  // with masks, an Inf or NaN written here raises the flag (bwd_fix_kernel):
  // x * 0 is 0 for finite x and NaN otherwise
  float nf = 0.f;
  if (key_ok) {
    __bf16* dkp = (__bf16*)p.dk + b * p.dk_sb + (int64_t)key * p.dk_ss + hkv * p.dk_sh;
    __bf16* dvp = (__bf16*)p.dv + b * p.dv_sb + (int64_t)key * p.dv_ss + hkv * p.dv_sh;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = dkacc[mb];
        const f32x16& v = dvacc[mb];
        if constexpr (CAUSAL || BLOCK)
          for (int i = 0; i < 4; ++i)
            nf = __builtin_fmaf(a[4 * jj + i], 0.f, __builtin_fmaf(v[4 * jj + i], 0.f, nf));
        *(bf16x4*)(dkp + 32 * mb + 8 * jj + 4 * h) =
            cvt4(a[4 * jj] * p.scale, a[4 * jj + 1] * p.scale, a[4 * jj + 2] * p.scale,
                 a[4 * jj + 3] * p.scale);
        *(bf16x4*)(dvp + 32 * mb + 8 * jj + 4 * h) =
            cvt4(v[4 * jj], v[4 * jj + 1], v[4 * jj + 2], v[4 * jj + 3]);
      }
  }
  if constexpr (CAUSAL || BLOCK) raise_flag(p, nf != 0.f);
}

// ---- dK and dV at d = 128 with each 32-key block's work split over two
// waves, so that each holds half the stationary registers and two waves share
// a SIMD. Workgroup: 128 keys of one (batch, KV head), 8 waves; waves w and
// w + 4 cover keys 32w .. 32w+31 (lane (c, h): key c, elements 16t + 8h):
//  * wave w (the P wave) holds K and accumulates dV^T: S = Q K^T, P =
//    exp2(c S - lse2) with the masks, P to LDS as bf16, dV^T += dO^T P;
//  * wave w + 4 (the dS wave) holds V and accumulates dK^T: dP = dO V^T, P
//    from LDS, dS = P (dP - D), dK^T += Q^T dS.
// The dS wave runs one tile behind the P wave, so one barrier per tile
// publishes both a tile's P and the next tile's Q and dO: three Q/dO buffers
// (the P wave's tile, the dS wave's tile, the one loading) and two P buffers.
// Fragment layouts and the order of products into each accumulator are the
// d = 64 kernel's; dS is formed from the bf16 P that dV also consumes. Q and
// dO sit in LDS as bswz (under vswz the row reads meet each bank four times).
constexpr int NWS = 8;

template <bool CAUSAL, bool BLOCK>
__global__ void __launch_bounds__(64 * NWS, 2) bwd_dkdv_split_kernel(const BwdParams p) {
  constexpr int D = 128;
  constexpr int CH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int MB = D / 32;
  constexpr int RPI = 1024 / (D * 2);
  constexpr int NIW = BT / RPI / NWS;  // load instructions per wave per tile and tensor

  __shared__ __attribute__((aligned(16))) __bf16 sQ[3][BT * D];
  __shared__ __attribute__((aligned(16))) __bf16 sG[3][BT * D];   // dO
  __shared__ __attribute__((aligned(16))) float sSt[3][2 * BT];  // lse2 then dsum
  __shared__ bf16x8 sP[2][NW][2][2][64];  // [buffer][key block][query block][half][lane]
  __shared__ short sTile[BLOCK ? kMaxBwdTiles : 1];
  __shared__ int sNT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kw = wave & (NW - 1);  // key block of the wave
  const bool pw = wave < NW;       // P wave (else dS wave)
  const int qc = lane & 31;
  const int h = lane >> 5;

  const int nbh = p.B * p.Hkv;
  const int bh = blockIdx.x % nbh;
  const int kt = blockIdx.x / nbh;
  const int b = bh / p.Hkv;
  const int hkv = bh % p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int k0w = kt * 128 + 32 * kw;
  const int key = k0w + qc;
  const bool key_ok = key < p.Nk;

  // stationary fragments: K (P wave) or V (dS wave)
  bf16x8 sf[KSTEPS];
  {
    const __bf16* sp = pw ? (const __bf16*)p.k + b * p.k_sb + (int64_t)key * p.k_ss + hkv * p.k_sh
                          : (const __bf16*)p.v + b * p.v_sb + (int64_t)key * p.v_ss + hkv * p.v_sh;
    const bf16x8 z = {};
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) sf[t] = key_ok ? *(const bf16x8*)(sp + 8 * h + 16 * t) : z;
  }

  int qb0 = 0;
  if constexpr (CAUSAL) qb0 = max(0, kt * 128 - p.causal_off) / BT * BT;
  int n_qt = p.Nq > qb0 ? (p.Nq - qb0 + BT - 1) / BT : 0;
  if constexpr (BLOCK) {
    if (wave == 0) {
      const int kb0 = kt * 128 / p.block_k, kb1 = (min(kt * 128 + 128, p.Nk) - 1) / p.block_k;
      const int n = live_tiles<false>(
          p, qb0 / BT, (p.Nq + BT - 1) / BT, kb0, kb1,
          [&](int t, int& a, int& b) {
            a = t * BT / p.block_q;
            b = (min(t * BT + BT, p.Nq) - 1) / p.block_q;
          },
          sTile, lane);
      if (lane == 0) sNT = n;
    }
    __syncthreads();
    n_qt = sNT;
  }
  auto tile_row = [&](int i) { return BLOCK ? (int)sTile[i] * BT : qb0 + i * BT; };
  const int n_steps = G * n_qt;

  const int dma_row0 = wave * NIW * RPI + lane / CH;
  const int dma_slot = lane % CH;
  uint32_t qo[NIW], go[NIW];
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int r = dma_row0 + j * RPI;
    qo[j] = (uint32_t)(r * p.q_ss + bswz<D>(r, dma_slot) * 8) * 2u;
    go[j] = (uint32_t)(r * p.do_ss + bswz<D>(r, dma_slot) * 8) * 2u;
  }
  const int64_t nstat = (int64_t)p.B * p.Hq * p.npad;
  const DmaRsrc rst = dma_rsrc(p.stats, (uint32_t)(2 * nstat * 4));
  auto issue = [&](int g, int r0, int buf) {
    const int hq = hkv * G + g;
    const int nvalid = min(BT, p.Nq - r0);
    const __bf16* qb = (const __bf16*)p.q + b * p.q_sb + (int64_t)r0 * p.q_ss + hq * p.q_sh;
    const __bf16* gb = (const __bf16*)p.dout + b * p.do_sb + (int64_t)r0 * p.do_ss + hq * p.do_sh;
    const DmaRsrc rq = dma_rsrc(qb, span<D>(nvalid, p.q_ss));
    const DmaRsrc rg = dma_rsrc(gb, span<D>(nvalid, p.do_ss));
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int lds_row = (wave * NIW + j) * RPI;
      buf_load_lds16(rq, sQ[buf] + lds_row * D, qo[j]);
      buf_load_lds16(rg, sG[buf] + lds_row * D, go[j]);
    }
    if (wave == 0 && lane < 32) {
      const int64_t srow = ((int64_t)b * p.Hq + hq) * p.npad + r0;
      const uint32_t off = (uint32_t)((srow + (lane >= 16 ? nstat : 0)) * 4 + 16 * (lane & 15));
      buf_load_lds16(rst, sSt[buf], off);
    }
  };

  f32x16 acc[MB];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  const float c = p.scale_log2;
  const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_ch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_half = 4 * (lane & 1);
  const int key_blk = (BLOCK && key_ok) ? key / p.block_k : 0;

  // per 32-query block of the tile at row r0: 0 no pair visible, 1 all
  // visible, 2 apply the masks element by element (the same for both waves)
  auto states = [&](int r0, int* state) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qs = r0 + 32 * qb;
      state[qb] = 1;
      if (qs >= p.Nq || k0w >= p.Nk) state[qb] = 0;
      else if (CAUSAL) {
        if (qs + 31 + p.causal_off < k0w) state[qb] = 0;
        else if (qs + p.causal_off < k0w + 31) state[qb] = 2;
      }
      if (BLOCK && state[qb] != 0) {
        const int bs = block_state(p, qs, min(qs + 31, p.Nq - 1), k0w, min(k0w + 31, p.Nk - 1));
        state[qb] = bs == 0 ? 0 : (bs == 2 ? 2 : state[qb]);
      }
    }
  };

  // P wave, a tile with a masked or empty block: block by block
  auto p_general = [&](int r0, const int* state, const __bf16* sq, const __bf16* sg, const float* ss,
                       bf16x8* pdst) {
    f32x16 s[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (state[qb] == 0) continue;
      s[qb] = f32x16{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) s[qb] = mfma32(row_frag<D, SW_B>(sq, qb, t, qc, h), sf[t], s[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (state[qb] == 0) continue;
      const int qs = r0 + 32 * qb;
      const bool masked = state[qb] == 2;
      bool fl0 = false, fl1 = false, fl2 = false;
      int qbb1 = 0, qbb2 = 0;
      if (BLOCK && masked) {
        const int qbk = qs / p.block_q, nqb = p.Nq / p.block_q;
        qbb1 = (qbk + 1) * p.block_q;
        qbb2 = (qbk + 2) * p.block_q;
        const uint8_t* col = p.block_mask + key_blk;
        if (key_ok) {
          fl0 = col[(int64_t)qbk * p.nkb] != 0;
          fl1 = qbk + 1 < nqb && col[(int64_t)(qbk + 1) * p.nkb] != 0;
          fl2 = qbk + 2 < nqb && col[(int64_t)(qbk + 2) * p.nkb] != 0;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 l4 = *(const f32x4*)(ss + 32 * qb + 8 * j + 4 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * j + i;
          float pr = ex2(__builtin_fmaf(s[qb][r], c, -l4[i]));
          if ((CAUSAL || BLOCK) && masked) {
            const int q = qs + 8 * j + 4 * h + i;
            bool ok = true;
            if (CAUSAL) ok = key <= q + p.causal_off;
            if (BLOCK) ok = ok && q < p.Nq && (q >= qbb2 ? fl2 : q >= qbb1 ? fl1 : fl0);
            pr = ok ? pr : 0.f;
          }
          s[qb][r] = pr;
        }
      }
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int o8 = 8 * uu;
        const bf16x8 pf = cvt8(s[qb][o8 + 0], s[qb][o8 + 1], s[qb][o8 + 2], s[qb][o8 + 3],
                               s[qb][o8 + 4], s[qb][o8 + 5], s[qb][o8 + 6], s[qb][o8 + 7]);
        pdst[(qb * 2 + uu) * 64 + lane] = pf;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = mfma32(tr_frag<D, SW_B>(sg, 2 * qb + uu, mb, tr_row, tr_ch, tr_half), pf, acc[mb]);
      }
    }
  };

  // dS wave, a tile with a masked or empty block: block by block
  auto ds_general = [&](const int* state, const __bf16* sq, const __bf16* sg, const float* ss,
                        const bf16x8* psrc) {
    f32x16 dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (state[qb] == 0) continue;
      dp[qb] = f32x16{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) dp[qb] = mfma32(row_frag<D, SW_B>(sg, qb, t, qc, h), sf[t], dp[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (state[qb] == 0) continue;
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const bf16x8 pf = psrc[(qb * 2 + uu) * 64 + lane];
        const f32x4 d0 = *(const f32x4*)(ss + BT + 32 * qb + 16 * uu + 4 * h);
        const f32x4 d1 = *(const f32x4*)(ss + BT + 32 * qb + 16 * uu + 8 + 4 * h);
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float dsum = e < 4 ? d0[e] : d1[e - 4];
          ds[e] = bf2f(pf[e]) * (dp[qb][8 * uu + e] - dsum);
        }
        const bf16x8 df = cvt8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = mfma32(tr_frag<D, SW_B>(sq, 2 * qb + uu, mb, tr_row, tr_ch, tr_half), df, acc[mb]);
      }
    }
  };

  // Both 32-query blocks fully visible: four straight-line stages in a fixed
  // order (sched_barrier between steps), the LDS operands read two products
  // ahead and the elementwise work of one block spread over the other's
  // products. The products reach each accumulator in the block-by-block
  // order, so results are bitwise those of the general path.
  //   P wave:  S(b0) | S(b1), P(b0) | dV(b0), P(b1) | dV(b1)
  //   dS wave: dP(b0) | dP(b1), dS(b0) | dK(b0), dS(b1) | dK(b1)
  auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
  constexpr int LEAD = 2;
  // sc: row operand t of block qb (S or dP); gr: transposed operand i of block
  // qb (step u = 2 qb + i / MB, column block i % MB)
  auto p_fast = [&](const __bf16* sq, const __bf16* sg, const float* ss, bf16x8* pdst)
      __attribute__((always_inline)) {
    auto sc = [&](int qb, int t) __attribute__((always_inline)) { return row_frag<D, SW_B>(sq, qb, t, qc, h); };
    auto gr = [&](int qb, int i) __attribute__((always_inline)) {
      return tr_frag<D, SW_B>(sg, 2 * qb + i / MB, i % MB, tr_row, tr_ch, tr_half);
    };
    f32x4 l4[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int j = 0; j < 4; ++j) l4[qb][j] = *(const f32x4*)(ss + 32 * qb + 8 * j + 4 * h);
    f32x16 sb[2];
    sb[0] = f32x16{};
    sb[1] = f32x16{};
    auto sm = [&](int qb, int j) __attribute__((always_inline)) {
      sb[qb][j] = ex2(__builtin_fmaf(sb[qb][j], c, -l4[qb][j >> 2][j & 3]));
    };
    bf16x8 op[KSTEPS];
#pragma unroll
    for (int i = 0; i < LEAD; ++i) op[i] = sc(0, i);
    fence();
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      sb[0] = mfma32(op[i], sf[i], sb[0]);
      if (i + LEAD < KSTEPS) op[i + LEAD] = sc(0, i + LEAD);
      else op[i + LEAD - KSTEPS] = sc(1, i + LEAD - KSTEPS);
      fence();
    }
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      sb[1] = mfma32(op[i], sf[i], sb[1]);
      if (i + LEAD < KSTEPS) op[i + LEAD] = sc(1, i + LEAD);
      else op[i + LEAD - KSTEPS] = gr(0, i + LEAD - KSTEPS);
      sm(0, 2 * i);
      sm(0, 2 * i + 1);
      fence();
    }
    bf16x8 pf0 = cvt8(sb[0][0], sb[0][1], sb[0][2], sb[0][3], sb[0][4], sb[0][5], sb[0][6], sb[0][7]);
    bf16x8 pf1 = cvt8(sb[0][8], sb[0][9], sb[0][10], sb[0][11], sb[0][12], sb[0][13], sb[0][14], sb[0][15]);
    pdst[0 * 64 + lane] = pf0;
    pdst[1 * 64 + lane] = pf1;
    fence();
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      acc[i % MB] = mfma32(op[i], i < MB ? pf0 : pf1, acc[i % MB]);
      if (i + LEAD < KSTEPS) op[i + LEAD] = gr(0, i + LEAD);
      else op[i + LEAD - KSTEPS] = gr(1, i + LEAD - KSTEPS);
      sm(1, 2 * i);
      sm(1, 2 * i + 1);
      fence();
    }
    pf0 = cvt8(sb[1][0], sb[1][1], sb[1][2], sb[1][3], sb[1][4], sb[1][5], sb[1][6], sb[1][7]);
    pf1 = cvt8(sb[1][8], sb[1][9], sb[1][10], sb[1][11], sb[1][12], sb[1][13], sb[1][14], sb[1][15]);
    pdst[2 * 64 + lane] = pf0;
    pdst[3 * 64 + lane] = pf1;
    fence();
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      acc[i % MB] = mfma32(op[i], i < MB ? pf0 : pf1, acc[i % MB]);
      if (i + LEAD < KSTEPS) op[i + LEAD] = gr(1, i + LEAD);
      fence();
    }
  };
  auto ds_fast = [&](const __bf16* sq, const __bf16* sg, const float* ss, const bf16x8* psrc)
      __attribute__((always_inline)) {
    auto sc = [&](int qb, int t) __attribute__((always_inline)) { return row_frag<D, SW_B>(sg, qb, t, qc, h); };
    auto gr = [&](int qb, int i) __attribute__((always_inline)) {
      return tr_frag<D, SW_B>(sq, 2 * qb + i / MB, i % MB, tr_row, tr_ch, tr_half);
    };
    bf16x8 pv[2][2];
    f32x4 d4[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) pv[qb][uu] = psrc[(qb * 2 + uu) * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) d4[qb][j] = *(const f32x4*)(ss + BT + 32 * qb + 8 * j + 4 * h);
    }
    f32x16 db[2];
    db[0] = f32x16{};
    db[1] = f32x16{};
    auto dss = [&](int qb, int e) __attribute__((always_inline)) {
      db[qb][e] = bf2f(pv[qb][e >> 3][e & 7]) * (db[qb][e] - d4[qb][e >> 2][e & 3]);
    };
    bf16x8 op[KSTEPS];
#pragma unroll
    for (int i = 0; i < LEAD; ++i) op[i] = sc(0, i);
    fence();
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      db[0] = mfma32(op[i], sf[i], db[0]);
      if (i + LEAD < KSTEPS) op[i + LEAD] = sc(0, i + LEAD);
      else op[i + LEAD - KSTEPS] = sc(1, i + LEAD - KSTEPS);
      fence();
    }
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      db[1] = mfma32(op[i], sf[i], db[1]);
      if (i + LEAD < KSTEPS) op[i + LEAD] = sc(1, i + LEAD);
      else op[i + LEAD - KSTEPS] = gr(0, i + LEAD - KSTEPS);
      dss(0, 2 * i);
      dss(0, 2 * i + 1);
      fence();
    }
    bf16x8 df0 = cvt8(db[0][0], db[0][1], db[0][2], db[0][3], db[0][4], db[0][5], db[0][6], db[0][7]);
    bf16x8 df1 = cvt8(db[0][8], db[0][9], db[0][10], db[0][11], db[0][12], db[0][13], db[0][14], db[0][15]);
    fence();
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      acc[i % MB] = mfma32(op[i], i < MB ? df0 : df1, acc[i % MB]);
      if (i + LEAD < KSTEPS) op[i + LEAD] = gr(0, i + LEAD);
      else op[i + LEAD - KSTEPS] = gr(1, i + LEAD - KSTEPS);
      dss(1, 2 * i);
      dss(1, 2 * i + 1);
      fence();
    }
    df0 = cvt8(db[1][0], db[1][1], db[1][2], db[1][3], db[1][4], db[1][5], db[1][6], db[1][7]);
    df1 = cvt8(db[1][8], db[1][9], db[1][10], db[1][11], db[1][12], db[1][13], db[1][14], db[1][15]);
    fence();
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      acc[i % MB] = mfma32(op[i], i < MB ? df0 : df1, acc[i % MB]);
      if (i + LEAD < KSTEPS) op[i + LEAD] = gr(1, i + LEAD);
      fence();
    }
  };

  auto tile_p = [&](int r0, int buf, bf16x8* pdst) {
    int state[2];
    states(r0, state);
    if (state[0] == 1 && state[1] == 1) p_fast(sQ[buf], sG[buf], sSt[buf], pdst);
    else p_general(r0, state, sQ[buf], sG[buf], sSt[buf], pdst);
  };
  auto tile_ds = [&](int r0, int buf, const bf16x8* psrc) {
    int state[2];
    states(r0, state);
    if (state[0] == 1 && state[1] == 1) ds_fast(sQ[buf], sG[buf], sSt[buf], psrc);
    else ds_general(state, sQ[buf], sG[buf], sSt[buf], psrc);
  };

  // step s: query head hkv*G + s / n_qt, tile s % n_qt, tracked as
  // (head, tile index) for steps st - 1, st and st + 1
  if (n_steps > 0) issue(0, tile_row(0), 0);
  wait_all_loads();
  __syncthreads();
  int ba = 0;          // buffer of tile st
  int ic = 0, ip = 0;  // tile index of steps st and st - 1
  int gc = 0;          // query head of step st
  for (int st = 0; st <= n_steps; ++st) {
    const int bn = ba == 2 ? 0 : ba + 1;  // tile st + 1
    const int bp = ba == 0 ? 2 : ba - 1;  // tile st - 1
    int in = ic + 1, gn = gc;
    if (in == n_qt) {
      in = 0;
      ++gn;
    }
    if (st + 1 < n_steps) issue(gn, tile_row(in), bn);
    if (pw) {
      if (st < n_steps) tile_p(tile_row(ic), ba, &sP[st & 1][kw][0][0][0]);
    } else if (st >= 1) {
      tile_ds(tile_row(ip), bp, &sP[(st - 1) & 1][kw][0][0][0]);
    }
    wait_all_loads();
    __syncthreads();  // tile st's P and tile st + 1's Q, dO published; tile st - 1 free
    ba = bn;
    ip = ic;
    ic = in;
    gc = gn;
  }

  // ---- epilogue: dV = acc (P wave), dK = scale * acc (dS wave); lane (c, h)
  // holds dims 32mb + 8jj + 4h .. +3 of key c
  // with masks, an Inf or NaN written here raises the flag (bwd_fix_kernel):
  // x * 0 is 0 for finite x and NaN otherwise
  float nf = 0.f;
  if (key_ok) {
    __bf16* op = pw ? (__bf16*)p.dv + b * p.dv_sb + (int64_t)key * p.dv_ss + hkv * p.dv_sh
                    : (__bf16*)p.dk + b * p.dk_sb + (int64_t)key * p.dk_ss + hkv * p.dk_sh;
    const float sc = pw ? 1.f : p.scale;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = acc[mb];
        if constexpr (CAUSAL || BLOCK)
          for (int i = 0; i < 4; ++i) nf = __builtin_fmaf(a[4 * jj + i], 0.f, nf);
        *(bf16x4*)(op + 32 * mb + 8 * jj + 4 * h) =
            cvt4(a[4 * jj] * sc, a[4 * jj + 1] * sc, a[4 * jj + 2] * sc, a[4 * jj + 3] * sc);
      }
  }
  if constexpr (CAUSAL || BLOCK) raise_flag(p, nf != 0.f);
}

// ---- dQ. Workgroup: 128 query rows of one (batch, query head); wave w holds
// rows 32w .. 32w+31 as B operands (lane (c, h): row c). S^T = K Q^T and
// dP^T = V dO^T come out with lane (c, h) holding query c for the 16 keys
// 8*(r/4) + 4h + r%4 of a 32-key block; dS^T in that layout is the B operand
// of dQ^T += K^T dS^T, whose A operand is a transposed read of the K tile.
template <int D, bool CAUSAL, bool BLOCK>
__global__ void __launch_bounds__(64 * NW, 2) bwd_dq_kernel(const BwdParams p) {
  constexpr int CH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int MB = D / 32;
  constexpr int RPI = 1024 / (D * 2);
  constexpr int NIW = BT / RPI / NW;

  __shared__ __attribute__((aligned(16))) __bf16 sK[2][BT * D];  // vswz (read both ways)
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][BT * D];  // kswz (read as rows)
  __shared__ short sTile[BLOCK ? kMaxBwdTiles : 1];  // live key tiles (block mask)
  __shared__ int sNT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qc = lane & 31;
  const int h = lane >> 5;

  const int n_qt = (p.Nq + 127) / 128;
  const int hq = blockIdx.x % p.Hq;
  const int t2 = blockIdx.x / p.Hq;
  const int b = t2 % p.B;
  const int rank = t2 / p.B;
  const int qt = CAUSAL ? n_qt - 1 - rank : rank;  // causal: longest rows first
  const int hkv = hq / (p.Hq / p.Hkv);
  const int q0 = qt * 128 + 32 * wave;
  const int qrow = q0 + qc;
  const bool row_ok = qrow < p.Nq;
  const int wave_last = min(q0 + 31, p.Nq - 1);
  const int row_blk = (BLOCK && row_ok) ? qrow / p.block_q : 0;  // this lane's mask row

  bf16x8 qf[KSTEPS], gf[KSTEPS];
  {
    const __bf16* qp = (const __bf16*)p.q + b * p.q_sb + (int64_t)qrow * p.q_ss + hq * p.q_sh + 8 * h;
    const __bf16* gp =
        (const __bf16*)p.dout + b * p.do_sb + (int64_t)qrow * p.do_ss + hq * p.do_sh + 8 * h;
    const bf16x8 z = {};
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      qf[t] = row_ok ? *(const bf16x8*)(qp + 16 * t) : z;
      gf[t] = row_ok ? *(const bf16x8*)(gp + 16 * t) : z;
    }
  }
  const int64_t nstat = (int64_t)p.B * p.Hq * p.npad;
  const int64_t srow = ((int64_t)b * p.Hq + hq) * p.npad;
  const float lse2 = row_ok ? p.stats[srow + qrow] : __builtin_inff();
  const float dsum = row_ok ? p.stats[nstat + srow + qrow] : 0.f;

  int kv_end = p.Nk;
  if constexpr (CAUSAL)
    kv_end = min(p.Nk, max(0, min(qt * 128 + 127, p.Nq - 1) + p.causal_off + 1));
  int n_tiles = (kv_end + BT - 1) / BT;
  if constexpr (BLOCK) {
    // key tiles meeting a live block of the workgroup's block rows
    if (wave == 0) {
      const int r_lo = qt * 128, r_hi = min(qt * 128 + 128, p.Nq) - 1;
      const int n = live_tiles<true>(
          p, 0, n_tiles, r_lo / p.block_q, r_hi / p.block_q,
          [&](int t, int& a, int& b) {
            a = t * BT / p.block_k;
            b = (min(t * BT + BT, kv_end) - 1) / p.block_k;
          },
          sTile, lane);
      if (lane == 0) sNT = n;
    }
    __syncthreads();
    n_tiles = sNT;
  }
  auto tile_of = [&](int i) { return BLOCK ? (int)sTile[i] : i; };

  const __bf16* kg = (const __bf16*)p.k + b * p.k_sb + hkv * p.k_sh;
  const __bf16* vg = (const __bf16*)p.v + b * p.v_sb + hkv * p.v_sh;
  const int dma_row0 = wave * NIW * RPI + lane / CH;
  const int dma_slot = lane % CH;
  // byte offsets of this lane's chunk in the tile rows of load j. The K rows'
  // swizzle depends on the row only through r % 4 (d = 128) or bit 1 of r
  // (d = 64), the same for rows RPI apart, so the rows of different j differ
  // by whole rows and only j = 0 is kept (fewer live registers through the
  // tile loop).
  static_assert(RPI % 4 == 0, "K row swizzle period");
  uint32_t ko0, vo[NIW];
  {
    const int r = dma_row0;
    ko0 = (uint32_t)(r * p.k_ss + vswz<D>(r, dma_slot) * 8) * 2u;
  }
  const uint32_t kstep = (uint32_t)(RPI * p.k_ss) * 2u;
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int r = dma_row0 + j * RPI;
    vo[j] = (uint32_t)(r * p.v_ss + kswz<D>(r, dma_slot) * 8) * 2u;
  }
  auto issue = [&](int t, int buf) {
    const int r0 = t * BT;
    const int nvalid = min(BT, kv_end - r0);
    const DmaRsrc rk = dma_rsrc(kg + (int64_t)r0 * p.k_ss, span<D>(nvalid, p.k_ss));
    const DmaRsrc rv = dma_rsrc(vg + (int64_t)r0 * p.v_ss, span<D>(nvalid, p.v_ss));
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int lds_row = (wave * NIW + j) * RPI;
      buf_load_lds16(rk, sK[buf] + lds_row * D, ko0 + j * kstep);
      buf_load_lds16(rv, sV[buf] + lds_row * D, vo[j]);
    }
  };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  // d = 128: byte offsets (within a tile) of the K-row fragments of k-steps
  // 0, 2, 4, 6 (the fixed-order tile below)
  int kofs[4] = {0, 0, 0, 0};
  if constexpr (D == 128) {
#pragma unroll
    for (int m = 0; m < 4; ++m) kofs[m] = (qc * D + vswz<D>(qc, 4 * m + h) * 8) * 2;
  }
  const float c = p.scale_log2;
  const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_ch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_half = 4 * (lane & 1);

  // A fully visible tile at d = 128 as four straight-line stages in a fixed
  // order (sched_barrier between steps; LDS operands two products ahead; at
  // d = 64 the compiler's own order measured faster):
  //   A. S^T and dP^T of key block 0
  //   B. the same for key block 1, with block 0's dS^T elements in between
  //   C. dQ^T products of block 0, with block 1's dS^T elements in between
  //   D. dQ^T products of block 1
  constexpr int NPS = 2 * KSTEPS;  // score-stage products
  constexpr int NPG = 2 * MB;      // gradient-stage products
  constexpr int LEAD = 2;
  constexpr int SPG = (17 + NPG - 1) / NPG;  // softmax steps per gradient product
  auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
  auto fast = [&](const __bf16* sk, const __bf16* sv) __attribute__((always_inline)) {
    auto sc_op = [&](int kb, int i) __attribute__((always_inline)) {
      if (i & 1) return row_frag<D, SW_K>(sv, kb, i >> 1, qc, h);
      // K rows (vswz, d = 128): chunk 2ks + h of row 32 kb + qc sits at the
      // slot of chunk 4 (ks / 2) + h plus 2 for odd ks, 32 rows further per
      // block: four lane offsets and immediates
      const int ks = i >> 1;
      return *(const bf16x8*)((const char*)sk + kofs[ks >> 1] + 32 * (ks & 1) + kb * (64 * D));
    };
    // gradient product i of block kb: step u = 2 kb + i / MB, column block i % MB
    auto gr_op = [&](int kb, int i) __attribute__((always_inline)) {
      return tr_frag<D, SW_V>(sk, 2 * kb + i / MB, i % MB, tr_row, tr_ch, tr_half);
    };
    f32x16 sb[2], db[2];
    auto sm_step = [&](int kb, int j) __attribute__((always_inline)) {
      if (j < 16) sb[kb][j] = ex2(__builtin_fmaf(sb[kb][j], c, -lse2));
      if (j >= 1 && j <= 16) db[kb][j - 1] = sb[kb][j - 1] * (db[kb][j - 1] - dsum);
    };
    bf16x8 op[NPS];
#pragma unroll
    for (int i = 0; i < LEAD; ++i) op[i] = sc_op(0, i);
    sb[0] = f32x16{};
    db[0] = f32x16{};
    sb[1] = f32x16{};
    db[1] = f32x16{};
    fence();
    // A
#pragma unroll
    for (int i = 0; i < NPS; ++i) {
      if (i & 1) db[0] = mfma32(op[i], gf[i >> 1], db[0]);
      else sb[0] = mfma32(op[i], qf[i >> 1], sb[0]);
      if (i + LEAD < NPS) op[i + LEAD] = sc_op(0, i + LEAD);
      else op[i + LEAD - NPS] = sc_op(1, i + LEAD - NPS);
      fence();
    }
    // B
#pragma unroll
    for (int i = 0; i < NPS; ++i) {
      if (i & 1) db[1] = mfma32(op[i], gf[i >> 1], db[1]);
      else sb[1] = mfma32(op[i], qf[i >> 1], sb[1]);
      if (i + LEAD < NPS) op[i + LEAD] = sc_op(1, i + LEAD);
      else op[i + LEAD - NPS] = gr_op(0, i + LEAD - NPS);
#pragma unroll
      for (int k = 0; k < 16 / NPS; ++k) sm_step(0, i * (16 / NPS) + k);
      fence();
    }
    sm_step(0, 16);
    bf16x8 df = cvt8(db[0][0], db[0][1], db[0][2], db[0][3], db[0][4], db[0][5], db[0][6], db[0][7]);
    fence();
    // C
#pragma unroll
    for (int i = 0; i < NPG; ++i) {
      if (i == MB)
        df = cvt8(db[0][8], db[0][9], db[0][10], db[0][11], db[0][12], db[0][13], db[0][14], db[0][15]);
      acc[i % MB] = mfma32(op[i], df, acc[i % MB]);
      if (i + LEAD < NPG) op[i + LEAD] = gr_op(0, i + LEAD);
      else op[i + LEAD - NPG] = gr_op(1, i + LEAD - NPG);
#pragma unroll
      for (int k = 0; k < SPG; ++k)
        if (i * SPG + k <= 16) sm_step(1, i * SPG + k);
      fence();
    }
#pragma unroll
    for (int j = NPG * SPG; j <= 16; ++j) sm_step(1, j);
    df = cvt8(db[1][0], db[1][1], db[1][2], db[1][3], db[1][4], db[1][5], db[1][6], db[1][7]);
    fence();
    // D
#pragma unroll
    for (int i = 0; i < NPG; ++i) {
      if (i == MB)
        df = cvt8(db[1][8], db[1][9], db[1][10], db[1][11], db[1][12], db[1][13], db[1][14], db[1][15]);
      acc[i % MB] = mfma32(op[i], df, acc[i % MB]);
      if (i + LEAD < NPG) op[i + LEAD] = gr_op(1, i + LEAD);
      fence();
    }
  };

  auto body = [&](int t, int buf) {
    const int k0 = t * BT;
    int state = 1;  // 0: nothing visible, 1: all visible, 2: apply the rules
    if (q0 >= p.Nq) state = 0;
    else {
      if (CAUSAL) {
        if (k0 > wave_last + p.causal_off) state = 0;
        else if (k0 + BT - 1 > q0 + p.causal_off) state = 2;
      }
      if (state == 1 && k0 + BT > p.Nk) state = 2;
      if (BLOCK && state != 0) {
        const int bs = block_state(p, q0, wave_last, k0, min(k0 + BT - 1, p.Nk - 1));
        state = bs == 0 ? 0 : (bs == 2 ? 2 : state);
      }
    }
    if (state == 0) return;
    const __bf16* sk = sK[buf];
    const __bf16* sv = sV[buf];
    if (D == 128 && state == 1) {
      fast(sk, sv);
      return;
    }
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        s[kb] = mfma32(row_frag<D, SW_V>(sk, kb, ks, qc, h), qf[ks], s[kb]);
        dp[kb] = mfma32(row_frag<D, SW_K>(sv, kb, ks, qc, h), gf[ks], dp[kb]);
      }
    }
    // block mask, mixed region: the tile's 64 keys span at most five key
    // blocks; their flags for this lane's row block are read once, and each
    // key picks one by comparing with the key-block boundaries
    bool fl[5] = {false, false, false, false, false};
    int kb0 = 0;
    if (BLOCK && state == 2) {
      kb0 = k0 / p.block_k;
      const uint8_t* rowm = p.block_mask + (int64_t)row_blk * p.nkb;
#pragma unroll
      for (int x = 0; x < 5; ++x) fl[x] = row_ok && kb0 + x < p.nkb && rowm[kb0 + x] != 0;
    }
    // dS^T = P^T (dP^T - D) in place of dP^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = ex2(__builtin_fmaf(s[kb][r], c, -lse2));
        if (state == 2) {
          const int kk = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          bool ok = kk < p.Nk;
          if (CAUSAL) ok = ok && kk <= qrow + p.causal_off;
          if (BLOCK) {
            const int x = (kk >= (kb0 + 1) * p.block_k) + (kk >= (kb0 + 2) * p.block_k) +
                          (kk >= (kb0 + 3) * p.block_k) + (kk >= (kb0 + 4) * p.block_k);
            ok = ok && (x == 0 ? fl[0] : x == 1 ? fl[1] : x == 2 ? fl[2] : x == 3 ? fl[3] : fl[4]);
          }
          pr = ok ? pr : 0.f;
        }
        dp[kb][r] = pr * (dp[kb][r] - dsum);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x16& sb = dp[u >> 1];
      const int o8 = 8 * (u & 1);
      const bf16x8 df = cvt8(sb[o8 + 0], sb[o8 + 1], sb[o8 + 2], sb[o8 + 3], sb[o8 + 4], sb[o8 + 5],
                             sb[o8 + 6], sb[o8 + 7]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = mfma32(tr_frag<D, SW_V>(sk, u, mb, tr_row, tr_ch, tr_half), df, acc[mb]);
    }
  };

  if (n_tiles > 0) issue(tile_of(0), 0);
  wait_all_loads();
  __syncthreads();
  for (int i = 0; i < n_tiles; ++i) {
    const int buf = i & 1;
    if (i + 1 < n_tiles) issue(tile_of(i + 1), buf ^ 1);
    body(tile_of(i), buf);
    wait_all_loads();
    __syncthreads();
  }

  // with masks, an Inf or NaN written here raises the flag (bwd_fix_kernel):
  // x * 0 is 0 for finite x and NaN otherwise
  float nf = 0.f;
  if (row_ok) {
    __bf16* op = (__bf16*)p.dq + b * p.dq_sb + (int64_t)qrow * p.dq_ss + hq * p.dq_sh;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = acc[mb];
        if constexpr (CAUSAL || BLOCK)
          for (int e = 0; e < 4; ++e) nf = __builtin_fmaf(a[4 * jj + e], 0.f, nf);
        *(bf16x4*)(op + 32 * mb + 8 * jj + 4 * h) =
            cvt4(a[4 * jj] * p.scale, a[4 * jj + 1] * p.scale, a[4 * jj + 2] * p.scale,
                 a[4 * jj + 3] * p.scale);
      }
  }
  if constexpr (CAUSAL || BLOCK) raise_flag(p, nf != 0.f);
}

// ---- After the main kernels, with masks only: nothing unless a wave raised
// the flag; then every gradient row holding an Inf or NaN is recomputed
// exactly (one wave per row, rows strided over the grid: the keys' dK and dV
// rows first, then the query rows' dQ).
template <int D, bool CAUSAL, bool BLOCK>
__global__ void __launch_bounds__(256) bwd_fix_kernel(const BwdParams p) {
  if (*(const volatile int*)p.flag == 0) return;
  const int64_t nkeys = (int64_t)p.B * p.Hkv * p.Nk;
  const int64_t total = nkeys + (int64_t)p.B * p.Hq * p.Nq;
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x / 64);
  for (int64_t r = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64; r < total; r += stride) {
    if (r < nkeys) {
      const int key = (int)(r % p.Nk);
      const int bh = (int)(r / p.Nk);
      const int b = bh / p.Hkv, hkv = bh % p.Hkv;
      const __bf16* dkr = (const __bf16*)p.dk + b * p.dk_sb + (int64_t)key * p.dk_ss + hkv * p.dk_sh;
      const __bf16* dvr = (const __bf16*)p.dv + b * p.dv_sb + (int64_t)key * p.dv_ss + hkv * p.dv_sh;
      const bool bad_k = row_nonfinite<D>(dkr), bad_v = row_nonfinite<D>(dvr);
      if (bad_k || bad_v) exact_key_row<D, CAUSAL, BLOCK>(p, b, hkv, key);
    } else {
      const int64_t rq = r - nkeys;
      const int q = (int)(rq % p.Nq);
      const int bh = (int)(rq / p.Nq);
      const int b = bh / p.Hq, hq = bh % p.Hq;
      const __bf16* dqr = (const __bf16*)p.dq + b * p.dq_sb + (int64_t)q * p.dq_ss + hq * p.dq_sh;
      if (row_nonfinite<D>(dqr)) exact_q_row<D, CAUSAL, BLOCK>(p, b, hq, q);
    }
  }
}

template <int D, bool CAUSAL, bool BLOCK>
hipError_t launch(const BwdParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.Hq * p.npad;
  if (rows > 0) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       s, p);
  }
  const int64_t nkw = (int64_t)((p.Nk + 127) / 128) * p.B * p.Hkv;
  if (nkw > 0) {
    if constexpr (D == 128)
      hipLaunchKernelGGL((bwd_dkdv_split_kernel<CAUSAL, BLOCK>), dim3((unsigned)nkw), dim3(64 * NWS), 0,
                         s, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, BLOCK>), dim3((unsigned)nkw), dim3(64 * NW), 0, s, p);
  }
  const int64_t nqw = (int64_t)((p.Nq + 127) / 128) * p.B * p.Hq;
  if (nqw > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, BLOCK>), dim3((unsigned)nqw), dim3(64 * NW), 0, s, p);
  // the flag lives in the workspace, which exists when there are query rows
  if ((CAUSAL || BLOCK) && rows > 0)
    hipLaunchKernelGGL((bwd_fix_kernel<D, CAUSAL, BLOCK>), dim3(256), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

template <int D>
hipError_t launch_d(const BwdParams& p, bool causal, bool block, hipStream_t s) {
  if (block) return causal ? launch<D, true, true>(p, s) : launch<D, false, true>(p, s);
  return causal ? launch<D, true, false>(p, s) : launch<D, false, false>(p, s);
}

hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, bool block, hipStream_t s) {
  return d == 64 ? launch_d<64>(p, causal, block, s) : launch_d<128>(p, causal, block, s);
}

}  // namespace miattn
