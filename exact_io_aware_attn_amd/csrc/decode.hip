// Decode attention: one new query token per sequence against a KV cache,
// split over the cache ("split-K") and merged with the block rule.
//
// Decode reads every cached key and value once per generated token and does
// O(1) FLOPs per byte, so it is bound by HBM bandwidth ("Attention Mechanism
// Optimization for Efficient LLM Inference", "Why Decode is Memory-bound").
// The design therefore aims at bytes in flight, not at arithmetic:
//  * a workgroup owns (batch b, KV head, chunk of `chunk` keys) and serves all
//    G = Hq/Hkv query heads of that KV head, so each cache byte is read once;
//  * each wave streams 32-key slices: K goes from global memory straight into
//    MFMA A-operand registers (16-byte loads), V is staged through a
//    double-buffered per-wave LDS region and read back transposed
//    (ds_read_b64_tr_b16) for O^T = V^T P^T; the next slice's loads are
//    issued before the current slice is consumed;
//  * S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_16x16x32_bf16 with the G
//    query heads as the 16-wide N dimension (zero-padded);
//  * rows at or past seqlens[b] are never read; the last slice masks them;
//  * the four waves' running (m, l, O) are combined through LDS and the chunk
//    writes its normalised O_c and LSE_c; a second kernel merges the chunks
//    with weights exp(LSE_c - LSE) ("플래시어텐션: 메모리를 아끼는 정확한 어텐션",
//    §2 타일링: rescale each block by exp(m_block - m_total) and add).

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace miattn {

namespace {

constexpr int NW = 4;      // waves per workgroup
constexpr int SL = 32;     // keys per wave slice

template <int D>
__global__ void __launch_bounds__(NW * 64, 2) decode_chunk_kernel(const DecodeParams p) {
  constexpr int KST = D / 32;  // k-steps (32 d each) of S^T
  constexpr int MB = D / 16;   // 16-row blocks of O^T
  constexpr int VCH = D / 8;   // 16-byte chunks per row
  // per-wave double-buffered V slice, row-major [SL][D] bf16, 16-byte chunks
  // swizzled so the transpose reads of 4 rows x 2 chunks hit distinct banks.
  // After the key loop the same bytes hold the waves' O^T for the combine.
  constexpr int kVBytes = NW * 2 * SL * D * 2;
  static_assert(kVBytes >= NW * D * 17 * 4, "combine buffer must fit");
  __shared__ __attribute__((aligned(16))) char smem[kVBytes];
  __shared__ float sM[NW][16], sL[NW][16];
  __bf16* const sVbase = (__bf16*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;    // query head (column) of this lane
  const int g4 = lane >> 4;   // lane group

  const int b = blockIdx.z, hkv = blockIdx.y, chunk = blockIdx.x;
  const int len = p.seqlens[b];
  const int k_begin = chunk * p.chunk;
  if (k_begin >= len) return;  // whole workgroup exits together
  const int k_end = min(len, k_begin + p.chunk);
  const int G = p.Hq / p.Hkv;

  const __bf16* __restrict__ kg = (const __bf16*)p.kc + b * p.k_sb + hkv * p.k_sh;
  const __bf16* __restrict__ vg = (const __bf16*)p.vc + b * p.v_sb + hkv * p.v_sh;

  // Q^T as B operand: lane (n, g4), k-step t holds q[head n][32t + 8g4 .. +8]
  bf16x8 qf[KST];
  {
    const bool ok = n < G;
    const __bf16* qp = (const __bf16*)p.q + ((int64_t)b * p.Hq + hkv * G + (ok ? n : 0)) * D + 8 * g4;
#pragma unroll
    for (int t = 0; t < KST; ++t) {
      bf16x8 z = {};
      qf[t] = ok ? *(const bf16x8*)(qp + 32 * t) : z;
    }
  }

  // slices of this chunk, dealt round-robin to the waves; every wave runs the
  // same number of iterations so the workgroup barriers match
  const int n_keys = k_end - k_begin;
  const int n_slices = (n_keys + SL - 1) / SL;
  const int n_iter = (n_slices + NW - 1) / NW;

  // K A-operand registers: slice row 16*mb2 + (lane&15), d 8*g4 + 32t
  bf16x8 kreg[2][2][KST];
  // V rows staged by this lane: row (lane >> 1) of the slice, chunks
  // (lane & 1) * VCH/2 .. +VCH/2 (VCH/2 16-byte loads)
  u32x4 vreg[2][VCH / 2];
  const int vrow = lane >> 1;
  const int vch0 = (lane & 1) * (VCH / 2);

  auto load_set = [&](int it, auto setc) {
    constexpr int set = decltype(setc)::value;
    const int sl = it * NW + wave;
    const int s0 = k_begin + sl * SL;
#pragma unroll
    for (int mb2 = 0; mb2 < 2; ++mb2) {
      const int key = s0 + 16 * mb2 + (lane & 15);
      const bool ok = sl < n_slices && key < k_end;
      const __bf16* kp = kg + (int64_t)key * p.k_ss + 8 * g4;
#pragma unroll
      for (int t = 0; t < KST; ++t) {
        bf16x8 z = {};
        kreg[set][mb2][t] = ok ? *(const bf16x8*)(kp + 32 * t) : z;
      }
    }
    {
      const int key = s0 + vrow;
      const bool ok = sl < n_slices && key < k_end;
      const __bf16* vp = vg + (int64_t)key * p.v_ss + vch0 * 8;
#pragma unroll
      for (int i = 0; i < VCH / 2; ++i) {
        u32x4 z = {0u, 0u, 0u, 0u};
        vreg[set][i] = ok ? *(const u32x4*)(vp + 8 * i) : z;
      }
    }
  };
  auto load = [&](int it, int set) {
    if (set == 0) load_set(it, std::integral_constant<int, 0>());
    else load_set(it, std::integral_constant<int, 1>());
  };
  auto vsw = [](int r, int ch) { return ch ^ ((r & 3) << 1); };

  f32x4 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // transpose-read addressing (see common.hpp): source lane s supplies
  // row 4*(s>>4) + ((s&15)>>2) (+16 for the second read), d 16mb + 4*(s&3)
  const int tr_row = 4 * g4 + ((lane & 15) >> 2);
  const int tr_d = 4 * (lane & 3);

  // one slice: stage V, prefetch the next slice into the other register
  // set, then S^T, softmax update and O^T += V^T P^T. SET is a compile-time
  // constant so the register sets stay in registers.
  auto step = [&](int it, auto setc) {
    constexpr int SET = decltype(setc)::value;
    const int sl = it * NW + wave;
    __bf16* sv = sVbase + (wave * 2 + SET) * SL * D;
#pragma unroll
    for (int i = 0; i < VCH / 2; ++i)
      *(u32x4*)(sv + vrow * D + vsw(vrow, vch0 + i) * 8) = vreg[SET][i];
    if (it + 1 < n_iter) load(it + 1, 1 - SET);
    __syncthreads();

    if (sl < n_slices) {
      const int s0 = k_begin + sl * SL;
      // S^T (keys x heads) for the two 16-key halves
      f32x4 s[2];
#pragma unroll
      for (int mb2 = 0; mb2 < 2; ++mb2) {
        s[mb2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KST; ++t) s[mb2] = mfma16k32(kreg[SET][mb2][t], qf[t], s[mb2]);
      }
      // lane (n, g4), register r of half mb2: key s0 + 16mb2 + 4g4 + r, head n
      float mx = kNegInf;
#pragma unroll
      for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = s0 + 16 * mb2 + 4 * g4 + r;
          float x = s[mb2][r] * p.scale_log2;
          if (key >= k_end) x = kNegInf;
          s[mb2][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = ex2(m_run - m_use);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
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
        const s16x4 lo = lds_tr16(sv + tr_row * D + vsw(tr_row, dd >> 3) * 8 + (dd & 7));
        const s16x4 hi = lds_tr16(sv + (16 + tr_row) * D + vsw(16 + tr_row, dd >> 3) * 8 + (dd & 7));
        const s16x8 a16 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[mb] = mfma16k32(__builtin_bit_cast(bf16x8, a16), pf, oacc[mb]);
      }
    }
    __syncthreads();
  };

  if (n_iter > 0) load(0, 0);
  for (int it = 0; it < n_iter; it += 2) {
    step(it, std::integral_constant<int, 0>());
    if (it + 1 < n_iter) step(it + 1, std::integral_constant<int, 1>());
  }

  // ---- combine the four waves: per head n, M = max m_w, weights 2^(m_w - M)
  float l_w = l_run;
  l_w += shfl_xor(l_w, 16);
  l_w += shfl_xor(l_w, 32);
  if (g4 == 0) {
    sM[wave][n] = m_run;
    sL[wave][n] = l_w;
  }
  float* const sO = (float*)smem;  // [NW][D][17]; the key loop ended on a barrier
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) sO[(wave * D + 16 * mb + 4 * g4 + r) * 17 + n] = oacc[mb][r];
  __syncthreads();

  // threads -> (head, d) pairs of the real heads
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int hn = idx / D, dd = idx - hn * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sM[w][hn]);
    const float Mu = M == kNegInf ? 0.f : M;
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = ex2(sM[w][hn] - Mu);
      L += wt * sL[w][hn];
      acc += wt * sO[(w * D + dd) * 17 + hn];
    }
    const int64_t row = ((int64_t)b * p.Hq + hkv * G + hn) * p.n_chunks + chunk;
    p.part_o[row * D + dd] = L > 0.f ? acc / L : 0.f;
    if (dd == 0) p.part_lse[row] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
  }
}

// One workgroup per (batch, query head): merge the chunks' (O_c, LSE_c).
template <int D>
__global__ void __launch_bounds__(D) decode_merge_kernel(const DecodeParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.Hq;
  const int dd = threadIdx.x;
  const int len = p.seqlens[b];
  const int nc = min(p.n_chunks, (len + p.chunk - 1) / p.chunk);
  const float* lse_c = p.part_lse + (int64_t)bh * p.n_chunks;
  const float* o_c = p.part_o + (int64_t)bh * p.n_chunks * D;
  float M = kNegInf;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, lse_c[c]);
  const float Mu = M == kNegInf ? 0.f : M;
  float W = 0.f, acc = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float w = __expf(lse_c[c] - Mu);
    W += w;
    acc += w * o_c[(int64_t)c * D + dd];
  }
  const float out = W > 0.f ? acc / W : 0.f;
  ((__bf16*)p.o)[(int64_t)bh * D + dd] = (__bf16)out;
  if (p.lse != nullptr && dd == 0) p.lse[bh] = W > 0.f ? Mu + logf(W) : kNegInf;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  const dim3 grid(p.n_chunks, p.Hkv, p.B);
  if (d == 64) {
    hipLaunchKernelGGL(decode_chunk_kernel<64>, grid, dim3(NW * 64), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(p.B * p.Hq), dim3(64), 0, s, p);
  } else {
    hipLaunchKernelGGL(decode_chunk_kernel<128>, grid, dim3(NW * 64), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(p.B * p.Hq), dim3(128), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace miattn
