// Key statistics for the fixed-max softmax ("TPU attention 최적화 실전 가이드",
// 4단계): the logit bound of a query row comes from the norms of the keys it
// can see (Cauchy-Schwarz), or from their distances to a centre.
//
// The keys of each (batch, KV head) are cut into blocks of kb_size keys (the
// block mask's key block, or 256 keys without one). Workgroup (block, bh)
// writes, for its block:
//  * pmax[j] = max |k_i| over the keys i of the block up to and including j
//    (a prefix max restarting at every block), so pmax at the block's last
//    key is the block's largest norm, and pmax at the last key a causal row
//    sees bounds the part of the block that row sees;
//  * centred mode: the block's mean key rounded to bf16 (the centre c, used
//    as an MFMA operand by the attention kernel) and max |k_i - c| over the
//    block, measured from that rounded centre so the bound stays exact.
// A block's statistics depend on its own keys only, so keys a row cannot see
// never enter its bound. No atomics: the result is deterministic.

#include "common.hpp"
#include "internal.hpp"

namespace miattn {

namespace {

constexpr int NT = 256;
constexpr int CHUNK = 1024;  // keys whose norms are scanned per step

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return (float)(*p); }

template <int D, typename T, bool CENTRED>
__global__ void __launch_bounds__(NT) kstats_kernel(const KStatParams p) {
  constexpr int TPR = D / 8 > 16 ? 16 : D / 8;  // threads per key row
  constexpr int EPT = D / TPR;                   // elements per thread
  constexpr int RPP = NT / TPR;                  // rows per pass
  __shared__ float nrm[CHUNK];
  __shared__ float ssum[CENTRED ? RPP : 1][D];
  __shared__ float sc[D];
  __shared__ float red[NT];
  __shared__ float carry;

  const int kb = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.Hkv, hkv = bh - b * p.Hkv;
  const int k0 = kb * p.kb_size;
  const int k1 = min(p.Nk, k0 + p.kb_size);
  const T* kg = (const T*)p.k + b * p.k_sb + hkv * p.k_sh;
  float* pm = p.pmax + (int64_t)bh * p.Nk;
  const int tr = threadIdx.x / TPR, te = threadIdx.x - tr * TPR;
  if (threadIdx.x == 0) carry = 0.f;

  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
  for (int c0 = k0; c0 < k1; c0 += CHUNK) {
    const int c1 = min(k1, c0 + CHUNK);
    // squared norms of the chunk's keys (TPR lanes per key; all lanes of a
    // key leave the loop together, so the shuffles stay within live lanes)
    for (int key = c0 + tr; key < c1; key += RPP) {
      const T* kp = kg + (int64_t)key * p.k_ss + te * EPT;
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const float x = ld(kp + e);
        if (CENTRED) acc[e] += x;
        sq += x * x;
      }
#pragma unroll
      for (int m = 1; m < TPR; m <<= 1) sq += __shfl_xor(sq, m, 64);
      if (te == 0) nrm[key - c0] = sq;
    }
    __syncthreads();
    // prefix max over the chunk by wave 0: 16 keys per lane, then across lanes
    if (threadIdx.x < 64) {
      const int l = threadIdx.x, n = c1 - c0;
      float v[CHUNK / 64];
      float run = 0.f;
#pragma unroll
      for (int i = 0; i < CHUNK / 64; ++i) {
        const int idx = l * (CHUNK / 64) + i;
        run = fmaxf(run, idx < n ? nrm[idx] : 0.f);
        v[i] = run;
      }
      float tot = run;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(tot, off, 64);
        if (l >= off) tot = fmaxf(tot, o);
      }
      float before = __shfl_up(tot, 1, 64);
      if (l == 0) before = 0.f;
      before = fmaxf(before, carry);
#pragma unroll
      for (int i = 0; i < CHUNK / 64; ++i) {
        const int idx = l * (CHUNK / 64) + i;
        if (idx < n) pm[c0 + idx] = sqrtf(fmaxf(v[i], before));
      }
      const float last = __shfl(tot, 63, 64);
      if (l == 0) carry = fmaxf(carry, last);  // every lane has read carry above
    }
    __syncthreads();
  }

  if constexpr (CENTRED) {
    // the block's mean key, rounded to bf16 (the centre), then max |k - c|
#pragma unroll
    for (int e = 0; e < EPT; ++e) ssum[tr][te * EPT + e] = acc[e];
    __syncthreads();
    const float inv_n = 1.f / (float)max(1, k1 - k0);
    __bf16* cout = p.centre + ((int64_t)bh * p.nkb + kb) * D;
    for (int d = threadIdx.x; d < D; d += NT) {
      float s = 0.f;
      for (int r = 0; r < RPP; ++r) s += ssum[r][d];
      const bf16x2 c2 = cvt2(s * inv_n, 0.f);
      cout[d] = c2[0];
      sc[d] = bf2f(c2[0]);
    }
    __syncthreads();
    float best = 0.f;
    for (int key = k0 + tr; key < k1; key += RPP) {
      const T* kp = kg + (int64_t)key * p.k_ss + te * EPT;
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const float x = ld(kp + e) - sc[te * EPT + e];
        sq += x * x;
      }
#pragma unroll
      for (int m = 1; m < TPR; m <<= 1) sq += __shfl_xor(sq, m, 64);
      best = fmaxf(best, sq);
    }
    red[threadIdx.x] = best;
    __syncthreads();
    for (int w = NT / 2; w > 0; w >>= 1) {
      if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
      __syncthreads();
    }
    if (threadIdx.x == 0) p.radius[(int64_t)bh * p.nkb + kb] = sqrtf(red[0]);
  }
}

template <int D, typename T>
hipError_t run(const KStatParams& p, bool centred, hipStream_t s) {
  const dim3 grid(p.nkb, p.B * p.Hkv);
  if (centred) hipLaunchKernelGGL((kstats_kernel<D, T, true>), grid, dim3(NT), 0, s, p);
  else hipLaunchKernelGGL((kstats_kernel<D, T, false>), grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kstats(const KStatParams& p, int d, bool bf16, bool centred, hipStream_t s) {
  if (p.B == 0 || p.Hkv == 0 || p.nkb == 0) return hipSuccess;
  if (bf16) return d == 64 ? run<64, __bf16>(p, centred, s) : run<128, __bf16>(p, centred, s);
  return d == 64 ? run<64, float>(p, centred, s) : run<128, float>(p, centred, s);
}

}  // namespace miattn
