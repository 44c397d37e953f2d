// Key statistics for the fixed-max softmax ("TPU attention 최적화 실전 가이드",
// 4단계): the largest key norm max_j |k_j| per (batch, KV head), or, for the
// centred bound, the mean key kbar and max_j |k_j - kbar|.
//
// The keys of each (batch, KV head) are split into nsplit ranges; workgroup
// (split, bh) reduces its range to one partial maximum of a squared norm,
// which the attention kernel folds on load (no atomics, deterministic).
// The centred form needs kbar first, so it runs two passes: pass 1 writes
// per-range partial sums of k; pass 2 rebuilds kbar from them (range 0 also
// stores it) and reduces max |k_j - kbar|^2. Each pass reads K once.

#include "common.hpp"
#include "internal.hpp"

namespace miattn {

namespace {

constexpr int NT = 256;

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return (float)(*p); }

// mode 0: max |k|^2; mode 1: partial sums of k; mode 2: max |k - kbar|^2
template <int D, typename T, int MODE>
__global__ void __launch_bounds__(NT) kstats_kernel(const KStatParams p) {
  constexpr int TPR = D / 8 > 16 ? 16 : D / 8;  // threads per key row
  constexpr int EPT = D / TPR;                   // elements per thread
  constexpr int RPP = NT / TPR;                  // rows per pass
  __shared__ float red[NT];
  __shared__ float sbar[D];
  __shared__ float ssum[RPP][D];

  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.Hkv, hkv = bh - b * p.Hkv;
  const int k0 = split * p.keys_per_split;
  const int k1 = min(p.Nk, k0 + p.keys_per_split);
  const T* kg = (const T*)p.k + b * p.k_sb + hkv * p.k_sh;
  const int tr = threadIdx.x / TPR, te = threadIdx.x - tr * TPR;

  if (MODE == 2) {
    // kbar from all ranges' partial sums
    for (int d = threadIdx.x; d < D; d += NT) {
      float s = 0.f;
      for (int i = 0; i < p.nsplit; ++i) s += p.part_sum[((int64_t)bh * kMaxSplit + i) * D + d];
      const float m = p.Nk > 0 ? s / (float)p.Nk : 0.f;
      sbar[d] = m;
      if (split == 0) p.kbar[(int64_t)bh * D + d] = m;
    }
    __syncthreads();
  }

  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
  float best = 0.f;
  for (int key = k0 + tr; key < k1; key += RPP) {
    const T* kp = kg + (int64_t)key * p.k_ss + te * EPT;
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      float x = ld(kp + e);
      if (MODE == 1) acc[e] += x;
      if (MODE == 2) x -= sbar[te * EPT + e];
      sq += x * x;
    }
    if (MODE != 1) {
#pragma unroll
      for (int m = 1; m < TPR; m <<= 1) sq += __shfl_xor(sq, m, 64);
      best = fmaxf(best, sq);
    }
  }

  if (MODE == 1) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) ssum[tr][te * EPT + e] = acc[e];
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += NT) {
      float s = 0.f;
      for (int r = 0; r < RPP; ++r) s += ssum[r][d];
      p.part_sum[((int64_t)bh * kMaxSplit + split) * D + d] = s;
    }
  } else {
    red[threadIdx.x] = best;
    __syncthreads();
    for (int w = NT / 2; w > 0; w >>= 1) {
      if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
      __syncthreads();
    }
    if (threadIdx.x == 0) p.part_max[(int64_t)bh * kMaxSplit + split] = red[0];
  }
}

template <int D, typename T>
hipError_t run(const KStatParams& p, bool centred, hipStream_t s) {
  const dim3 grid(p.nsplit, p.B * p.Hkv);
  if (!centred) {
    hipLaunchKernelGGL((kstats_kernel<D, T, 0>), grid, dim3(NT), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((kstats_kernel<D, T, 1>), grid, dim3(NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((kstats_kernel<D, T, 2>), grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kstats(const KStatParams& p, int d, bool bf16, bool centred, hipStream_t s) {
  if (p.B == 0 || p.nsplit == 0) return hipSuccess;
  if (bf16) return d == 64 ? run<64, __bf16>(p, centred, s) : run<128, __bf16>(p, centred, s);
  return d == 64 ? run<64, float>(p, centred, s) : run<128, float>(p, centred, s);
}

}  // namespace miattn
