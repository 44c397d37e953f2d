// Prefill attention in fp32 throughout (no bf16 rounding anywhere).
//
// Same method as the bf16 kernel -- keys streamed in tiles through LDS, a
// running row max and sum per query, the output rescaled when the max grows
// ("Attention Mechanism Optimization for Efficient LLM Inference",
// "Online-Softmax") -- but on the vector ALU: one lane per query row, 64 rows
// per workgroup, K/V tiles of 32 keys in LDS. This is the accuracy path for
// fp32 inputs; it is not the throughput path.
//
// Masked pairs are excluded by selection, not by multiplying with zero, so a
// non-finite value at an excluded position never reaches the output.

#include "common.hpp"
#include "internal.hpp"

namespace miattn {

namespace {

constexpr int BQ = 64;
constexpr int TK = 32;

template <int D, bool CAUSAL, bool BLOCK>
__global__ void __launch_bounds__(BQ) fwd_f32_kernel(const FwdParams p) {
  __shared__ float sK[TK][D];
  __shared__ float sV[TK][D];
  __shared__ __attribute__((aligned(16))) float sQ[BQ][D + 4];  // this lane's query row

  const int qt = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);
  const int lane = threadIdx.x;
  const int qrow = qt * BQ + lane;
  const bool row_ok = qrow < p.Nq;

  float o[D];
  float* q = sQ[lane];
  {
    const float* qp = (const float*)p.q + b * p.q_sb + (int64_t)(row_ok ? qrow : 0) * p.q_ss + hq * p.q_sh;
#pragma unroll
    for (int d = 0; d < D; d += 4)
      *(float4*)(q + d) = row_ok ? *(const float4*)(qp + d) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;
  }
  const float* kg = (const float*)p.k + b * p.k_sb + hkv * p.k_sh;
  const float* vg = (const float*)p.v + b * p.v_sb + hkv * p.v_sh;

  // fixed-max bound, and eligibility per group of 32 rows (each half-wave),
  // the same rule as the bf16 kernel's
  bool fixed = false;
  float m_fix = 0.f;
  if (p.fixed) {
    float qq = 0.f, qk = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) qq += q[d] * q[d];
    const int64_t bk = (int64_t)b * p.Hkv + hkv;
    float r2 = lane < p.ks.nsplit ? p.ks.part_max[bk * kMaxSplit + lane] : 0.f;
    r2 = wave_max(r2);
    const float rho = sqrtf(r2);
    if (p.fixed == 2)
      for (int d = 0; d < D; ++d) qk += q[d] * p.ks.kbar[bk * D + d];
    const float qn = sqrtf(qq);
    m_fix = p.scale * (qk + qn * rho) * kLog2e;
    float gap = row_ok ? 2.f * p.scale * qn * rho : 0.f;
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) gap = fmaxf(gap, shfl_xor(gap, m));
    fixed = gap <= kTau;
  }

  float m_run = kNegInf, l_run = 0.f;
  const int my_qb = BLOCK ? (row_ok ? qrow : 0) / p.block_q : 0;
  for (int k0 = 0; k0 < p.Nk; k0 += TK) {
    __syncthreads();
    for (int i = lane; i < TK * D / 4; i += BQ) {
      const int r = (i * 4) / D, d = (i * 4) - r * D;
      const int key = k0 + r;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (key < p.Nk) {
        kv = *(const float4*)(kg + (int64_t)key * p.k_ss + d);
        vv = *(const float4*)(vg + (int64_t)key * p.v_ss + d);
      }
      *(float4*)&sK[r][d] = kv;
      *(float4*)&sV[r][d] = vv;
    }
    __syncthreads();

    // block rule per 16-key group (block_k is a multiple of 16)
    bool grp[TK / 16];
#pragma unroll
    for (int gi = 0; gi < TK / 16; ++gi) {
      const int key = k0 + 16 * gi;
      grp[gi] = !BLOCK || (key < p.Nk && p.block_mask[(int64_t)my_qb * p.nkb + key / p.block_k] != 0);
    }
    // excluded pairs carry -inf and are skipped below
    float s[TK];
    float mx = kNegInf;
#pragma unroll 1
    for (int j = 0; j < TK; ++j) {
      const int key = k0 + j;
      bool a = key < p.Nk && row_ok && grp[j / 16];
      if (CAUSAL) a = a && key <= qrow + p.causal_off;
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], sK[j][d], acc);
      s[j] = a ? acc * p.scale_log2 : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    float m_ref;
    if (!fixed) {
      const float m_new = fmaxf(m_run, mx);
      m_ref = m_new == kNegInf ? 0.f : m_new;
      const float alpha = ex2(m_run - m_ref);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
    } else {
      m_ref = m_fix;
    }
#pragma unroll 1
    for (int j = 0; j < TK; ++j) {
      if (s[j] != kNegInf) {
        const float e = ex2(s[j] - m_ref);
        l_run += e;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(e, sV[j][d], o[d]);
      }
    }
  }

  if (row_ok) {
    const bool live = l_run > 0.f;
    const float inv = live ? 1.f / l_run : 0.f;
    float* op = (float*)p.o + b * p.o_sb + (int64_t)qrow * p.o_ss + hq * p.o_sh;
#pragma unroll
    for (int d = 0; d < D; d += 4)
      *(float4*)(op + d) = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
    if (p.lse != nullptr) {
      const float m_ref = fixed ? m_fix : m_run;
      p.lse[((int64_t)b * p.Hq + hq) * p.Nq + qrow] = live ? (m_ref + log2f(l_run)) * kLn2 : kNegInf;
    }
  }
}

template <int D, bool C, bool K>
hipError_t launch_one(const FwdParams& p, hipStream_t s) {
  const dim3 grid((p.Nq + BQ - 1) / BQ, p.B * p.Hq);
  hipLaunchKernelGGL((fwd_f32_kernel<D, C, K>), grid, dim3(BQ), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, bool block, hipStream_t s) {
  if (p.Nq == 0 || p.B == 0) return hipSuccess;
#define MIATTN_DISPATCH(DD)                                  \
  if (causal && block) return launch_one<DD, true, true>(p, s);   \
  if (causal) return launch_one<DD, true, false>(p, s);           \
  if (block) return launch_one<DD, false, true>(p, s);            \
  return launch_one<DD, false, false>(p, s);
  if (d == 64) { MIATTN_DISPATCH(64) }
  MIATTN_DISPATCH(128)
#undef MIATTN_DISPATCH
}

}  // namespace miattn
