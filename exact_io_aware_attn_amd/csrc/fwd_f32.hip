// Prefill attention in fp32 throughout (no bf16 rounding anywhere).
//
// Same method as the bf16 kernel -- keys streamed in tiles through LDS, a
// running row max and sum per query, the output rescaled when the max grows
// ("Attention Mechanism Optimization for Efficient LLM Inference",
// "Online-Softmax") -- but on the vector ALU: 16 lanes per query row, each
// holding a 1/16 slice of d for q and O (a score is a partial dot product
// summed over the row's lanes), 16 rows per workgroup of 4 waves, K/V tiles
// of 32 keys in LDS. This is the accuracy path for fp32 inputs; it is not
// the throughput path.
//
// Masked pairs are excluded by selection, not by multiplying with zero, so a
// non-finite value at an excluded position never reaches the output.

#include "common.hpp"
#include "internal.hpp"

namespace miattn {

namespace {

constexpr int LPR = 16;           // lanes per query row (each holds D / 16 of d)
constexpr int RPW = 64 / LPR;     // query rows per wave
constexpr int NWF = 4;            // waves per workgroup
constexpr int BQ = RPW * NWF;     // query rows per workgroup
constexpr int TK = 32;            // keys per LDS tile

// sum over the LPR lanes of one query row (lane ids differ in the low bits)
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

template <int D, bool CAUSAL, bool BLOCK>
__global__ void __launch_bounds__(64 * NWF) fwd_f32_kernel(const FwdParams p) {
  constexpr int DL = D / LPR;  // elements of d per lane
  __shared__ __attribute__((aligned(16))) float sK[TK][D];
  __shared__ __attribute__((aligned(16))) float sV[TK][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int d0 = (tid % LPR) * DL;  // this lane's slice of d
  const int qt = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / p.Hq, hq = bh - b * p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);
  const int qrow = qt * BQ + tid / LPR;
  const bool row_ok = qrow < p.Nq;

  float q[DL], o[DL];
  {
    const float* qp = (const float*)p.q + b * p.q_sb + (int64_t)(row_ok ? qrow : 0) * p.q_ss +
                      hq * p.q_sh + d0;
#pragma unroll
    for (int i = 0; i < DL; i += 4) {
      const float4 x = row_ok ? *(const float4*)(qp + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      q[i] = x.x;
      q[i + 1] = x.y;
      q[i + 2] = x.z;
      q[i + 3] = x.w;
    }
#pragma unroll
    for (int i = 0; i < DL; ++i) o[i] = 0.f;
  }
  const float* kg = (const float*)p.k + b * p.k_sb + hkv * p.k_sh;
  const float* vg = (const float*)p.v + b * p.v_sb + hkv * p.v_sh;

  // fixed-max bound of the row and its eligibility, the same rule as the bf16
  // kernel's: over the key blocks the row sees (whole blocks: |q| max|k|, or
  // q.c +- |q| R around the block centre; a block cut by the causal rule: |q|
  // times the prefix max of |k| up to the row's last key), eligible iff the
  // gap between the bound and the lower bound of the row max is <= kTau and
  // the row sees at least kMinFixedKeys keys
  bool fixed = false;
  float m_fix = 0.f;
  if (p.fixed) {
    float qq = 0.f;
#pragma unroll
    for (int i = 0; i < DL; ++i) qq += q[i] * q[i];
    const float qn = sqrtf(row_sum(qq));
    const int64_t bk = (int64_t)b * p.Hkv + hkv;
    const int KB = p.ks.kb_size, nkb = p.ks.nkb;
    const int vis_end = CAUSAL ? min(qrow + p.causal_off, p.Nk - 1) : p.Nk - 1;
    const int qb = BLOCK ? (row_ok ? qrow : 0) / p.block_q : 0;
    const float* pm = p.ks.pmax + bk * p.Nk;
    float up = kNegInf, lo = kNegInf;
    int cnt = 0;
    for (int kb = 0; kb < nkb; ++kb) {
      float dot = 0.f;
      if (p.fixed == 2) {
        const __bf16* cp = p.ks.centre + (bk * nkb + kb) * D + d0;
#pragma unroll
        for (int i = 0; i < DL; ++i) dot = fmaf(q[i], bf2f(cp[i]), dot);
        dot = row_sum(dot);
      }
      const int ks0 = kb * KB, ks1 = min(ks0 + KB, p.Nk) - 1;
      const bool live = !BLOCK || p.block_mask[(int64_t)qb * p.nkb + kb] != 0;
      if (!row_ok || !live || ks0 > vis_end) continue;
      float u, l;
      cnt += min(ks1, vis_end) - ks0 + 1;
      if (ks1 > vis_end) {
        u = qn * pm[vis_end];
        l = -u;
      } else if (p.fixed == 2) {
        const float rq = qn * p.ks.radius[bk * nkb + kb];
        u = dot + rq;
        l = dot - rq;
      } else {
        u = qn * pm[ks1];
        l = -u;
      }
      up = fmaxf(up, u);
      lo = fmaxf(lo, l);
    }
    const float gap = p.scale * (up - lo);
    fixed = row_ok && cnt >= kMinFixedKeys && up > kNegInf && gap <= kTau;
    m_fix = p.scale * up * kLog2e;
    if (p.ks.flags != nullptr && row_ok && d0 == 0)
      p.ks.flags[((int64_t)b * p.Hq + hq) * p.Nq + qrow] = fixed ? 1 : 0;
  }

  float m_run = kNegInf, l_run = 0.f;
  const int my_qb = BLOCK ? (row_ok ? qrow : 0) / p.block_q : 0;
  for (int k0 = 0; k0 < p.Nk; k0 += TK) {
    __syncthreads();
    for (int i = tid; i < TK * D / 4; i += 64 * NWF) {
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
    // scores of the tile: each lane's partial dot product over its slice of
    // d, summed over the row's lanes; excluded pairs carry -inf
    float s[TK];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const int key = k0 + j;
      bool a = key < p.Nk && row_ok && grp[j / 16];
      if (CAUSAL) a = a && key <= qrow + p.causal_off;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DL; ++i) acc = fmaf(q[i], sK[j][d0 + i], acc);
      acc = row_sum(acc);
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
      for (int i = 0; i < DL; ++i) o[i] *= alpha;
    } else {
      m_ref = m_fix;
    }
    // excluded pairs are skipped, never multiplied by zero
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      if (s[j] != kNegInf) {
        const float e = ex2(s[j] - m_ref);
        l_run += e;
#pragma unroll
        for (int i = 0; i < DL; ++i) o[i] = fmaf(e, sV[j][d0 + i], o[i]);
      }
    }
  }

  if (row_ok) {
    const bool live = l_run > 0.f;
    const float inv = live ? 1.f / l_run : 0.f;
    float* op = (float*)p.o + b * p.o_sb + (int64_t)qrow * p.o_ss + hq * p.o_sh + d0;
#pragma unroll
    for (int i = 0; i < DL; i += 4)
      *(float4*)(op + i) = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
    if (p.lse != nullptr && d0 == 0) {
      const float m_ref = fixed ? m_fix : m_run;
      p.lse[((int64_t)b * p.Hq + hq) * p.Nq + qrow] = live ? (m_ref + log2f(l_run)) * kLn2 : kNegInf;
    }
  }
}

template <int D, bool C, bool K>
hipError_t launch_one(const FwdParams& p, hipStream_t s) {
  const dim3 grid((p.Nq + BQ - 1) / BQ, p.B * p.Hq);
  hipLaunchKernelGGL((fwd_f32_kernel<D, C, K>), grid, dim3(64 * NWF), 0, s, p);
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
