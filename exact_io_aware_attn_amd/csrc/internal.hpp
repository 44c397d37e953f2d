// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

// Key-statistics pre-pass (fixed-max softmax): per (batch, KV head) the keys
// are split into at most kMaxSplit ranges; each range reports a partial max
// of |k|^2 (or |k - kbar|^2) that the attention kernel reduces on load.
constexpr int kMaxSplit = 64;
constexpr int kMaxLiveBlocks = 4096;

struct KStats {
  const float* part_max;  // [B*Hkv][kMaxSplit], max |k|^2 or |k - kbar|^2
  const float* kbar;      // [B*Hkv][d] mean key (centred mode) or nullptr
  int nsplit;
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int B, Hq, Hkv, Nq, Nk;
  float scale;        // softmax scale on q . k
  float scale_log2;   // scale * log2(e)
  int causal_off;     // Nk - Nq: key j visible to row i iff j <= i + causal_off
  const uint8_t* block_mask;
  int block_q, block_k, nkb;  // nkb = Nk / block_k
  int fixed;          // 0 online, 1 fixed max, 2 fixed max with centred keys
  KStats ks;
  int n_qtiles;
};

struct KStatParams {
  const void* k;
  int64_t k_sb, k_ss, k_sh;
  int B, Hkv, Nk;
  int nsplit, keys_per_split;
  float* part_sum;   // [B*Hkv][kMaxSplit][d] (centred pass 1)
  float* part_max;   // [B*Hkv][kMaxSplit]
  float* kbar;       // [B*Hkv][d]
};

struct DecodeParams {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* seqlens;
  void* o;
  float* lse;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int B, Hq, Hkv, max_len;
  float scale_log2;
  int n_splits;      // ranges the flattened cache is cut into (<= kMaxSplits)
  float* part_o;     // [n_splits + B][Hq][d], slot = range + batch
  float* part_lse;   // [n_splits + B][Hq]
};

constexpr int kMaxSplits = 4096;
int decode_waves_per_group(int Hkv);

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, bool block,
                           hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, bool block,
                          hipStream_t s);
hipError_t launch_kstats(const KStatParams& p, int d, bool bf16, bool centred,
                         hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t s);

}  // namespace miattn
