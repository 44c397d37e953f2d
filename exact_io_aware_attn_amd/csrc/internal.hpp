// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

constexpr int kMaxLiveBlocks = 4096;

// Row segments of a block mask with block_q not a multiple of 32 (built by
// launch_segments): seg[s] = {first query row, rows (1..32)} in row order,
// *count of them; no segment mixes block rows whose mask rows differ.
struct SegTable {
  const int* count;
  const int2* seg;
};

// Key statistics of the fixed-max softmax (launch_kstats writes them): the
// keys of each (batch, KV head) are cut into nkb blocks of kb_size keys.
struct KStats {
  const float* pmax;      // [B*Hkv][Nk]: max |k_i| over the block's keys i <= j
  const __bf16* centre;   // [B*Hkv][nkb][d]: block mean rounded to bf16 (centred mode)
  const float* radius;    // [B*Hkv][nkb]: max |k_i - centre| over the block (centred mode)
  int kb_size, nkb;
  uint8_t* flags;         // [B][Hq][Nq]: 1 if the row took the fixed max, 0 if it fell back
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
  SegTable segs;              // block masks with block_q % 32 != 0
  int fixed;          // 0 online, 1 fixed max, 2 fixed max with centred keys
  KStats ks;
  int n_qtiles;
  // q = n / d as (umulhi(n, m) + n) >> s for 0 <= n < 2^31 (division by an
  // invariant integer through a multiply, Granlund and Montgomery 1994)
  uint32_t dv_G_m, dv_G_s, dv_8G_m, dv_8G_s, dv_Hkv_m, dv_Hkv_s, dv_B_m, dv_B_s;
  int G;
};

struct KStatParams {
  const void* k;
  int64_t k_sb, k_ss, k_sh;
  int B, Hkv, Nk;
  int kb_size, nkb;   // keys per block, blocks per (batch, KV head)
  float* pmax;        // [B*Hkv][Nk]
  __bf16* centre;     // [B*Hkv][nkb][d] (centred mode) or nullptr
  float* radius;      // [B*Hkv][nkb] (centred mode) or nullptr
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
  int nt;            // new tokens per sequence (rows of q per sequence), nt * Hq/Hkv <= 16
  // paged cache (table != nullptr): row r of sequence b is row r % page_size of
  // page table[b * max_pages + r / page_size]; k_sb / v_sb are then page strides
  const int32_t* table;
  int page_shift, max_pages;
  float scale_log2;
  int n_splits;      // ranges the flattened cache is cut into (<= kMaxSplits)
  float* part_o;     // [n_splits + B][nt][Hq][d], slot = range + batch
  float* part_lse;   // [n_splits + B][nt][Hq]
};

// Backward pass (bf16). The statistics live in the caller's workspace, one
// row of npad floats per (batch, query head), lse2 rows first, then dsum rows.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;   // [B][Hq][Nq], natural log (the forward's output)
  void* dq;
  void* dk;
  void* dv;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t do_sb, do_ss, do_sh;
  int64_t dq_sb, dq_ss, dq_sh;
  int64_t dk_sb, dk_ss, dk_sh;
  int64_t dv_sb, dv_ss, dv_sh;
  int B, Hq, Hkv, Nq, Nk;
  float scale;        // softmax scale on q . k
  float scale_log2;   // scale * log2(e)
  int causal_off;     // Nk - Nq
  const uint8_t* block_mask;  // [Nq / block_q][nkb] or nullptr
  int block_q, block_k, nkb;
  int npad;           // Nq rounded up to 64
  float* stats;       // [2][B*Hq][npad]: lse * log2(e) (+inf past Nq), rowsum(dO * O) (0 past Nq)
  int* flag;          // in the workspace after stats: set when a gradient accumulator turned non-finite
};

constexpr int kMaxSplits = 4096;
// backward with a block mask: at most this many 64-row tiles per side
constexpr int kMaxBwdTiles = 4096;
int decode_waves_per_group(int Hkv);

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, bool block,
                           hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, bool block,
                          hipStream_t s);
hipError_t launch_kstats(const KStatParams& p, int d, bool bf16, bool centred,
                         hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int d, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, bool block, hipStream_t s);

inline int64_t align16(int64_t n) { return (n + 15) & ~(int64_t)15; }
// workspace bytes of the segment table of an Nq-row mask with block_q rows per block
size_t segment_table_bytes(int Nq, int block_q);
// builds the table in ws (segment_table_bytes(Nq, block_q) bytes) on stream s
hipError_t launch_segments(const uint8_t* block_mask, int Nq, int block_q, int nkb, void* ws,
                           SegTable* out, hipStream_t s);

}  // namespace miattn
