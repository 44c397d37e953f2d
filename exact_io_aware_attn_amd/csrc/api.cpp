// C ABI of libmiattn: host-side validation, workspace sizing and dispatch.
// Every check runs before anything is enqueued; see include/miattn.h for the
// meaning of each argument.

#include "../../include/miattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "internal.hpp"

namespace {

using miattn::kMaxLiveBlocks;

constexpr size_t kAlign = 256;
// keys per block of the fixed-max key statistics without a block mask
constexpr int kKeyBlock = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace of the fixed-max modes, in this order (each part 256-byte
// aligned): pmax fp32 [B*Hkv][Nk], flags uint8 [B][Hq][Nq], then in centred
// mode radius fp32 [B*Hkv][nkb] and centre bf16 [B*Hkv][nkb][d].
struct FwdWs {
  size_t pmax = 0, flags = 0, radius = 0, centre = 0, total = 0;
  int kb_size = 0, nkb = 0;
};

FwdWs fwd_ws(int B, int Hq, int Hkv, int Nq, int Nk, int d, int mask_kind, int block_k,
             int mode) {
  FwdWs w;
  if (mode == MIATTN_SOFTMAX_ONLINE || Nk <= 0) return w;
  w.kb_size = (mask_kind & MIATTN_MASK_BLOCK) && block_k > 0 ? block_k : kKeyBlock;
  w.nkb = (Nk + w.kb_size - 1) / w.kb_size;
  const size_t bh = (size_t)B * Hkv;
  w.pmax = 0;
  w.flags = align_up(bh * Nk * sizeof(float));
  w.total = w.flags + align_up((size_t)B * Hq * Nq);
  if (mode == MIATTN_SOFTMAX_FIXED_MAX_CENTERED) {
    w.radius = w.total;
    w.centre = w.radius + align_up(bh * w.nkb * sizeof(float));
    w.total = w.centre + align_up(bh * w.nkb * d * 2);
  }
  return w;
}

// Segment table of a block mask whose block_q is not a multiple of 32
// (placed after the fixed-max part of the workspace).
size_t seg_ws(int Nq, int mask_kind, int block_q) {
  if (!(mask_kind & MIATTN_MASK_BLOCK) || block_q <= 0 || block_q % 32 == 0) return 0;
  return align_up(miattn::segment_table_bytes(Nq, block_q));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool strides_ok(const miattn_strides& s, int64_t mult) {
  return s.b >= 0 && s.s >= 0 && s.h >= 0 && s.b % mult == 0 && s.s % mult == 0 &&
         s.h % mult == 0;
}

// Decode partials: part_o [(kMaxSplits + B) * Hq][d] then part_lse
// [(kMaxSplits + B) * Hq], fp32; sized for the largest split count.
size_t decode_ws(int B, int Hq, int d) {
  const size_t slots = (size_t)(miattn::kMaxSplits + B) * Hq;
  return align_up(slots * d * sizeof(float)) + align_up(slots * sizeof(float));
}

// Ranges the decode cache is cut into: the caller's count, or enough
// workgroups for every CU of the current device to hold one resident
// workgroup's worth of waves (eight 64-lane waves per CU).
int decode_splits(int Hkv, int kv_splits) {
  if (kv_splits > 0) return kv_splits;
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      ncu = v;
  }
  const int nw = miattn::decode_waves_per_group(Hkv);
  const int groups = Hkv / nw;
  int n = ncu * (8 / nw) / groups;
  if (n < 1) n = 1;
  if (n > miattn::kMaxSplits) n = miattn::kMaxSplits;
  return n;
}

}  // namespace

extern "C" {

const char* attn_status_str(int status) {
  switch (status) {
    case MIATTN_OK: return "ok";
    case MIATTN_ERR_NULL: return "a required pointer is NULL";
    case MIATTN_ERR_SHAPE: return "sizes are inconsistent or out of range";
    case MIATTN_ERR_UNSUPPORTED: return "request not supported (dtype, head dim, alignment or limit)";
    case MIATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case MIATTN_ERR_HIP: return "HIP runtime or launch error";
    case MIATTN_ERR_ARG: return "invalid scalar argument (scale, mask kind or softmax mode)";
    default: return "unknown status";
  }
}

size_t attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d, int mask_kind,
                                int block_q, int block_k, int softmax_mode) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || d <= 0) return 0;
  return fwd_ws(B, Hq, Hkv, Nq, Nk, d, mask_kind, block_k, softmax_mode).total +
         seg_ws(Nq, mask_kind, block_q);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int mask_kind,
             const uint8_t* block_mask, int block_q, int block_k, int softmax_mode,
             const miattn_strides* strides, void* workspace, size_t workspace_bytes,
             void* stream) {
  if (dtype != MIATTN_BF16 && dtype != MIATTN_F32) return MIATTN_ERR_UNSUPPORTED;
  if (B < 0 || Nq < 0 || Nk < 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return MIATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return MIATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return MIATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MIATTN_ERR_ARG;
  if (mask_kind < 0 || mask_kind > (MIATTN_MASK_CAUSAL | MIATTN_MASK_BLOCK)) return MIATTN_ERR_ARG;
  if (softmax_mode < MIATTN_SOFTMAX_ONLINE || softmax_mode > MIATTN_SOFTMAX_FIXED_MAX_CENTERED)
    return MIATTN_ERR_ARG;
  if (B == 0 || Nq == 0) return MIATTN_OK;  // nothing to compute
  if (q == nullptr || o == nullptr) return MIATTN_ERR_NULL;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return MIATTN_ERR_NULL;

  const bool causal = (mask_kind & MIATTN_MASK_CAUSAL) != 0;
  const bool block = (mask_kind & MIATTN_MASK_BLOCK) != 0;
  int nkb = 0;
  if (block) {
    if (block_mask == nullptr) return MIATTN_ERR_NULL;
    if (block_q <= 0 || block_k <= 0 || block_q % 16 != 0 || block_k % 16 != 0)
      return MIATTN_ERR_SHAPE;
    if (Nq % block_q != 0 || Nk % block_k != 0) return MIATTN_ERR_SHAPE;
    nkb = Nk / block_k;
    if (nkb > kMaxLiveBlocks) return MIATTN_ERR_UNSUPPORTED;
  }

  const int64_t esz = dtype == MIATTN_BF16 ? 2 : 4;
  const int64_t mult = 16 / esz;  // strides in whole 16-byte units
  miattn_strides sq{(int64_t)Nq * Hq * d, (int64_t)Hq * d, d};
  miattn_strides sk{(int64_t)Nk * Hkv * d, (int64_t)Hkv * d, d};
  miattn_strides sv = sk, so = sq;
  if (strides != nullptr) {
    sq = strides[0];
    sk = strides[1];
    sv = strides[2];
    so = strides[3];
  }
  if (!strides_ok(sq, mult) || !strides_ok(sk, mult) || !strides_ok(sv, mult) ||
      !strides_ok(so, mult))
    return MIATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(o) || !aligned16(k) || !aligned16(v))
    return MIATTN_ERR_UNSUPPORTED;
  // rows must not overlap, and one (batch, KV head) of K or V must span less
  // than 2 GiB (its rows are addressed with 32-bit byte offsets)
  if (sq.s < d || sk.s < d || sv.s < d || so.s < d) return MIATTN_ERR_UNSUPPORTED;
  if ((int64_t)Nk * sk.s * esz >= ((int64_t)1 << 31) || (int64_t)Nk * sv.s * esz >= ((int64_t)1 << 31))
    return MIATTN_ERR_UNSUPPORTED;

  const FwdWs fw = fwd_ws(B, Hq, Hkv, Nq, Nk, d, mask_kind, block_k, softmax_mode);
  const size_t ks_bytes = fw.total;
  const size_t need = ks_bytes + seg_ws(Nq, mask_kind, block_q);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MIATTN_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  miattn::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.q_sb = sq.b; p.q_ss = sq.s; p.q_sh = sq.h;
  p.k_sb = sk.b; p.k_ss = sk.s; p.k_sh = sk.h;
  p.v_sb = sv.b; p.v_ss = sv.s; p.v_sh = sv.h;
  p.o_sb = so.b; p.o_ss = so.s; p.o_sh = so.h;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal_off = Nk - Nq;
  p.block_mask = block_mask;
  p.block_q = block_q; p.block_k = block_k; p.nkb = nkb;
  // with no keys every row is empty and there is nothing to bound
  p.fixed = Nk > 0 ? softmax_mode : MIATTN_SOFTMAX_ONLINE;

  // the bf16 kernel takes the rows of such a mask in segments of identical
  // mask rows (the fp32 kernel works per block row)
  if (block && block_q % 32 != 0 && dtype == MIATTN_BF16) {
    if (miattn::launch_segments(block_mask, Nq, block_q, nkb, (char*)workspace + ks_bytes,
                                &p.segs, s) != hipSuccess)
      return MIATTN_ERR_HIP;
  }

  if (p.fixed != MIATTN_SOFTMAX_ONLINE) {
    char* ws = (char*)workspace;
    const bool centred = softmax_mode == MIATTN_SOFTMAX_FIXED_MAX_CENTERED;
    miattn::KStatParams kp{};
    kp.k = k; kp.k_sb = sk.b; kp.k_ss = sk.s; kp.k_sh = sk.h;
    kp.B = B; kp.Hkv = Hkv; kp.Nk = Nk;
    kp.kb_size = fw.kb_size; kp.nkb = fw.nkb;
    kp.pmax = (float*)(ws + fw.pmax);
    kp.radius = centred ? (float*)(ws + fw.radius) : nullptr;
    kp.centre = centred ? (__bf16*)(ws + fw.centre) : nullptr;
    if (miattn::launch_kstats(kp, d, dtype == MIATTN_BF16, centred, s) != hipSuccess)
      return MIATTN_ERR_HIP;
    p.ks.pmax = kp.pmax;
    p.ks.radius = kp.radius;
    p.ks.centre = kp.centre;
    p.ks.kb_size = fw.kb_size;
    p.ks.nkb = fw.nkb;
    p.ks.flags = (uint8_t*)(ws + fw.flags);
  }

  hipError_t e = dtype == MIATTN_BF16 ? miattn::launch_fwd_bf16(p, d, causal, block, s)
                                      : miattn::launch_fwd_f32(p, d, causal, block, s);
  return e == hipSuccess ? MIATTN_OK : MIATTN_ERR_HIP;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int max_len, int d, int kv_splits) {
  (void)max_len;
  (void)kv_splits;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return 0;
  return decode_ws(B, Hq, d);
}

size_t attn_decode_multi_workspace_bytes(int B, int n_new, int Hq, int Hkv, int max_len, int d,
                                         int kv_splits) {
  (void)max_len;
  (void)kv_splits;
  if (B <= 0 || n_new <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return 0;
  return decode_ws(B, Hq * n_new, d);
}

}  // extern "C"

namespace {

// ---- the allocation-free decode's scratch (attn_decode_noalloc): one static
// array per device, holding the split-K partials of the last such call
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of the current device's copy of `scratch`, looked up
// once per device with that device current (each device holds its own copy
// at its own address; the array's name in host code is only a stand-in).
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MIATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return MIATTN_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MIATTN_OK;
}

// noalloc: the partials go to the device's static scratch, sized for the
// split count actually used instead of the largest one
int decode_impl(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seqlens, void* o, float* lse, int dtype, int B, int nt, int Hq,
                int Hkv, int max_len, int d, float scale, int kv_splits,
                const miattn_strides* cache_strides, void* workspace, size_t workspace_bytes,
                void* stream, const int32_t* table = nullptr, int page_size = 0,
                int max_pages = 0, bool noalloc = false) {
  if (dtype != MIATTN_BF16) return MIATTN_ERR_UNSUPPORTED;
  if (B < 0 || nt <= 0 || Hq <= 0 || Hkv <= 0 || max_len < 0 || d <= 0) return MIATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return MIATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return MIATTN_ERR_UNSUPPORTED;
  if ((Hq / Hkv) * nt > 16) return MIATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MIATTN_ERR_ARG;
  if (kv_splits < 0 || kv_splits > miattn::kMaxSplits) return MIATTN_ERR_ARG;
  if (B == 0) return MIATTN_OK;
  if (q == nullptr || o == nullptr || seqlens == nullptr) return MIATTN_ERR_NULL;
  if (max_len > 0 && (k_cache == nullptr || v_cache == nullptr)) return MIATTN_ERR_NULL;

  const bool paged = table != nullptr;
  // paged: "b" strides step from page to page, max_len rows fit one page
  const int rows = paged ? page_size : max_len;
  miattn_strides sk{(int64_t)rows * Hkv * d, (int64_t)Hkv * d, d};
  miattn_strides sv = sk;
  if (cache_strides != nullptr) {
    sk = cache_strides[0];
    sv = cache_strides[1];
  }
  if (!strides_ok(sk, 8) || !strides_ok(sv, 8)) return MIATTN_ERR_UNSUPPORTED;
  // one (sequence, KV head) of a contiguous cache is addressed with 32-bit
  // byte offsets (a paged cache with 64-bit ones)
  if (!paged && ((int64_t)max_len * sk.s * 2 >= ((int64_t)1 << 31) ||
                 (int64_t)max_len * sv.s * 2 >= ((int64_t)1 << 31)))
    return MIATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return MIATTN_ERR_UNSUPPORTED;

  const int n_splits = decode_splits(Hkv, kv_splits);
  size_t need = decode_ws(B, Hq * nt, d);
  size_t po = align_up((size_t)(miattn::kMaxSplits + B) * Hq * nt * d * sizeof(float));
  if (noalloc) {
    const size_t slots = (size_t)(n_splits + B) * Hq * nt;
    po = align_up(slots * d * sizeof(float));
    need = po + align_up(slots * sizeof(float));
    if (need > kNoAllocScratchBytes) return MIATTN_ERR_WORKSPACE;
    const int rc = noalloc_scratch(&workspace);
    if (rc != MIATTN_OK) return rc;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (workspace == nullptr || workspace_bytes < need) return MIATTN_ERR_WORKSPACE;

  miattn::DecodeParams p{};
  p.q = q; p.kc = k_cache; p.vc = v_cache; p.seqlens = seqlens; p.o = o; p.lse = lse;
  p.k_sb = sk.b; p.k_ss = sk.s; p.k_sh = sk.h;
  p.v_sb = sv.b; p.v_ss = sv.s; p.v_sh = sv.h;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.max_len = max_len; p.nt = nt;
  p.table = table;
  p.page_shift = 0;
  while (paged && (1 << p.page_shift) < page_size) ++p.page_shift;
  p.max_pages = max_pages;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.n_splits = n_splits;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((char*)workspace + po);
  hipError_t e = miattn::launch_decode(p, d, (hipStream_t)stream);
  return e == hipSuccess ? MIATTN_OK : MIATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                      int dtype, int B, int n_new, int Hq, int Hkv, int page_size, int max_pages,
                      int d, float scale, int kv_splits, const miattn_strides* page_strides,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (page_size < 16 || (page_size & (page_size - 1)) != 0 || max_pages < 0)
    return MIATTN_ERR_SHAPE;
  if (B > 0 && block_table == nullptr) return MIATTN_ERR_NULL;
  if ((int64_t)page_size * max_pages > INT32_MAX) return MIATTN_ERR_SHAPE;
  return decode_impl(q, k_pages, v_pages, seqlens, o, lse, dtype, B, n_new, Hq, Hkv,
                     page_size * max_pages, d, scale, kv_splits, page_strides, workspace,
                     workspace_bytes, stream, block_table, page_size, max_pages);
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seqlens, void* o, float* lse, int dtype, int B, int Hq, int Hkv,
                int max_len, int d, float scale, int kv_splits,
                const miattn_strides* cache_strides, void* workspace, size_t workspace_bytes,
                void* stream) {
  return decode_impl(q, k_cache, v_cache, seqlens, o, lse, dtype, B, 1, Hq, Hkv, max_len, d, scale,
                     kv_splits, cache_strides, workspace, workspace_bytes, stream);
}

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens, void* o, float* lse, int dtype, int B, int Hq,
                        int Hkv, int max_len, int d, float scale, int kv_splits,
                        const miattn_strides* cache_strides, void* stream) {
  return decode_impl(q, k_cache, v_cache, seqlens, o, lse, dtype, B, 1, Hq, Hkv, max_len, d, scale,
                     kv_splits, cache_strides, nullptr, 0, stream, nullptr, 0, 0, true);
}

int attn_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seqlens, void* o, float* lse, int dtype, int B, int n_new,
                      int Hq, int Hkv, int max_len, int d, float scale, int kv_splits,
                      const miattn_strides* cache_strides, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, seqlens, o, lse, dtype, B, n_new, Hq, Hkv, max_len, d,
                     scale, kv_splits, cache_strides, workspace, workspace_bytes, stream);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq) {
  if (B < 0 || Hq <= 0 || Nq < 0) return 0;
  const size_t npad = (size_t)(Nq + 63) / 64 * 64;
  const size_t stats = align_up(2 * (size_t)B * Hq * npad * sizeof(float));
  return stats > 0 ? stats + align_up(sizeof(int)) : 0;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int dtype, int B, int Hq,
             int Hkv, int Nq, int Nk, int d, float scale, int mask_kind,
             const uint8_t* block_mask, int block_q, int block_k,
             const miattn_strides* strides, void* workspace, size_t workspace_bytes,
             void* stream) {
  if (dtype != MIATTN_BF16) return MIATTN_ERR_UNSUPPORTED;
  if (B < 0 || Nq < 0 || Nk < 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return MIATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return MIATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return MIATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MIATTN_ERR_ARG;
  if (mask_kind < 0 || mask_kind > (MIATTN_MASK_CAUSAL | MIATTN_MASK_BLOCK)) return MIATTN_ERR_ARG;
  const bool block = (mask_kind & MIATTN_MASK_BLOCK) != 0;
  if (block) {
    if (block_q <= 0 || block_k <= 0 || block_q % 16 != 0 || block_k % 16 != 0)
      return MIATTN_ERR_SHAPE;
    if (Nq % block_q != 0 || Nk % block_k != 0) return MIATTN_ERR_SHAPE;
    // live-tile lists of 64-row tiles per workgroup
    if ((Nq + 63) / 64 > miattn::kMaxBwdTiles || (Nk + 63) / 64 > miattn::kMaxBwdTiles)
      return MIATTN_ERR_UNSUPPORTED;
  }
  if (B == 0 || (Nq == 0 && Nk == 0)) return MIATTN_OK;
  if (block && Nq > 0 && Nk > 0 && block_mask == nullptr) return MIATTN_ERR_NULL;
  if (Nq > 0 && (q == nullptr || o == nullptr || dout == nullptr || lse == nullptr || dq == nullptr))
    return MIATTN_ERR_NULL;
  if (Nk > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return MIATTN_ERR_NULL;

  miattn_strides sq{(int64_t)Nq * Hq * d, (int64_t)Hq * d, d};
  miattn_strides sk{(int64_t)Nk * Hkv * d, (int64_t)Hkv * d, d};
  miattn_strides st[8] = {sq, sk, sk, sq, sq, sq, sk, sk};  // q k v o dout dq dk dv
  if (strides != nullptr)
    for (int i = 0; i < 8; ++i) st[i] = strides[i];
  for (int i = 0; i < 8; ++i) {
    if (!strides_ok(st[i], 8)) return MIATTN_ERR_UNSUPPORTED;
    if (st[i].s < d) return MIATTN_ERR_UNSUPPORTED;  // rows must not overlap
  }
  const void* ptrs[8] = {q, k, v, o, dout, dq, dk, dv};
  for (int i = 0; i < 8; ++i)
    if (ptrs[i] != nullptr && !aligned16(ptrs[i])) return MIATTN_ERR_UNSUPPORTED;
  // streamed tiles are addressed with 32-bit byte offsets within one
  // (batch, head) of Q, dO, K and V
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)Nq * st[0].s * 2 >= lim || (int64_t)Nq * st[4].s * 2 >= lim ||
      (int64_t)Nk * st[1].s * 2 >= lim || (int64_t)Nk * st[2].s * 2 >= lim)
    return MIATTN_ERR_UNSUPPORTED;
  const size_t need = attn_bwd_workspace_bytes(B, Hq, Nq);
  if (need >= (size_t)lim) return MIATTN_ERR_UNSUPPORTED;  // statistics offsets are 32-bit
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MIATTN_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return MIATTN_ERR_UNSUPPORTED;

  miattn::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.q_sb = st[0].b; p.q_ss = st[0].s; p.q_sh = st[0].h;
  p.k_sb = st[1].b; p.k_ss = st[1].s; p.k_sh = st[1].h;
  p.v_sb = st[2].b; p.v_ss = st[2].s; p.v_sh = st[2].h;
  p.o_sb = st[3].b; p.o_ss = st[3].s; p.o_sh = st[3].h;
  p.do_sb = st[4].b; p.do_ss = st[4].s; p.do_sh = st[4].h;
  p.dq_sb = st[5].b; p.dq_ss = st[5].s; p.dq_sh = st[5].h;
  p.dk_sb = st[6].b; p.dk_ss = st[6].s; p.dk_sh = st[6].h;
  p.dv_sb = st[7].b; p.dv_ss = st[7].s; p.dv_sh = st[7].h;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal_off = Nk - Nq;
  p.block_mask = block ? block_mask : nullptr;
  p.block_q = block ? block_q : 0;
  p.block_k = block ? block_k : 0;
  p.nkb = block ? Nk / block_k : 0;
  p.npad = (Nq + 63) / 64 * 64;
  p.stats = (float*)workspace;
  p.flag = need > 0 ? (int*)((char*)workspace + align_up(2 * (size_t)B * Hq * p.npad * sizeof(float)))
                    : nullptr;
  hipError_t e = miattn::launch_bwd_bf16(p, d, (mask_kind & MIATTN_MASK_CAUSAL) != 0, block,
                                         (hipStream_t)stream);
  return e == hipSuccess ? MIATTN_OK : MIATTN_ERR_HIP;
}

}  // extern "C"
