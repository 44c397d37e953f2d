// Device-side helpers shared by the gfx950 kernels: vector types, the MFMA
// and LDS-transpose builtins, bf16 conversion and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// Fixed-max eligibility: the row max may sit at most this many nats below
// the bound (so every row normaliser stays >= exp(-kTau) >> FLT_MIN).
constexpr float kTau = 64.0f;
// ... and the row must see at least this many keys (one key tile): with
// fewer, the fixed max saves nothing and its bound leaves every weight of the
// row, the largest included, rounded to bf16 for the P V product.
constexpr int kMinFixedKeys = 64;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Raw buffer resource over [base, base + bytes): loads whose total offset
// (lane offset + scalar offset) falls at or past `bytes` return 0 per dword
// without touching memory, which zero-fills tails without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past any range used here
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
// HBM -> LDS without registers (buffer_load_dwordx4 ... lds): lane i's 16
// bytes (from voff, zero when out of range) land at lds_wave + 16 * i, where
// lds_wave is the same for the whole wave. Completion is counted by vmcnt.
//
// Issued from inline asm on purpose: the compiler cannot tell which LDS bytes
// such a load writes once a read goes through the transposing-read builtin,
// so with the builtin it waits for every load in flight (the next tile's)
// before the current tile's V reads. Here it does not see the load at all;
// the caller waits with wait_all_loads() before the barrier that publishes
// the tile, and never reads LDS that a load in flight may write. The load
// has no register result (no register of the asm is written later).
//
// Wait states: the compiler inserts none for an instruction inside inline
// asm, so the asm starts with s_nop 4 (five wait states). A vector-memory
// instruction that reads an SGPR written by a VALU instruction (the
// descriptor words below come from v_readfirstlane) needs five, and the
// LDS-DMA read of M0 after an SALU write of M0 needs one.
//
// The asm takes the buffer resource as four dwords in scalar registers (the
// same words make_rsrc builds: base, base_hi | stride 0, size, flags), each
// read from the first lane: the values are uniform, and this keeps the
// operand in SGPRs whatever the compiler can prove about them.
struct DmaRsrc {
  u32x4 w;
};
__device__ __forceinline__ DmaRsrc dma_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  DmaRsrc r;
  r.w[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r.w[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r.w[2] = __builtin_amdgcn_readfirstlane(bytes);
  r.w[3] = 0x00020000u;
  return r;
}
__device__ __forceinline__ void buf_load_lds16(DmaRsrc r, const void* lds_wave, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_wave);
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r.w),
               "{m0}"(m0v)
               : "memory");
}
// Waits until none of this wave's vector-memory loads is outstanding
// (s_waitcnt vmcnt(0); the other counters are left alone).
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x70 | 0xF00); }

// exp2 on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x2 cvt2(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_convertvector(x, bf16x2);
}
__device__ __forceinline__ bf16x8 cvt8(float a0, float a1, float a2, float a3, float a4,
                                       float a5, float a6, float a7) {
  bf16x2 p0 = cvt2(a0, a1), p1 = cvt2(a2, a3), p2 = cvt2(a4, a5), p3 = cvt2(a6, a7);
  bf16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}
__device__ __forceinline__ bf16x4 cvt4(float a0, float a1, float a2, float a3) {
  bf16x2 p0 = cvt2(a0, a1), p1 = cvt2(a2, a3);
  bf16x4 r = {p0[0], p0[1], p1[0], p1[1]};
  return r;
}

__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }

// D = A * B + C, 32x32 output, K = 16, bf16 inputs (8 per lane), fp32 accum.
// A[i][k] sits in lane i + 32*(k/8), element k%8; B[k][j] in lane j + 32*(k/8);
// C[i][j] in lane j + 32*((i/4)%2), register (i%4) + 4*(i/8).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16 output, K = 32: A[i][k] in lane i + 16*(k/8), element k%8;
// C[i][j] in lane j + 16*(i/4), register i%4.
__device__ __forceinline__ f32x4 mfma16k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16 output, K = 16: A[i][k] in lane i + 16*(k/4), element k%4.
__device__ __forceinline__ f32x4 mfma16k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i receives, as element j (j = 0..3), element i%4 of the 8 bytes that
// lane 4*j + i/4 of the same group addressed.
__device__ __forceinline__ s16x4 lds_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Orders this wave's earlier LDS writes before its later LDS reads of other
// lanes' data. LDS instructions of one wave execute in order, so only the
// compiler must be kept from reordering; no wait is emitted and, unlike
// __syncthreads(), outstanding global loads are not waited for.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS swizzles of [rows][D] bf16 tiles on 16-byte chunks (row r, logical
// chunk ch -> slot), chosen so the MFMA-side reads hit distinct banks: kswz
// for tiles read as rows (16 rows x one chunk per 16 lanes), vswz for tiles
// read by the transpose load (4 rows x 2 chunks per 16 lanes). Both are
// involutions.
template <int D>
__device__ __forceinline__ int kswz(int r, int ch) {
  if constexpr (D == 128) return ch ^ (r & 15);
  else return ch ^ ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int r, int ch) {
  if constexpr (D == 128) return ch ^ ((r & 3) << 2);
  else return ch ^ (((r >> 1) & 1) << 2);
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

}  // namespace miattn
