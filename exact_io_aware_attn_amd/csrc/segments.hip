// Row segments of a block mask whose block_q is not a multiple of 32.
//
// A wave of the prefill kernel takes 32 query rows. When block_q is not a
// multiple of 32, a wave must not mix rows whose mask rows differ, or one
// row would be multiplied with keys that are dead for it. Block rows whose
// mask rows are identical form a run, and every row of a run sees the same
// keys. So the rows of each run are cut into 32-row segments (the last one
// shorter), no segment crosses a run, and each wave takes one segment. With
// a frame-structured mask ("TPU attention 최적화 실전 가이드", 3단계: every
// block of a frame attends the same frames), a run is a whole frame, and a
// frame of 880 rows needs 28 waves instead of 33 for 11 block rows of 80.
//
// Two kernels build the table in the caller's workspace:
//   1. run_start_kernel: flag[i] = 1 if block row i starts a run (row 0, or
//      its mask row differs from row i - 1 in any block's zero/nonzero state)
//   2. segment_kernel (one workgroup): for each block row i, the segments that
//      start inside it, from the start of its run and the flags of the next
//      two block rows; written in row order: seg[s] = {first row, rows}, and
//      *count = the number of segments.
// The segments come out in increasing row order, and their number never
// exceeds (Nq / block_q) * ceil(block_q / 32), the count without merging.
#include "internal.hpp"

namespace miattn {
namespace {

constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(64) run_start_kernel(const uint8_t* __restrict__ mask,
                                                        int nkb, uint8_t* __restrict__ flag) {
  const int i = blockIdx.x;
  const int lane = threadIdx.x;
  bool diff = false;
  if (i > 0) {
    const uint8_t* a = mask + (int64_t)i * nkb;
    const uint8_t* b = a - nkb;
    for (int j = lane; j < nkb; j += 64) diff |= (a[j] != 0) != (b[j] != 0);
  }
  const bool start = i == 0 || __ballot(diff) != 0ull;
  if (lane == 0) flag[i] = start ? 1 : 0;
}

// inclusive scan over the workgroup (kScanThreads threads, 64-lane waves)
template <bool MAX>
__device__ int block_scan(int v, int* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int NWV = kScanThreads / 64;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v = MAX ? max(v, u) : v + u;
  }
  if (lane == 63) wtot[w] = v;
  __syncthreads();
  if (w == 0) {
    int x = lane < NWV ? wtot[lane] : (MAX ? -1 : 0);
#pragma unroll
    for (int d = 1; d < NWV; d <<= 1) {
      const int u = __shfl_up(x, d, 64);
      if (lane >= d) x = MAX ? max(x, u) : x + u;
    }
    if (lane < NWV) wtot[lane] = x;
  }
  __syncthreads();
  if (w > 0) v = MAX ? max(v, wtot[w - 1]) : v + wtot[w - 1];
  __syncthreads();  // wtot is reused by the next scan
  return v;
}

__global__ void __launch_bounds__(kScanThreads) segment_kernel(const uint8_t* __restrict__ flag,
                                                               int nqb, int block_q,
                                                               int* __restrict__ count,
                                                               int2* __restrict__ seg) {
  __shared__ int wtot[kScanThreads / 64];
  __shared__ int carry[2];  // run start of the last block row so far, segments so far
  const int t = threadIdx.x;
  if (t == 0) {
    carry[0] = 0;
    carry[1] = 0;
  }
  __syncthreads();
  for (int base = 0; base < nqb; base += kScanThreads) {
    const int rb_in = carry[0], seg_in = carry[1];
    const int i = base + t;
    const bool in = i < nqb;
    // first block row of i's run: the last run start at or before i
    int rb = block_scan<true>(in && flag[i] ? i : -1, wtot);
    rb = max(rb, rb_in);
    int cnt = 0, k0 = 0, avail = 0;
    if (in) {
      const int o = (i - rb) * block_q;       // rows of the run before block row i
      k0 = (o + 31) / 32;                     // first segment starting in block row i
      cnt = (o + block_q + 31) / 32 - k0;     // segments starting in block row i
      // a segment starting here ends at most two block rows further on
      // (block_q >= 16); the run's rows up to there:
      int ext = 1;
      if (i + 1 < nqb && !flag[i + 1]) {
        ext = 2;
        if (i + 2 < nqb && !flag[i + 2]) ext = 3;
      }
      avail = o + ext * block_q;
    }
    const int incl = block_scan<false>(cnt, wtot) + seg_in;
    const int first = incl - cnt;
    for (int m = 0; m < cnt; ++m) {
      const int k = k0 + m;
      seg[first + m] = make_int2(rb * block_q + 32 * k, min(32, avail - 32 * k));
    }
    if (t == kScanThreads - 1) {
      carry[0] = rb;
      carry[1] = incl;
    }
    __syncthreads();
  }
  if (t == 0) *count = carry[1];
}

}  // namespace

size_t segment_table_bytes(int Nq, int block_q) {
  if (Nq <= 0 || block_q <= 0) return 0;
  const int64_t nqb = Nq / block_q;
  const int64_t nseg = nqb * ((block_q + 31) / 32);
  return (size_t)(align16(nqb) + 16 + nseg * (int64_t)sizeof(int2));
}

hipError_t launch_segments(const uint8_t* block_mask, int Nq, int block_q, int nkb, void* ws,
                           SegTable* out, hipStream_t s) {
  const int nqb = Nq / block_q;
  uint8_t* flag = (uint8_t*)ws;
  int* count = (int*)((char*)ws + align16(nqb));
  int2* seg = (int2*)((char*)count + 16);
  hipLaunchKernelGGL(run_start_kernel, dim3(nqb), dim3(64), 0, s, block_mask, nkb, flag);
  hipLaunchKernelGGL(segment_kernel, dim3(1), dim3(kScanThreads), 0, s, flag, nqb, block_q, count,
                     seg);
  out->count = count;
  out->seg = seg;
  return hipGetLastError();
}

}  // namespace miattn
