// Split-KV tile scheduler: balances ragged visible ranges over the parts of
// the decode grid.  The FlashMLA page ("为什么 FlashMLA 的解码内核能跑到 660
// TFLOPS", sections 上手示例 and 设计 5) computes such a schedule once per
// decode step from the sequence lengths and reuses it for every layer; the
// partition below is this library's own.
//
// Cost model: unit u with nb_u > 0 blocks costs nb_u + kSplitPenalty (the
// penalty stands for loading Q and writing a result).  Units are laid end to
// end on a cost line; block k of unit u sits at position C_u + penalty + k,
// where C_u is the exclusive prefix sum of costs.  With T = ceil(total /
// num_parts), part p owns exactly the blocks whose position lies in
// [p*T, (p+1)*T).  Every block therefore lands in exactly one part, and a
// part's blocks are contiguous in (unit, block) order.
#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 1024;

__device__ inline int blocks_of(const Shape& s, const int32_t* seqlens, int u) {
  if (s.topk > 0) return (s.topk + kPage - 1) / kPage;
  int L = seqlens[u];
  L = L < 0 ? 0 : L;
  return (L + kPage - 1) / kPage;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ inline int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// In-place exclusive scan of v[0..n) in LDS by the whole block; returns the
// total.  Each thread scans a contiguous chunk; chunk sums are scanned with
// wave shuffles (16 waves), then the 16 wave totals by one wave.
__device__ int block_exclusive_scan(int* v, int n, int* partial) {
  const int tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = tid * per;
  const int hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += v[i];
  const int incl = wave_inclusive_scan(sum);
  const int wave = tid >> 6;
  if ((tid & 63) == 63) partial[wave] = incl;
  __syncthreads();
  if (tid < 64) {
    const int t = tid < kThreads / 64 ? partial[tid] : 0;
    const int ti = wave_inclusive_scan(t);
    if (tid < kThreads / 64) partial[kThreads / 64 + tid] = ti - t;  // exclusive wave offsets
    if (tid == kThreads / 64 - 1) partial[2 * (kThreads / 64)] = ti;  // total
  }
  __syncthreads();
  int run = partial[kThreads / 64 + wave] + incl - sum;
  for (int i = lo; i < hi; ++i) {
    const int x = v[i];
    v[i] = run;
    run += x;
  }
  const int total = partial[2 * (kThreads / 64)];
  __syncthreads();
  return total;
}

// First block whose cost position is >= x: (unit, block), or (U, 0).
__device__ inline void first_block_at(const int* C, const int* nb, int U, int x, int pen,
                                      int* u_out, int* k_out) {
  // smallest u with C[u+1] > x
  int lo = 0, hi = U;  // answer in [lo, hi]; hi == U means none
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (C[mid + 1] > x) hi = mid; else lo = mid + 1;
  }
  if (lo >= U) { *u_out = U; *k_out = 0; return; }
  int k = x - C[lo] - pen;
  k = k < 0 ? 0 : k;
  (void)nb;
  *u_out = lo;
  *k_out = k;
}

__global__ void __launch_bounds__(kThreads)
metadata_kernel(Shape s, const int32_t* __restrict__ seqlens, int32_t num_parts,
                int32_t* __restrict__ sched, int32_t* __restrict__ num_splits) {
  __shared__ int nb[kMaxUnits];
  __shared__ int C[kMaxUnits + 1];
  __shared__ int partial[2 * (kThreads / 64) + 1];
  const int U = s.units;
  const int pen = kSplitPenalty;
  for (int u = threadIdx.x; u < U; u += kThreads) {
    int n = blocks_of(s, seqlens, u);
    nb[u] = n;
    C[u] = n > 0 ? n + pen : 0;
  }
  __syncthreads();
  const int total = block_exclusive_scan(C, U, partial);
  if (threadIdx.x == 0) C[U] = total;
  __syncthreads();
  const int T = max(1, (total + num_parts - 1) / num_parts);

  for (int p = threadIdx.x; p < num_parts; p += kThreads) {
    int ub, kb, ue, ke;
    first_block_at(C, nb, U, p * T, pen, &ub, &kb);
    first_block_at(C, nb, U, (p + 1) * T, pen, &ue, &ke);
    int s0 = 0;
    if (ub < U) s0 = p - (C[ub] + pen) / T;
    int32_t* o = sched + 8 * (size_t)p;
    o[0] = ub; o[1] = kb; o[2] = ue; o[3] = ke; o[4] = s0; o[5] = T; o[6] = pen; o[7] = 0;
  }
  // segments per unit, then their exclusive prefix
  __syncthreads();
  for (int u = threadIdx.x; u < U; u += kThreads) {
    int n = nb[u];
    int segs = 0;
    if (n > 0) segs = (C[u] + pen + n - 1) / T - (C[u] + pen) / T + 1;
    nb[u] = segs;  // reuse
  }
  __syncthreads();
  const int all = block_exclusive_scan(nb, U, partial);
  for (int u = threadIdx.x; u < U; u += kThreads) num_splits[u] = nb[u];
  if (threadIdx.x == 0) num_splits[U] = all;
}

}  // namespace

hipError_t launch_metadata(const Shape& s, const int32_t* seqlens, int32_t num_parts,
                           int32_t* sched, int32_t* num_splits, hipStream_t stream) {
  hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kThreads), 0, stream, s, seqlens, num_parts,
                     sched, num_splits);
  return hipGetLastError();
}

}  // namespace mla
