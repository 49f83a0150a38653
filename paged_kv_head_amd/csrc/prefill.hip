// Helper kernels of the C ABI: the identity block table of sparse prefill and
// the device-side input check.
//
// Sparse prefill support: the prefill call of "为什么 FlashMLA 的解码内核能跑到
// 660 TFLOPS——内核里的 5 个关键设计" (section 上手示例) reads a flat latent
// cache kv [s_kv, d_qk] with no batch dimension and no block table.  A flat
// cache is a paged cache whose page p holds rows 64p..64p+63, so the library
// runs it through the sparse decode kernels with batch 1 and an identity
// block table; this kernel writes that table (and the one cache length,
// s_kv) into the caller's workspace before the decode launches.
#include "internal.h"

namespace mla {
namespace {

__global__ void __launch_bounds__(256)
identity_table_kernel(int32_t* __restrict__ table, int32_t pages, int32_t* __restrict__ seqlen,
                      int32_t s_kv) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < pages) table[i] = i;
  if (i == 0) *seqlen = s_kv;
}

}  // namespace

hipError_t launch_identity_table(int32_t* table, int32_t pages, int32_t* seqlen, int32_t s_kv,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(identity_table_kernel, dim3((pages + 255) / 256), dim3(256), 0, stream, table,
                     pages, seqlen, s_kv);
  return hipGetLastError();
}

}  // namespace mla

namespace mla {
namespace {

// Device-side check of the preconditions the decode calls do not test:
// 0 <= cache_seqlens[b] <= max_pages * 64 and, for every page a visible
// position of b can reach (j < ceil(L_b / 64)), 0 <= block_table[b][j] <
// num_pages.  One workgroup walks all sequences and reduces in LDS, so the
// result needs no atomics and no zeroed memory: result[0] = number of bad
// sequences, result[1] = the first bad sequence (-1 if none).
constexpr int kCheckThreads = 1024;

__global__ void __launch_bounds__(kCheckThreads)
check_inputs_kernel(int32_t batch, int32_t max_pages, int32_t num_pages,
                    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens,
                    int32_t* __restrict__ result) {
  __shared__ int bad_count[kCheckThreads / 64];
  __shared__ int bad_first[kCheckThreads / 64];
  int count = 0, first = INT32_MAX;
  for (int b = threadIdx.x; b < batch; b += kCheckThreads) {
    const int L = seqlens[b];
    bool bad = L < 0 || (int64_t)L > (int64_t)max_pages * kPage;
    const int pages = bad ? 0 : L / kPage + (L % kPage != 0);
    const int32_t* row = block_table + (int64_t)b * max_pages;
    for (int j = 0; j < pages && !bad; ++j) bad = row[j] < 0 || row[j] >= num_pages;
    if (bad) {
      ++count;
      first = min(first, b);
    }
  }
  for (int d = 32; d > 0; d >>= 1) {
    count += __shfl_xor(count, d);
    first = min(first, __shfl_xor(first, d));
  }
  if ((threadIdx.x & 63) == 0) {
    bad_count[threadIdx.x >> 6] = count;
    bad_first[threadIdx.x >> 6] = first;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0, f = INT32_MAX;
    for (int w = 0; w < kCheckThreads / 64; ++w) {
      c += bad_count[w];
      f = min(f, bad_first[w]);
    }
    result[0] = c;
    result[1] = c > 0 ? f : -1;
  }
}

}  // namespace

hipError_t launch_check_inputs(const Shape& s, const int32_t* block_table, const int32_t* seqlens,
                               int32_t* result, hipStream_t stream) {
  hipLaunchKernelGGL(check_inputs_kernel, dim3(1), dim3(kCheckThreads), 0, stream, s.batch,
                     s.max_pages, s.num_pages, block_table, seqlens, result);
  return hipGetLastError();
}

}  // namespace mla
