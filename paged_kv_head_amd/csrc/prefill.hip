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
