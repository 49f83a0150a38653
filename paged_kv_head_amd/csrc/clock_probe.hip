// Shader-clock probe: a measurement helper for benchmarks, not a step of the
// decode path.  Each workgroup keeps all four matrix pipes of its compute
// unit busy with independent bf16 MFMA chains (a power draw close to the
// decode kernel's) and records, on wave 0, the elapsed shader-clock counter
// (s_memtime) and the elapsed constant-rate counter (s_memrealtime, 100 MHz)
// over the same interval.  Their ratio is the shader clock under load.
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) clock_probe_kernel(int64_t* out, int32_t spins) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (float)i);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < spins; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  // the results are consumed so the chains are not removed
  const float z = c0[0] + c1[1] + c2[2] + c3[3];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = (int64_t)(t1 - t0) + (z == 1.0e30f ? 1 : 0);
    out[2 * blockIdx.x + 1] = (int64_t)(r1 - r0);
  }
}

}  // namespace

hipError_t launch_clock_probe(int64_t* out, int32_t workgroups, int32_t spins, hipStream_t stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(workgroups), dim3(256), 0, stream, out, spins);
  return hipGetLastError();
}

}  // namespace mla
