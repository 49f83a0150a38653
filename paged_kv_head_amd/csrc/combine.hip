// Combine: merges the split partial results of one query row.  Each split s
// holds its normalised output O_s (bf16) and lse_s (fp32, log2 units); with
// M = max_s lse_s the merged row is
//   lse = M + log2(sum_s 2^(lse_s - M)),   out = sum_s 2^(lse_s - lse) * O_s,
// the online-softmax merge of results over disjoint key ranges ("Modular
// Platform 设计文档全景导读", sections 六 and 七).  The FlashMLA page
// ("为什么 FlashMLA 的解码内核能跑到 660 TFLOPS", section 设计 5) runs this
// as a second kernel after the split decode.
//
// One wave per query row; each lane owns 8 of the 512 output columns.
// Units with no segment (empty visible range) get out = 0 and lse = -inf.
#include "internal.h"

namespace mla {
namespace {

constexpr int kRowsPerBlock = 4;

__device__ inline uint16_t bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

// Splits are merged online, in order, kAhead at a time: the loads of a
// group (each split's lse and this lane's 8 output values) are issued
// together, so a row costs about n / kAhead memory round trips instead of
// two per split.  With M the running max of the lse values seen, the
// running sum tot and output acc are kept relative to 2^M.
constexpr int kAhead = 4;

__global__ void __launch_bounds__(64 * kRowsPerBlock)
combine_kernel(Shape s, const int32_t* __restrict__ num_splits, const float* __restrict__ ws_lse,
               const uint16_t* __restrict__ ws_o, uint16_t* __restrict__ out,
               float* __restrict__ lse) {
  const int u = blockIdx.y;
  const int r = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= s.rows) return;
  const int first = num_splits[u];
  const int n = num_splits[u + 1] - first;
  if (n == 1) return;  // written by the decode kernel
  const int64_t row = (int64_t)u * s.rows + r;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  float M = -INFINITY, tot = 0.0f;
  for (int s0 = 0; s0 < n; s0 += kAhead) {
    float ls[kAhead];
    uint4 src[kAhead];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) {  // all loads of the group first
      const int sp = s0 + k < n ? s0 + k : n - 1;  // in range; a repeated split is given weight 0
      const int64_t wrow = (int64_t)(first + sp) * s.rows + r;
      ls[k] = s0 + k < n ? ws_lse[wrow] : -INFINITY;
      src[k] = *reinterpret_cast<const uint4*>(ws_o + wrow * kDv + lane * 8);
    }
#pragma unroll
    for (int k = 0; k < kAhead; ++k) {
      if (ls[k] == -INFINITY) continue;  // an empty split (or past the end) adds nothing
      const float Mn = fmaxf(M, ls[k]);
      const float fo = __builtin_amdgcn_exp2f(M - Mn);  // 0 while M is -inf
      const float w = __builtin_amdgcn_exp2f(ls[k] - Mn);
      tot = tot * fo + w;
      const uint32_t words[4] = {src[k].x, src[k].y, src[k].z, src[k].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {  // bf16 -> fp32 is exact: the high half of the word
        acc[2 * c] = acc[2 * c] * fo + w * __uint_as_float(words[c] << 16);
        acc[2 * c + 1] = acc[2 * c + 1] * fo + w * __uint_as_float(words[c] & 0xffff0000u);
      }
      M = Mn;
    }
  }
  float lse2 = -INFINITY;
  if (M != -INFINITY) {
    const float inv = 1.0f / tot;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] *= inv;
    lse2 = M + log2f(tot);
  }
  uint4 packed;
  packed.x = (uint32_t)bf16_bits(acc[0]) | ((uint32_t)bf16_bits(acc[1]) << 16);
  packed.y = (uint32_t)bf16_bits(acc[2]) | ((uint32_t)bf16_bits(acc[3]) << 16);
  packed.z = (uint32_t)bf16_bits(acc[4]) | ((uint32_t)bf16_bits(acc[5]) << 16);
  packed.w = (uint32_t)bf16_bits(acc[6]) | ((uint32_t)bf16_bits(acc[7]) << 16);
  *reinterpret_cast<uint4*>(out + row * kDv + lane * 8) = packed;
  if (lane == 0) lse[row] = s.natural ? lse2 * 0.69314718055994531f : lse2;
}

}  // namespace

hipError_t launch_combine(const Shape& s, const int32_t* num_splits, const float* ws_lse,
                          const uint16_t* ws_o, uint16_t* out, float* lse, hipStream_t stream) {
  dim3 grid((s.rows + kRowsPerBlock - 1) / kRowsPerBlock, s.units);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(64 * kRowsPerBlock), 0, stream, s, num_splits,
                     ws_lse, ws_o, out, lse);
  return hipGetLastError();
}

}  // namespace mla
