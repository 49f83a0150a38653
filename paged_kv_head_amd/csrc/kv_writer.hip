// FP8 KV writer: quantises new latent tokens (576 bf16 values each) into the
// 656-byte cache row and stores every row at its paged slot.
//
// Row layout ("为什么 FlashMLA 的解码内核能跑到 660 TFLOPS——内核里的 5 个关键
// 设计", section 设计 2, FP8 KV cache): the 512 NoPE values are cut into four
// 1x128 tiles; each tile keeps one fp32 scale and 128 e4m3 codes; the 64 RoPE
// values stay bf16.  Bytes [0,512) codes, [512,528) the four scales,
// [528,656) RoPE.  Quantisation rule (the page gives only the tile shape and
// the scale type): scale = amax / 448 as one fp32 division, code =
// e4m3fn(x / scale) with the quotient another fp32 division, rounded to the
// nearest code (ties to even) and saturated to +-448; an all-zero tile gets
// scale 0 and code 0x00 throughout.  The kernel computes exactly these
// correctly rounded fp32 quotients, through a reciprocal and two residual
// corrections instead of a full division per value.
//
// Slot of token j of sequence b: logical position t = start_pos[b] + j, page
// block_table[b][t / 64], slot t % 64 ("Modular Platform 设计文档全景导读",
// section 四, PagedAttention: divmod of the token index by the page size,
// then the block table).  Tokens whose position, page index or page entry is
// out of range are skipped.
//
// The kernel is HBM-bound: 1152 bytes read and 656 written per token.  One
// wave quantises one token at a time: lane l owns NoPE values 8l..8l+7 (one
// 16-byte load, one 8-byte store of codes), so the 16 lanes of a DPP row
// hold exactly one 1x128 tile and its amax is four DPP max steps; lanes 0..7
// also move the 128 bytes of RoPE.  Each wave handles kTokPerWave tokens with
// all their loads issued before any arithmetic; one token per wave and eight
// waves per workgroup measured fastest (more tokens per wave gave fewer waves
// in flight and about 8% less bandwidth).
#include "internal.h"

namespace mla {
namespace {

constexpr int kWaves = 8;
constexpr int kTokPerWave = 1;
constexpr int kTokPerBlock = kWaves * kTokPerWave;

// DPP controls (GFX9 encoding): quad permutations and the row (16-lane)
// mirrors.
constexpr int kQuadSwap1 = 0xB1;      // [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each half row
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each row

template <int kCtrl>
__device__ inline float dpp_max(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(o));
}

// Maximum over the 16 lanes of this lane's DPP row.
__device__ inline float row16_max(float v) {
  v = dpp_max<kQuadSwap1>(v);
  v = dpp_max<kQuadSwap2>(v);
  v = dpp_max<kRowHalfMirror>(v);
  v = dpp_max<kRowMirror>(v);
  return v;
}

__device__ inline uint32_t to_e4m3x4(float a, float b, float c, float d) {
  // Saturate first: 448 is the largest finite e4m3fn magnitude, and the
  // conversion itself rounds to nearest even.
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__global__ void __launch_bounds__(64 * kWaves)
kv_quantize_fp8_kernel(int32_t n_new, int32_t num_pages, int32_t max_pages, int32_t ntok,
                       const uint16_t* __restrict__ kv_new, const int32_t* __restrict__ start_pos,
                       const int32_t* __restrict__ block_table, uint8_t* __restrict__ kv_pool) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok0 = (blockIdx.x * kWaves + wave) * kTokPerWave;

  uint8_t* dst[kTokPerWave];
  uint4 nope[kTokPerWave], rope[kTokPerWave];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    const int tok = tok0 + i;
    dst[i] = nullptr;
    if (tok < ntok) {
      const int b = tok / n_new;
      const int64_t t = (int64_t)start_pos[b] + (tok - b * n_new);
      if (t >= 0 && (t >> 6) < max_pages) {
        const int page = block_table[(int64_t)b * max_pages + (t >> 6)];
        if (page >= 0 && page < num_pages)
          dst[i] = kv_pool + ((int64_t)page * kPage + (t & 63)) * 656;
      }
    }
    if (dst[i]) {
      const uint16_t* src = kv_new + (int64_t)tok * kDqk;
      nope[i] = *reinterpret_cast<const uint4*>(src + lane * 8);
      if (lane < 8) rope[i] = *reinterpret_cast<const uint4*>(src + kDv + lane * 8);
    }
  }

#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    if (!dst[i]) continue;
    const uint32_t w[4] = {nope[i].x, nope[i].y, nope[i].z, nope[i].w};
    float x[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // bf16 -> fp32 is exact: the bits move to the high half
      x[2 * c] = __uint_as_float(w[c] << 16);
      x[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(x[c]));
    amax = row16_max(amax);
    const float scale = amax / 448.0f;
    uint2 codes = {0u, 0u};
    if (amax != 0.0f) {
      float qv[8];
      if (amax >= 0x1p-80f) {
        // x / scale, correctly rounded, from the correctly rounded reciprocal
        // r = 1 / scale: q0 = x * r is within 1.5 ulp; one residual step
        // (exact residual x - q * scale by fma) makes it faithful, a second
        // one rounds it correctly (Markstein's theorem: a faithful quotient
        // corrected with the exact residual times the correctly rounded
        // reciprocal, rounded once, is the correctly rounded quotient).  The
        // bound on amax keeps the reciprocal finite and every residual that
        // can change a code normal, hence exact.  The corrections turn -0
        // into +0, so the sign is taken from x (the quotient's sign).
        const float r = 1.0f / scale;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float q = x[c] * r;
          q = __builtin_fmaf(__builtin_fmaf(-q, scale, x[c]), r, q);
          q = __builtin_fmaf(__builtin_fmaf(-q, scale, x[c]), r, q);
          qv[c] = __builtin_copysignf(q, x[c]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) qv[c] = x[c] / scale;
      }
      codes.x = to_e4m3x4(qv[0], qv[1], qv[2], qv[3]);
      codes.y = to_e4m3x4(qv[4], qv[5], qv[6], qv[7]);
    }
    uint8_t* row = dst[i];
    *reinterpret_cast<uint2*>(row + lane * 8) = codes;
    if ((lane & 15) == 0) *reinterpret_cast<float*>(row + kDv + (lane >> 4) * 4) = scale;
    if (lane < 8) *reinterpret_cast<uint4*>(row + kDv + 16 + lane * 16) = rope[i];
  }
}

}  // namespace

hipError_t launch_kv_quantize_fp8(int32_t batch, int32_t n_new, int32_t num_pages,
                                  int32_t max_pages, const uint16_t* kv_new,
                                  const int32_t* start_pos, const int32_t* block_table,
                                  uint8_t* kv_pool, hipStream_t stream) {
  const int32_t ntok = batch * n_new;  // the caller checked that this fits in int32
  const int blocks = (ntok + kTokPerBlock - 1) / kTokPerBlock;
  hipLaunchKernelGGL(kv_quantize_fp8_kernel, dim3(blocks), dim3(64 * kWaves), 0, stream, n_new,
                     num_pages, max_pages, ntok, kv_new, start_pos, block_table, kv_pool);
  return hipGetLastError();
}

}  // namespace mla
