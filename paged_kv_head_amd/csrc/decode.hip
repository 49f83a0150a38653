// Paged MLA decode kernel for gfx950.
//
// What it computes (per query row, over the row's visible latent rows K_t):
// scores P_t = scale * q.K_t, lse = log2 sum 2^P_t, out = sum 2^(P_t-lse) K_t[:512]
// ("为什么 FlashMLA 的解码内核能跑到 660 TFLOPS", section 上手示例), with the
// online-softmax recurrence over 64-token tiles ("Modular Platform 设计文档
// 全景导读", sections 六 and 七: running max, correction factor, running sum).
//
// Work decomposition.  A workgroup of 4 waves owns 128 query rows of one
// work unit (all heads of a query token share the single latent KV head, so
// one latent tile feeds 128 rows) and walks the (unit, block) range its
// split-KV part was given by the scheduler.  Wave w owns rows 32w..32w+31;
// each lane keeps one row's Q (36 bf16x8 MFMA operands) and, after the PV
// product, 256 fp32 output columns of that row in registers.
//
// Per 64-token tile:
//   1. 64 threads translate tokens to cache rows through the block table
//      (page = table[t / 64], slot = t % 64; "Modular Platform 设计文档全景
//      导读", section 四) or, for sparse units, through the index list.
//   2. The tile is staged in LDS as bf16 [64 keys][576 dims] (rows padded to
//      1168 bytes so MFMA operand reads hit distinct banks).  FP8 rows are
//      dequantised on the way: bf16(float(e4m3) * tile scale), FlashMLA
//      page section 设计 2.  Rows that are not visible are zero-filled so
//      that masked keys contribute exactly 0 to P*V.
//   3. S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from
//      LDS, B = 16 dims x 32 rows from registers).  The transposed product
//      leaves each lane holding 32 keys of ONE query row, so the row max and
//      row sum are lane-local plus one exchange with lane^32.
//   4. Online softmax in base 2 with a lazily refreshed running max: the
//      output is rescaled only when some row's max grew by more than 8
//      (p stays <= 2^8), which is exact because the final division and the
//      lse use the same stale max.
//   5. O^T += V^T P^T with the same MFMA: B = P^T straight from the S^T
//      accumulators (keys permuted consistently on both operands), A = V^T
//      gathered from the same LDS tile (V = first 512 latent dims).
// Epilogue: a unit processed in one segment writes bf16 out and lse; a split
// unit writes normalised fp32 partials and their lse to the workspace for the
// combine kernel.
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kKsStride = 1168;  // bytes per staged key row (1152 + 16)
constexpr int kQSteps = kDqk / 16;  // 36 MFMA k-steps over the 576 dims
constexpr float kRescaleThreshold = 8.0f;

__device__ inline float wave_max_pair(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

__device__ inline uint16_t bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

template <int FMT>
struct RowBytes;
template <>
struct RowBytes<0> { static constexpr int value = 1152; };
template <>
struct RowBytes<1> { static constexpr int value = 656; };

// Stage one 64-token tile into LDS.  rowoff[j] is the byte offset of key j's
// cache row, or -1 when key j is not visible (zero-filled).  Thread
// assignments keep every address a per-thread base plus a constant, and a
// wave instruction reads whole 128-byte lines of a row.
template <int FMT>
__device__ inline void stage_tile(const uint8_t* __restrict__ kv, const int64_t* rowoff,
                                  uint8_t* ks) {
  const int tid = threadIdx.x;
  if constexpr (FMT == 0) {
    // bf16: 8 threads per key row, 9 chunks of 16 bytes each, two rounds
#pragma unroll
    for (int round = 0; round < 2; ++round) {
      const int key = round * 32 + (tid >> 3);
      const int sub = tid & 7;
      const int64_t off = rowoff[key];
      const uint8_t* src = kv + off + sub * 16;
      uint8_t* dst = ks + key * kKsStride + sub * 16;
      u32x4 v[9];
#pragma unroll
      for (int j = 0; j < 9; ++j)
        v[j] = off >= 0 ? *reinterpret_cast<const u32x4*>(src + 128 * j) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 9; ++j) *reinterpret_cast<u32x4*>(dst + 128 * j) = v[j];
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // FP8: 4 threads per key row.  NoPE: 8 chunks of 16 codes per thread.
    const int key = tid >> 2;
    const int sub = tid & 3;
    const int64_t off = rowoff[key];
    const uint8_t* src = kv + off;
    uint8_t* dst = ks + key * kKsStride;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 v[4];
      float sc[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = half * 4 + jj;  // chunk cc = sub + 4*j covers dims 16*cc..
        if (off >= 0) {
          v[jj] = *reinterpret_cast<const u32x4*>(src + sub * 16 + 64 * j);
          sc[jj] = *reinterpret_cast<const float*>(src + 512 + (j >> 1) * 4);
        } else {
          v[jj] = u32x4{0, 0, 0, 0};
          sc[jj] = 0.0f;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = half * 4 + jj;
        u16x8 lo, hi;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(v[jj][w], false);
          const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(v[jj][w], true);
          const uint16_t b0 = bf16_bits(f01[0] * sc[jj]), b1 = bf16_bits(f01[1] * sc[jj]);
          const uint16_t b2 = bf16_bits(f23[0] * sc[jj]), b3 = bf16_bits(f23[1] * sc[jj]);
          if (w < 2) {
            lo[4 * w + 0] = b0; lo[4 * w + 1] = b1; lo[4 * w + 2] = b2; lo[4 * w + 3] = b3;
          } else {
            hi[4 * w - 8] = b0; hi[4 * w - 7] = b1; hi[4 * w - 6] = b2; hi[4 * w - 5] = b3;
          }
        }
        uint8_t* d = dst + sub * 32 + 128 * j;
        *reinterpret_cast<u16x8*>(d) = lo;
        *reinterpret_cast<u16x8*>(d + 16) = hi;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // RoPE: 2 chunks of 8 bf16 per thread
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 v = u32x4{0, 0, 0, 0};
      if (off >= 0) v = *reinterpret_cast<const u32x4*>(src + 528 + sub * 16 + 64 * j);
      *reinterpret_cast<u32x4*>(dst + 1024 + sub * 16 + 64 * j) = v;
    }
  }
}

// Four accumulator values of a lane, copied out through the lane's private
// 16-byte LDS slot.  Doing VALU arithmetic only on such copies keeps the
// output accumulators in AGPRs for the whole kernel (arithmetic directly on
// them makes the register allocator spill).
__device__ inline f32x4 acc_quad(const f32x16& acc, int q4, f32x4* slot) {
  *slot = f32x4{acc[4 * q4 + 0], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
  asm volatile("" ::: "memory");
  const f32x4 v = *slot;
  asm volatile("" ::: "memory");
  return v;
}

// Move a lane's (O, m, l) into its flush record, merging with what is
// already there (two partial sums with references m1, m2 merge as
// M = max, each scaled by 2^(m_i - M)), and restart O and l from zero.
__device__ inline __attribute__((always_inline)) void flush_rows(float* rec, bool had, f32x16* o,
                                                                 float m, float& l, f32x4* slot) {
  float a = 0.0f, c = 1.0f, M = m;
  if (had) {
    const float mf = rec[257];
    M = fmaxf(mf, m);
    a = __builtin_amdgcn_exp2f(mf - M);
    c = __builtin_amdgcn_exp2f(m - M);
  }
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4* dst = reinterpret_cast<f32x4*>(rec + cb * 16 + 4 * q4);
      const f32x4 old = had ? *dst * a : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      *dst = old + acc_quad(o[cb], q4, slot) * c;
    }
    o[cb] = f32x16{};
  }
  rec[256] = (had ? rec[256] * a : 0.0f) + l * c;
  rec[257] = M;
  l = 0.0f;
}

template <int FMT, bool SPARSE>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ks[kPage * kKsStride];
  __shared__ int64_t rowoff[kPage];
  __shared__ uint32_t vmask[2];
  __shared__ f32x4 oslots[kThreads];  // per-lane slot for copying accumulators
  f32x4* const oslot = &oslots[threadIdx.x];

  const Shape& s = a.s;
  constexpr int kRowBytes = RowBytes<FMT>::value;

  // Workgroup -> (part, row group).  Workgroups are dealt round-robin to
  // the 8 XCDs, so the row groups of one part get ids congruent mod 8 and
  // share that XCD's L2 for the tiles they both read.
  const int wg = blockIdx.x;
  const int span = 8 * s.groups;
  const int part = (wg / span) * 8 + (wg % span) % 8;
  const int grp = (wg % span) / 8;
  if (part >= a.num_parts) return;
  const int32_t* sc = a.sched + 8 * (size_t)part;
  const int ub = sc[0], kb0 = sc[1], ue = sc[2], ke = sc[3], split0 = sc[4];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;  // row within the wave / key-slot group
  const int h = lane >> 5;  // half of the wave
  const int r = grp * kRowsPerGroup + wave * 32 + n;  // query row in unit
  const bool row_ok = r < s.rows;
  // per-lane flush record: 256 output columns, l, m
  float* flush = a.ws_flush + ((int64_t)(part * s.groups + grp) * kThreads + threadIdx.x) * kFlushFloats;

  for (int u = ub; u < s.units && (u < ue || (u == ue && ke > 0)); ++u) {
    const int b = SPARSE ? u / s.s_q : u;
    const int L = a.seqlens[b];
    const int nb = SPARSE ? (s.topk + kPage - 1) / kPage : (max(L, 0) + kPage - 1) / kPage;
    const int kfirst = (u == ub) ? kb0 : 0;
    const int kend = (u == ue) ? ke : nb;
    if (kfirst >= kend) continue;
    const int seg = (u == ub) ? split0 : 0;
    const int nsplit = a.num_splits[u + 1] - a.num_splits[u];

    // Q operand fragments of this lane's row: dims 16*s + 8*h .. +8
    bf16x8 qf[kQSteps];
    {
      const uint16_t* qrow = a.q + ((int64_t)u * s.rows + (row_ok ? r : 0)) * kDqk + 8 * h;
#pragma unroll
      for (int st = 0; st < kQSteps; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st);
    }
    // last visible position for this row (dense causal)
    int tlim = L - 1;
    if (!SPARSE && s.is_causal) tlim = L - s.s_q + (r / s.h_q);

    float m = -INFINITY;  // running (possibly stale) max, log2 units
    float l = 0.0f;       // running sum of this lane's half of the keys
    bool flushed = false; // wave-uniform: rows parked in the flush area
    f32x16 o[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = f32x16{};

    for (int kt = kfirst; kt < kend; ++kt) {
      __syncthreads();  // previous tile fully consumed
      if (threadIdx.x < kPage) {
        const int j = threadIdx.x;
        int t;
        bool valid;
        if constexpr (SPARSE) {
          const int k = kt * kPage + j;
          t = k < s.topk ? a.indices[(int64_t)u * s.topk + k] : -1;
          valid = t >= 0 && t < L;
        } else {
          t = kt * kPage + j;
          valid = t < L;
        }
        int64_t off = -1;
        if (valid) {
          const int page = a.block_table[(int64_t)b * s.max_pages + (t >> 6)];
          off = ((int64_t)page * kPage + (t & 63)) * kRowBytes;
        }
        rowoff[j] = off;
        const uint64_t bal = __ballot(valid);
        if (j == 0) {
          vmask[0] = (uint32_t)bal;
          vmask[1] = (uint32_t)(bal >> 32);
        }
      }
      __syncthreads();
      stage_tile<FMT>(a.kv, rowoff, ks);
      __syncthreads();

      const uint64_t vm = (uint64_t)vmask[0] | ((uint64_t)vmask[1] << 32);
      const int jlim = SPARSE ? 63 : min(63, tlim - kt * kPage);  // keys j <= jlim may count

      // The tile is consumed as two 32-key halves to bound register use.
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        // ---- S^T = K Q^T for keys 32*kb2 .. 32*kb2+31
        f32x16 sacc = f32x16{};
        {
          const uint8_t* kbase = ks + (kb2 * 32 + n) * kKsStride + h * 16;
#pragma unroll
          for (int st = 0; st < kQSteps; ++st) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kbase + st * 32);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], sacc, 0, 0, 0);
            if ((st & 3) == 3) __builtin_amdgcn_sched_barrier(0);
          }
        }
        // ---- mask, scale, max over this half
        float tmax = -INFINITY;
        const uint32_t lanemask = (uint32_t)(vm >> (kb2 * 32 + 4 * h));
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb2 * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          const bool ok = ((lanemask >> (8 * (v >> 2) + (v & 3))) & 1) && key <= jlim;
          const float x = ok ? sacc[v] * s.scale_log2 : -INFINITY;
          sacc[v] = x;
          tmax = fmaxf(tmax, x);
        }
        tmax = wave_max_pair(tmax);
        const float mnew = fmaxf(m, tmax);
        // A row that has seen no visible key yet holds O = 0 and l = 0: it
        // adopts the new max for free.
        if (m == -INFINITY) m = mnew;
        const bool grow = mnew > m + kRescaleThreshold;
        if (__any(grow)) {
          // Rare: park this wave's rows in the flush area and restart them
          // from zero (O never goes through a loop-carried rescale).
          flush_rows(flush, flushed, o, m, l, oslot);
          flushed = true;
          if (grow) m = mnew;
        }
        const float muse = (m == -INFINITY) ? 0.0f : m;
        // ---- probabilities -> bf16 P^T operands (key-slot order = S^T order)
        bf16x8 pf[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(sacc[v] - muse);
          l += p;
          pf[v >> 3][v & 7] = (__bf16)p;
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- O^T += V^T P^T over 16 column blocks of 32
        const uint8_t* vbase = ks + (32 * kb2 + 4 * h) * kKsStride + 2 * n;
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) {
            // k slot (h, e) <-> key 32*kb2 + 16*sp + 8*(e/4) + 4*h + e%4
            const uint8_t* vb = vbase + 16 * sp * kKsStride + 64 * cb;
            u16x8 vv;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              vv[e] = *reinterpret_cast<const uint16_t*>(vb + (8 * (e >> 2) + (e & 3)) * kKsStride);
            o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[sp],
                                                            o[cb], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // ---- epilogue: fold in a flush record (if any), normalise, store.
    float fa = 0.0f, fc = 1.0f, mfin = m, lfin = l;
    if (flushed) {
      const float mf = flush[257];
      mfin = fmaxf(mf, m);
      fa = __builtin_amdgcn_exp2f(mf - mfin);
      fc = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mfin);
      lfin = flush[256] * fa + l * fc;
    }
    const float ltot = lfin + __shfl_xor(lfin, 32);
    const float lse2 = ltot > 0.0f ? mfin + log2f(ltot) : -INFINITY;
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    const float ca = fa * inv, cc = fc * inv;
    if (row_ok) {
      const int64_t row = (int64_t)u * s.rows + r;
      const bool direct = nsplit == 1;
      const int64_t wrow = direct ? 0 : ((int64_t)a.num_splits[u] + seg) * s.rows + r;
      uint16_t* orow16 = a.out + row * kDv + 4 * h;
      float* orow32 = a.ws_o + wrow * kDv + 4 * h;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int col = 32 * cb + 8 * q4;  // + 4*h folded into the row pointers
          f32x4 v = acc_quad(o[cb], q4, oslot) * cc;
          if (flushed) {
            const f32x4 f = *reinterpret_cast<const f32x4*>(flush + cb * 16 + 4 * q4);
            v += f * ca;
          }
          if (direct) {
            const uint32_t w0 = (uint32_t)bf16_bits(v[0]) | ((uint32_t)bf16_bits(v[1]) << 16);
            const uint32_t w1 = (uint32_t)bf16_bits(v[2]) | ((uint32_t)bf16_bits(v[3]) << 16);
            *reinterpret_cast<uint2*>(orow16 + col) = make_uint2(w0, w1);
          } else {
            *reinterpret_cast<f32x4*>(orow32 + col) = v;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (h == 0) {
        if (direct)
          a.lse[row] = s.natural ? lse2 * 0.69314718055994531f : lse2;
        else
          a.ws_lse[wrow] = lse2;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int span = 8 * a.s.groups;
  const int grid = ((a.num_parts + 7) / 8) * span;
  const bool sparse = a.s.topk > 0;
  if (a.s.kv_format == 0) {
    if (sparse)
      hipLaunchKernelGGL((decode_kernel<0, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<0, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  } else {
    if (sparse)
      hipLaunchKernelGGL((decode_kernel<1, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<1, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
