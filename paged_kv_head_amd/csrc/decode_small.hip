// Paged MLA decode for units of few query rows (s_q * h_q <= 32, over a bf16
// latent cache or the 656-byte FP8 cache), dense: the shape a GPU
// holds when the 128 query heads are split across GPUs ("Modular Platform
// 设计文档全景导读", section 九: for MLA only the query heads can be split,
// the latent KV is replicated).  It computes what the main decode kernel
// computes (per row: scores P_t = scale * q.K_t, lse = log2 sum 2^P_t,
// out = sum 2^(P_t - lse) K_t[:512]; "为什么 FlashMLA 的解码内核能跑到 660
// TFLOPS", section 上手示例; online softmax and merges as in the Modular
// guide, sections 六 and 七), and writes the same outputs and split partials.
//
// With so few rows the work per key is small and the cache stream from HBM
// is the bound, so the design keeps loads flowing instead of sharing tiles.
// A workgroup owns all rows of its unit (one or two 16-row MFMA blocks).
// Inside a workgroup:
//   * wave w owns keys 16w .. 16w+15 of every 64-key page of the segment (a
//     quarter tile) and streams them into its own pair of LDS buffers with
//     direct global->LDS copies (1 KiB per instruction, no registers): the
//     next quarter's copies are issued before the current one is computed,
//     and no barrier is needed inside the loop;
//   * scores are computed transposed, S^T = K Q^T, with 16x16x32 bf16 MFMAs
//     (K from LDS, Q in registers); a lane ends up with 4 keys of one row,
//     which is exactly the B-operand layout of P^T for O^T += V^T P^T
//     (16x16x16 MFMAs), so the probabilities never leave the registers;
//   * FP8 rows are staged raw and dequantised into the MFMA operands (the
//     page's rule, bf16(float(code) * tile scale)) where they are used;
//   * O^T keeps one row per lane; the probabilities are taken against the
//     first max a row sees, which may lag the true max by up to 2^64 (far
//     inside the fp32 range), so the output is never rescaled in the loop;
//     a row whose scores climb further makes the wave run its segment again
//     against the exact max it found;
//   * each wave keeps its own running max, sum and output over its own keys;
//     at the end of a segment the four are merged in LDS in a fixed order
//     (deterministic results) and written like the main kernel's.
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8s __attribute__((ext_vector_type(8)));
typedef float f32x4s __attribute__((ext_vector_type(4)));

constexpr int kSWaves = 4;
constexpr int kSQuarter = 16;  // keys per wave per page

// LDS layout of a staged quarter tile.  bf16 rows (1152 bytes) get a pitch
// of 1168 bytes; FP8 rows (656 bytes) keep theirs.  Either way 16
// consecutive rows start on 16 distinct 4-bank groups, so the operand reads
// below are free of bank conflicts.  Slot 64*c + lane of a buffer is
// 16-byte chunk `slot % kSlots` of row `slot / kSlots`.
template <int FMT>
struct SmallLayout;
template <>
struct SmallLayout<0> {
  static constexpr int kRowBytes = 1152, kPitch = 1168, kSlots = 73, kDataSlots = 72;
};
template <>
struct SmallLayout<1> {
  static constexpr int kRowBytes = 656, kPitch = 656, kSlots = 41, kDataSlots = 41;
};
template <int FMT>
constexpr int kSCopies = (kSQuarter * SmallLayout<FMT>::kSlots + 63) / 64;  // 19 (bf16), 11 (FP8)
template <int FMT>
constexpr int kSBuf = kSCopies<FMT> * 1024;
constexpr int kSSteps = kDqk / 32;  // 18 k-steps of 32 dims (16 NoPE, 2 RoPE)
constexpr int kSOPitch = 516;  // floats per merge-buffer row
// The running max a row's probabilities are taken against may lag the true
// max by up to this much (log2 units): probabilities stay <= 2^64, sums far
// inside the fp32 range.  A larger climb restarts the wave's segment.
constexpr float kSLag = 64.0f;
// LDS operand reads in flight ahead of their MFMA (the LDS counter holds at
// most 15 outstanding reads: one K read per step, one V read per column
// block, and the two phases do not overlap)
constexpr int kSKAhead = 4;
constexpr int kSVAhead = 3;
// FP8 rows: pairs of V^T operands (one transposing read each) in flight.
constexpr int kSVPairAhead = 2;

// Stands in for the cache bytes of keys that are not visible.
__device__ __attribute__((aligned(16))) const uint8_t g_zero16[16] = {};

// 16 bytes per lane from global memory into LDS at m0 + 16 * lane.  Issued
// from inline assembly, so completion is waited for explicitly (vmcnt).
__device__ inline void dma16_to_lds(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(m0) : "memory", "m0");
}

__device__ inline uint16_t to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

typedef __bf16 bf16x4s __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4s __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2s __attribute__((ext_vector_type(2)));
typedef float f32x2s __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (nearest even), lo in bits 0..15, as one
// paired conversion: built as a bf16 vector that the MFMA operand then
// reinterprets, the compiler would convert each value on its own and pack.
__device__ inline uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2s{lo, hi}, bf16x2s));
}
using cint32s = const __attribute__((address_space(4))) int32_t;

// The copy slots of a lane, the same for every quarter: copy c loads slot
// 64*c + lane of the buffer, which is chunk `slot % kSlots` of key
// `slot / kSlots`.  FP8 rows keep them in registers, packed as
// (key << 16) | byte offset of the chunk in the quarter; padding slots get
// key 16, past every key, so one unsigned compare against
// (visible keys << 16) picks the cache row or the zero row.  bf16 rows (19
// copies, in a kernel short of registers) walk the slots as they go.
template <int FMT>
struct CopySlots {
  __device__ inline void init(int) {}
};
template <>
struct CopySlots<1> {
  uint32_t v[kSCopies<1>];
  __device__ inline void init(int lane) {
    using Lay = SmallLayout<1>;
#pragma unroll
    for (int c = 0; c < kSCopies<1>; ++c) {
      const int slot = 64 * c + lane, key = slot / Lay::kSlots, chunk = slot % Lay::kSlots;
      v[c] = key < kSQuarter ? ((uint32_t)key << 16) | (uint32_t)(key * Lay::kRowBytes + chunk * 16)
                             : (uint32_t)kSQuarter << 16;
    }
  }
};

// Copies of one quarter tile (keys 16*wave .. +15 of page `page`, logical
// positions tbase ..) into the LDS buffer at lds (layout above); padding
// slots and keys at or past L come from the zero row.
template <int FMT>
__device__ inline void issue_quarter(const uint8_t* __restrict__ kv, int page, int wave, int tbase,
                                     int L, uint32_t lds, int lane, const CopySlots<FMT>& slots) {
  using Lay = SmallLayout<FMT>;
  const uint8_t* src0 = kv + ((int64_t)page * kPage + kSQuarter * wave) * Lay::kRowBytes;
  if constexpr (FMT == 1) {
    static_assert(Lay::kDataSlots == Lay::kSlots && kSQuarter * Lay::kRowBytes <= 0x10000,
                  "every in-row slot holds data; offsets fit in 16 bits");
    const uint32_t lim = (uint32_t)min(max(L - tbase, 0), kSQuarter) << 16;
#pragma unroll
    for (int c = 0; c < kSCopies<FMT>; ++c) {
      const uint32_t sl = slots.v[c];
      const void* src = sl < lim ? (const void*)(src0 + (sl & 0xFFFFu)) : (const void*)g_zero16;
      dma16_to_lds(src, lds + 1024 * c);
    }
  } else {
    // slot 64*c + lane = (key, chunk); stepping by 64 slots wraps the chunk
    // at most once (73 slots a row)
    static_assert(Lay::kSlots >= 64, "one wrap per step");
    int key = lane / Lay::kSlots, chunk = lane % Lay::kSlots;
#pragma unroll 1
    for (int c = 0; c < kSCopies<FMT>; ++c) {
      const bool ok = key < kSQuarter && chunk < Lay::kDataSlots && tbase + key < L;
      const void* src = ok ? (const void*)(src0 + key * Lay::kRowBytes + chunk * 16) : (const void*)g_zero16;
      dma16_to_lds(src, lds + 1024 * c);
      chunk += 64;
      if (chunk >= Lay::kSlots) {
        chunk -= Lay::kSlots;
        ++key;
      }
    }
  }
}

// bf16(float(e4m3 code) * scale) for 8 codes (bytes of lo, then hi): the
// FP8 dequantisation rule of the 656-byte row, product in fp32, one
// rounding to bf16 ("为什么 FlashMLA 的解码内核能跑到 660 TFLOPS", section 设计 2).
__device__ inline bf16x8s dequant8(uint32_t lo, uint32_t hi, float sc) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  bf16x8s r;
  r[0] = (__bf16)(a[0] * sc);
  r[1] = (__bf16)(a[1] * sc);
  r[2] = (__bf16)(b[0] * sc);
  r[3] = (__bf16)(b[1] * sc);
  r[4] = (__bf16)(c[0] * sc);
  r[5] = (__bf16)(c[1] * sc);
  r[6] = (__bf16)(d[0] * sc);
  r[7] = (__bf16)(d[1] * sc);
  return r;
}

// FMT: cache row format (0 bf16, 1 the 656-byte FP8 row).  RB 16-row MFMA
// blocks per workgroup (the whole unit: RB = 1 for up to 16 rows, 2 for up
// to 32).  K and V operands read from LDS feed all RB blocks.
template <int FMT, int RB>
__global__ void __launch_bounds__(64 * kSWaves, 1) decode_small_kernel(DecodeArgs a) {
  constexpr int kRows = 16 * RB;
  constexpr int kPitch = SmallLayout<FMT>::kPitch;
  constexpr int kBuf = kSBuf<FMT>;
  constexpr int kCopies = kSCopies<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[kSWaves * 2 * kBuf];
  __shared__ float m_sh[kSWaves][kRows];
  __shared__ float l_sh[kSWaves][kRows];
  static_assert(kRows * kSOPitch * sizeof(float) <= sizeof(kbuf), "the merge buffer reuses the quarter buffers");

  const Shape& s = a.s;
  const int part = blockIdx.x;
  if (part >= a.num_parts) return;
  const int32_t* sc = a.sched + 8 * (size_t)part;
  const int ub = sc[0], kb0 = sc[1], ue = sc[2], ke = sc[3], split0 = sc[4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j16 = lane & 15;  // row within a 16-row block (score and output)
  const int g = lane >> 4;    // lane group: keys 4g .. 4g+3; dims 8g .. of a k-step
  uint8_t* const buf0 = kbuf + wave * 2 * kBuf;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)buf0);
  CopySlots<FMT> slots;
  slots.init(lane);

  for (int u = ub; u < s.units && (u < ue || (u == ue && ke > 0)); ++u) {
    const int L = a.seqlens[u];
    const int nb = (max(L, 0) + kPage - 1) / kPage;
    const int kfirst = (u == ub) ? kb0 : 0;
    const int kend = (u == ue) ? ke : nb;
    if (kfirst >= kend) continue;
    const int seg = (u == ub) ? split0 : 0;
    const int nsplit = a.num_splits[u + 1] - a.num_splits[u];
    cint32s* btc = (cint32s*)(a.block_table + (int64_t)u * s.max_pages);  // scalar loads

    // Q^T operands of rows 16*rb + j16 (dims 32*st + 8*g .. +7; zero for
    // padding rows) and each row's last visible position.
    bf16x8s qf[RB][kSSteps];
    int tlim[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = 16 * rb + j16;
      const bool ok = r < s.rows;
      const uint16_t* qrow = a.q + ((int64_t)u * s.rows + (ok ? r : 0)) * kDqk + 8 * g;
#pragma unroll
      for (int st = 0; st < kSSteps; ++st)
        qf[rb][st] = ok ? *reinterpret_cast<const bf16x8s*>(qrow + 32 * st) : bf16x8s{};
      tlim[rb] = s.is_causal ? L - s.s_q + (ok ? r : 0) / s.h_q : L - 1;
    }
    f32x4s o[RB][32];  // O^T: columns 16*cb + 4*g + v of row 16*rb + j16
    float m[RB], l[RB];
    // Pass 0 takes the probabilities against the first max a row sees.  If a
    // row's scores later climb more than kSLag above it, the wave runs its
    // segment again (pass 1) against the exact maximum found in pass 0, so
    // the output never needs rescaling inside the loop.
    float mstart[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mstart[rb] = -INFINITY;
    for (int pass = 0; pass < 2; ++pass) {
    // The first quarter's copies go out while Q is in flight; Q is waited for
    // here, before the loop, so that no wait for it lands inside the loop
    // (it would also wait for the copies in flight there).
    issue_quarter<FMT>(a.kv, btc[kfirst], wave, kfirst * kPage + kSQuarter * wave, L, lds0, lane, slots);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int st = 0; st < kSSteps; ++st) asm volatile("" ::"v"(qf[rb][st]));

#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) o[rb][cb] = f32x4s{0.0f, 0.0f, 0.0f, 0.0f};
    float mseen[RB];
    bool restart = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m[rb] = mstart[rb];   // reference max of the row (log2 units)
      l[rb] = 0.0f;         // this lane's part of the row sum
      mseen[rb] = -INFINITY;
    }

    int cur = 0;
    for (int kt = kfirst; kt < kend; ++kt) {
      const int tbase = kt * kPage + kSQuarter * wave;  // logical position of key 0
      if (kt + 1 < kend) {
        // the other buffer was last read by the previous quarter's products
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue_quarter<FMT>(a.kv, btc[kt + 1], wave, tbase + kPage, L, lds0 + (cur ^ 1) * kBuf, lane, slots);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopies) : "memory");  // this quarter has landed
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      const uint8_t* qb = buf0 + cur * kBuf;
      cur ^= 1;

      // S^T (16 keys x 16 rows per block); K operands are read kSKAhead
      // steps before their MFMAs, so the LDS latency hides behind the chain.
      f32x4s acc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4s{0.0f, 0.0f, 0.0f, 0.0f};
      // K operand of step st for key j16, dims 32*st + 8*g .. +7: bf16 rows are
      // read as is; FP8 rows give 8 codes (NoPE steps, dequantised with the
      // row's scale of their 128-dim tile) or 8 bf16 RoPE values (steps 16, 17).
      const uint8_t* krow = qb + j16 * kPitch;
      f32x4s ksc = f32x4s{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (FMT == 1) ksc = *reinterpret_cast<const f32x4s*>(krow + 512);
      auto k_raw = [&](int st) -> uint4 {
        if constexpr (FMT == 0) return *reinterpret_cast<const uint4*>(krow + 64 * st + 16 * g);
        if (st < 16) {
          const uint2 c = *reinterpret_cast<const uint2*>(krow + 32 * st + 8 * g);
          return make_uint4(c.x, c.y, 0u, 0u);
        }
        return *reinterpret_cast<const uint4*>(krow + 528 + 64 * (st - 16) + 16 * g);
      };
      auto k_operand = [&](uint4 raw, int st) -> bf16x8s {
        if (FMT == 1 && st < 16) return dequant8(raw.x, raw.y, ksc[st >> 2]);
        return __builtin_bit_cast(bf16x8s, raw);
      };
      uint4 kop[kSKAhead];
#pragma unroll
      for (int i = 0; i < kSKAhead; ++i) kop[i] = k_raw(i);
#pragma unroll
      for (int st = 0; st < kSSteps; ++st) {
        const bf16x8s kcur = k_operand(kop[st % kSKAhead], st);
        if (st + kSKAhead < kSSteps) kop[st % kSKAhead] = k_raw(st + kSKAhead);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kcur, qf[rb][st], acc[rb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      // Online softmax (base 2) of each row over keys 4g .. 4g+3 of this quarter.
      bf16x4s pf[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float x[4];
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x[v] = tbase + 4 * g + v <= tlim[rb] ? acc[rb][v] * s.scale_log2 : -INFINITY;
          mx = fmaxf(mx, x[v]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mseen[rb] = fmaxf(mseen[rb], mx);
        if (m[rb] == -INFINITY) m[rb] = mx;  // first visible keys: output and sum still zero
        restart |= mx > m[rb] + kSLag;
        float p[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[v] = x[v] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[v] - m[rb]);
          l[rb] += p[v];
        }
        pf[rb] = __builtin_bit_cast(bf16x4s, make_uint2(pk_bf16(p[0], p[1]), pk_bf16(p[2], p[3])));
      }

      // O^T += V^T P^T: column block cb; V^T[col][key] for keys 4g .. 4g+3 of
      // column 16*cb + j16: 4 bf16 values, or 4 FP8 codes dequantised with
      // their rows' scales of tile cb / 8.
      const uint8_t* vrow = qb + 4 * g * kPitch;
      f32x4s vsc[4];
      if constexpr (FMT == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) vsc[e] = *reinterpret_cast<const f32x4s*>(vrow + e * kPitch + 512);
      }
      if constexpr (FMT == 0) {
        // One transposing read per column block: in each 16-lane group, lane
        // j loads columns 16*cb + 4*(j % 4) .. +3 of key 4g + j / 4, and lane
        // j16 receives column 16*cb + j16 of keys 4g .. 4g+3, the operand as
        // the MFMA takes it.  Read kSVAhead column blocks ahead.
        const uint8_t* vlane = vrow + (j16 >> 2) * kPitch + 8 * (j16 & 3);
        auto v_raw = [&](int cb) -> i16x4s {
          return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) i16x4s*>(
              (__attribute__((address_space(3))) uint8_t*)(vlane + 32 * cb)));
        };
        i16x4s vop[kSVAhead];  // V^T operands read kSVAhead column blocks ahead
#pragma unroll
        for (int i = 0; i < kSVAhead; ++i) vop[i] = v_raw(i);
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) {
          const bf16x4s vcur = __builtin_bit_cast(bf16x4s, vop[cb % kSVAhead]);
          if (cb + kSVAhead < 32) vop[cb % kSVAhead] = v_raw(cb + kSVAhead);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            o[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vcur, pf[rb], o[rb][cb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // FP8 codes of two column blocks per transposing byte read.  In each
        // 16-lane group, lane j loads 8 codes of key 4g + (j % 8) / 2 at
        // columns 16*cb + 8*(j % 2) + 16*(j / 8) ..; the read hands lane r
        // byte r % 8 of the loads of the group's even lanes (r < 8) or odd
        // lanes (r >= 8), so lane j16 receives keys 4g .. 4g+3 of column
        // 16*cb + j16 (bytes 0..3) and of column 16*(cb + 1) + j16 (bytes
        // 4..7).  Two paired conversions and four multiplies with the keys'
        // scales of the columns' tile per column block.
        const uint8_t* vlane = vrow + ((j16 & 7) >> 1) * kPitch + 8 * (j16 & 1) + 16 * (j16 >> 3);
        auto v_pair = [&](int cp) -> uint2 {  // column blocks 2cp, 2cp + 1
          const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              reinterpret_cast<__attribute__((address_space(3))) i32x2*>(
                  (__attribute__((address_space(3))) uint8_t*)(vlane + 32 * cp)));
          return make_uint2((uint32_t)r[0], (uint32_t)r[1]);
        };
        auto v_deq = [&](uint32_t w, int t) -> bf16x4s {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
          return __builtin_bit_cast(bf16x4s, make_uint2(pk_bf16(lo[0] * vsc[0][t], lo[1] * vsc[1][t]),
                                                         pk_bf16(hi[0] * vsc[2][t], hi[1] * vsc[3][t])));
        };
        uint2 vop[kSVPairAhead];  // pairs of V^T operands read kSVPairAhead pairs ahead
#pragma unroll
        for (int i = 0; i < kSVPairAhead; ++i) vop[i] = v_pair(i);
#pragma unroll
        for (int cp = 0; cp < 16; ++cp) {
          const uint2 r = vop[cp % kSVPairAhead];
          if (cp + kSVPairAhead < 16) vop[cp % kSVPairAhead] = v_pair(cp + kSVPairAhead);
          const int t = cp >> 2;  // the 128-column tile of columns 32cp .. 32cp + 31
          const bf16x4s v0 = v_deq(r.x, t);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            o[rb][2 * cp] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, pf[rb], o[rb][2 * cp], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          const bf16x4s v1 = v_deq(r.y, t);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            o[rb][2 * cp + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v1, pf[rb], o[rb][2 * cp + 1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (!__builtin_amdgcn_ballot_w64(restart)) break;  // wave-uniform
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mstart[rb] = mseen[rb];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // buffer 0 is rewritten by the next pass
    }

    // Merge the four waves' partial results of each row: M = max of the
    // maxima, total = sum of l_w * 2^(m_w - M); each wave's output enters
    // with weight 2^(m_w - M) / total.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l[rb] += __shfl_xor(l[rb], 16);
      l[rb] += __shfl_xor(l[rb], 32);
      if (g == 0) {
        m_sh[wave][16 * rb + j16] = m[rb];
        l_sh[wave][16 * rb + j16] = l[rb];
      }
    }
    __syncthreads();  // every wave is past its last quarter; the buffers are free
    float wgt[RB], lse2[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = 16 * rb + j16;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) M = fmaxf(M, m_sh[w][r]);
      float tot = 0.0f;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) {
        const float mw = m_sh[w][r];
        tot += mw == -INFINITY ? 0.0f : l_sh[w][r] * __builtin_amdgcn_exp2f(mw - M);
      }
      wgt[rb] = (tot > 0.0f && m[rb] != -INFINITY) ? __builtin_amdgcn_exp2f(m[rb] - M) / tot : 0.0f;
      lse2[rb] = tot > 0.0f ? M + log2f(tot) : -INFINITY;
    }
    float* const fbuf = reinterpret_cast<float*>(kbuf);  // [kRows rows][kSOPitch]
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) {  // fixed order: deterministic sums
      if (wave == w) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 32; ++cb) {
            f32x4s* dst =
                reinterpret_cast<f32x4s*>(fbuf + (16 * rb + j16) * kSOPitch + 16 * cb + 4 * g);
            const f32x4s v = o[rb][cb] * wgt[rb];
            *dst = w == 0 ? v : *dst + v;
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      __syncthreads();
    }
    const bool direct = nsplit == 1;
    const int64_t orow0 = direct ? (int64_t)u * s.rows : ((int64_t)a.num_splits[u] + seg) * s.rows;
    uint16_t* const obase = direct ? a.out : a.ws_o;
    for (int row = wave; row < s.rows; row += kSWaves) {
      const f32x4s v0 = *reinterpret_cast<const f32x4s*>(fbuf + row * kSOPitch + 8 * lane);
      const f32x4s v1 = *reinterpret_cast<const f32x4s*>(fbuf + row * kSOPitch + 8 * lane + 4);
      uint4 pk;
      pk.x = (uint32_t)to_bf16_bits(v0[0]) | ((uint32_t)to_bf16_bits(v0[1]) << 16);
      pk.y = (uint32_t)to_bf16_bits(v0[2]) | ((uint32_t)to_bf16_bits(v0[3]) << 16);
      pk.z = (uint32_t)to_bf16_bits(v1[0]) | ((uint32_t)to_bf16_bits(v1[1]) << 16);
      pk.w = (uint32_t)to_bf16_bits(v1[2]) | ((uint32_t)to_bf16_bits(v1[3]) << 16);
      *reinterpret_cast<uint4*>(obase + (orow0 + row) * kDv + 8 * lane) = pk;
    }
    if (wave == 0 && g == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int r = 16 * rb + j16;
        if (r < s.rows) {
          if (direct)
            a.lse[(int64_t)u * s.rows + r] = s.natural ? lse2[rb] * 0.69314718055994531f : lse2[rb];
          else
            a.ws_lse[((int64_t)a.num_splits[u] + seg) * s.rows + r] = lse2[rb];
        }
      }
    }
    __syncthreads();  // the merge buffer is read before the next segment's copies
  }
}

}  // namespace

bool small_decode_applies(const Shape& s) {
  return s.topk == 0 && s.rows <= (s.kv_format == 0 ? kSmallMaxRows : kSmallMaxRowsFp8);
}

hipError_t launch_decode_small(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_parts), block(64 * kSWaves);
  if (a.s.kv_format == 1 && a.s.rows <= 16)
    hipLaunchKernelGGL((decode_small_kernel<1, 1>), grid, block, 0, stream, a);
  else if (a.s.kv_format == 1)
    hipLaunchKernelGGL((decode_small_kernel<1, 2>), grid, block, 0, stream, a);
  else if (a.s.rows <= 16)
    hipLaunchKernelGGL((decode_small_kernel<0, 1>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_small_kernel<0, 2>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
