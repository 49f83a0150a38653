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
// each lane keeps one row's Q (36 bf16x8 MFMA operands) in VGPRs and 256
// fp32 output columns of that row in AGPRs.  One wave per SIMD: all latency
// hiding comes from instruction-level overlap inside the wave.
//
// Per 64-token tile:
//   1. Rows are resolved two tiles ahead: position t -> page = table[t / 64],
//      slot = t % 64 ("Modular Platform 设计文档全景导读", section 四), or for
//      sparse units through the index list first.
//   2. The tile is copied one tile ahead, straight from global memory into
//      LDS (global_load_lds_dwordx4, no registers).  bf16 tiles are double
//      buffered; FP8 rows land in a staging buffer and are dequantised into
//      the bf16 tile: bf16(float(e4m3) * tile scale) (FlashMLA page, section
//      设计 2).  Keys that are not visible are copied from a zero row, so
//      masked keys contribute exactly 0 to P*V.
//   3. S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from
//      LDS, B = 16 dims x 32 rows from registers).  The transposed product
//      leaves each lane holding 32 keys of ONE query row, so the row max and
//      row sum are lane-local plus one exchange with lane^32.
//   4. Online softmax in base 2 with a lazily refreshed running max: the
//      running output is never rescaled in the loop; if some row's max grows
//      by more than 8 the wave parks its partial result in a per-lane flush
//      record and restarts (rare), merged back exactly in the epilogue.
//   5. O^T += V^T P^T with the same MFMA: B = P^T straight from the S^T
//      accumulators (keys permuted consistently on both operands), A = V^T
//      read from the same tile with LDS transpose reads (V = first 512 dims).
// Epilogue: a unit processed in one segment writes bf16 out and lse; a split
// unit writes normalised fp32 partials and their lse to the workspace for the
// combine kernel.
//
// LDS tile layout.  A key row of 576 bf16 is 72 chunks of 16 bytes; chunk c
// of row r sits at chunk position
//     (c / 8) * 512 + r * 8 + ((c + swz(r)) % 8),
//     swz(r) = (r/4)%4 + 4*((r/2)%2).
// Grouping by c / 8 makes every 1 KiB direct copy cover 8 rows x 8 chunks
// (addresses need only shifts and masks).  The LDS has 64 banks of 4 bytes,
// i.e. 16 groups of 16 bytes; a chunk's group is 8*(r%2) + its slot.  The
// rotation keeps both read patterns free of bank conflicts: 16 consecutive
// rows at one chunk (K operand reads, 16 lanes of 16 bytes per cycle) and
// 4 consecutive rows x 4 adjacent chunks (transpose reads of V, 32 lanes of
// 8 bytes per cycle) each touch the 16 groups once.
#include "internal.h"

#include <type_traits>

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kQSteps = kDqk / 16;   // 36 MFMA k-steps over the 576 dims
constexpr float kRescaleThreshold = 8.0f;
constexpr int kTileBytes = kPage * kDqk * 2;  // 73728: 72 chunk groups of 1 KiB
constexpr int kTileLoads = kTileBytes / 1024;  // 72 direct copies, 18 per wave
constexpr int kStageGroups = 6;                // raw FP8 row: 41 chunks in 6 groups of 8
constexpr int kStageBytes = kStageGroups * 8 * 16 * kPage;  // 49152
constexpr int kStageLoads = kStageBytes / 1024;             // 48, 12 per wave

template <typename T>
__device__ inline __attribute__((address_space(3))) T* lds_ptr(const void* p) {
  return (__attribute__((address_space(3))) T*)(p);
}

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

__device__ inline int swz(int r) { return ((r >> 2) & 3) + 4 * ((r >> 1) & 1); }

// Byte offset of 16-byte chunk c of key row r in the tile layout above.
__device__ inline int tile_chunk(int r, int c) {
  return ((c >> 3) * 512 + r * 8 + ((c + swz(r)) & 7)) * 16;
}

// Zero bytes that stand in for the cache row of a key that is not visible.
__device__ __attribute__((aligned(16))) const uint8_t g_zero_row[1168] = {};

// 16 bytes per lane from global memory straight into LDS at
// M0 + 16 * lane (lane layout checked on the device).  Issued from inline
// assembly so the compiler's wait-count bookkeeping does not see it: it
// would otherwise treat every later LDS read as unordered and wait for all
// of them.  Completion is tracked by hand with MLA_WAIT_VMCNT.
__device__ inline void lds_dma16(const void* g, void* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(m0) : "memory", "m0");
}

// Copy of one bf16 tile.  Copy I = 4*t + wave (t < 18) fills chunk group
// g = t/2 of rows 8*(I%8) .. +7: lane L takes row 32*(t%2) + 8*wave + L/8
// and tile position L%8 of that row's group, i.e. source chunk
// 8*g + ((L%8 - swz(row)) mod 8).
__device__ inline void issue_tile_bf16(const uint8_t* __restrict__ kv, const int64_t* rowoff,
                                       uint8_t* buf, int wave, int lane) {
  asm volatile("" : "+v"(lane), "+v"(wave));  // keep the address math inside the tile loop
  const uint8_t* base[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 32 * half + 8 * wave + (lane >> 3);
    const int c8 = ((lane & 7) - swz(row)) & 7;
    const int64_t off = rowoff[row];
    base[half] = (off >= 0 ? kv + off : g_zero_row) + 16 * c8;
  }
#pragma unroll
  for (int t = 0; t < kTileLoads / 4; ++t) {
    lds_dma16(base[t & 1] + 128 * (t >> 1), buf + 1024 * (4 * t + wave));
  }
}

// Copy of 64 raw 656-byte FP8 rows into the staging buffer, laid out as
// [group g < 6][row][8 chunks]: chunk c of a row is at g = c/8, slot c%8
// (chunks 41..47 do not exist and are copied from the zero row).
__device__ inline void issue_tile_fp8(const uint8_t* __restrict__ kv, const int64_t* rowoff,
                                      uint8_t* stage, int wave, int lane) {
  asm volatile("" : "+v"(lane), "+v"(wave));
  const uint8_t* base[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int64_t off = rowoff[32 * half + 8 * wave + (lane >> 3)];
    base[half] = (off >= 0 ? kv + off : g_zero_row) + 16 * (lane & 7);
  }
  const bool tail_real = (lane & 7) == 0;  // chunk 40, the last RoPE chunk
#pragma unroll
  for (int t = 0; t < kStageLoads / 4; ++t) {
    const uint8_t* src = base[t & 1] + 128 * (t >> 1);
    if ((t >> 1) == 5) src = tail_real ? src : g_zero_row;
    lds_dma16(src, stage + 1024 * (4 * t + wave));
  }
}

// Dequantise the staged FP8 rows into the bf16 tile: value =
// bf16(float(e4m3) * scale of its 1x128 tile), RoPE bf16 copied through.
__device__ inline void dequant_stage(const uint8_t* stage, uint8_t* ks) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int key = tid >> 2;
  const int sub = tid & 3;
  auto stage_chunk = [&](int c) -> const uint8_t* {
    return stage + ((c >> 3) * 512 + key * 8 + (c & 7)) * 16;
  };
  const f32x4 scales = *reinterpret_cast<const f32x4*>(stage_chunk(32));
#pragma unroll
  for (int j = 0; j < 8; ++j) {  // code chunk cc = sub + 4*j: dims 16*cc .. 16*cc+15
    const int cc = sub + 4 * j;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage_chunk(cc));
    const float sc = scales[j >> 1];
    u32x4 lo, hi;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(v[w], false);
      const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(v[w], true);
      const bf16x2 p01 = __builtin_convertvector(f32x2{f01[0] * sc, f01[1] * sc}, bf16x2);
      const bf16x2 p23 = __builtin_convertvector(f32x2{f23[0] * sc, f23[1] * sc}, bf16x2);
      const uint32_t w01 = __builtin_bit_cast(uint32_t, p01), w23 = __builtin_bit_cast(uint32_t, p23);
      if (w < 2) { lo[2 * w] = w01; lo[2 * w + 1] = w23; } else { hi[2 * w - 4] = w01; hi[2 * w - 3] = w23; }
    }
    *reinterpret_cast<u32x4*>(ks + tile_chunk(key, 2 * cc)) = lo;
    *reinterpret_cast<u32x4*>(ks + tile_chunk(key, 2 * cc + 1)) = hi;
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // RoPE: bf16 chunks 64..71 <- raw chunks 33..40
    const int i = sub + 4 * j;
    *reinterpret_cast<u32x4*>(ks + tile_chunk(key, 64 + i)) =
        *reinterpret_cast<const u32x4*>(stage_chunk(33 + i));
  }
}

// Workgroup barrier without a memory fence: the compiler's fence would wait
// for every outstanding global->LDS copy, including the next tile's.  LDS
// reads issued before it are complete (their values were consumed); the
// asm memory clobber keeps the compiler from moving LDS accesses across it.
#define MLA_BARRIER_NO_FENCE() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// s_waitcnt with only the vector-memory counter limited to n (n < 64).
#define MLA_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// The score product S^T = K Q^T accumulates in VGPRs.  Written as inline
// assembly because the compiler puts every MFMA accumulator in AGPRs once a
// kernel uses them, and the 256 AGPRs are all taken by the output: score
// accumulators there force the output blocks to be shuffled every tile.
// Back-to-back MFMAs chained through srcC need no wait states; the drain
// below pads the chain before any VALU reads the result (an MFMA result read
// by the VALU needs wait states the compiler cannot see through asm).
__device__ inline void mfma_s_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_s_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_s_drain(f32x16& acc) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" : "+v"(acc));
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
    // zero through the MFMA unit: keeps the accumulators in AGPRs
    o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf16x8{}, bf16x8{}, f32x16{}, 0, 0, 0);
  }
  rec[256] = (had ? rec[256] * a : 0.0f) + l * c;
  rec[257] = M;
  l = 0.0f;
}

template <int FMT, bool SPARSE>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(DecodeArgs a) {
  // bf16: two tile buffers (double buffering).  FP8: one bf16 tile plus a
  // staging buffer for the raw rows of the next tile.  Separate objects let
  // the compiler see that copies into one buffer never alias reads of the
  // other.
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[FMT == 0 ? kTileBytes : kStageBytes];
  __shared__ int64_t rowoff[2][kPage];
  __shared__ uint32_t vmask[2][2];
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
  const int n = lane & 31;    // row within the wave / key-slot group
  const int h = lane >> 5;    // half of the wave
  const int j16 = lane & 15;  // lane within its 16-lane group
  const int r = grp * kRowsPerGroup + wave * 32 + n;  // query row in unit
  const bool row_ok = r < s.rows;
  // per-lane flush record: 256 output columns, l, m
  float* flush = a.ws_flush + ((int64_t)(part * s.groups + grp) * kThreads + threadIdx.x) * kFlushFloats;

  // Lane-constant parts of the LDS operand addresses (tile layout above).
  // K operand, step st: row 32*kb2 + n, chunk 2*st + h.
  int k_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) k_off[i] = n * 128 + 16 * ((2 * i + h + swz(n)) & 7);
  // V^T operand (transpose read), column block cb, key sub-block (kb2, sp,
  // e4): row 32*kb2 + 16*sp + 8*e4 + 4*h + j16/4, chunk 4*cb + 2*(n/16) +
  // (j16%4)/2, byte 8*(j16%2) inside the chunk.  The row rotation depends on
  // e4 but not on kb2 or sp.
  int v_off[2][2];
#pragma unroll
  for (int e4 = 0; e4 < 2; ++e4) {
    const int y = 2 * (n >> 4) + ((j16 & 3) >> 1) + swz(8 * e4 + 4 * h + (j16 >> 2));
#pragma unroll
    for (int p = 0; p < 2; ++p)
      v_off[p][e4] = (8 * e4 + 4 * h + (j16 >> 2)) * 128 + 16 * ((4 * p + y) & 7) + 8 * (j16 & 1);
  }

  for (int u = ub; u < s.units && (u < ue || (u == ue && ke > 0)); ++u) {
    const int b = SPARSE ? u / s.s_q : u;
    const int L = a.seqlens[b];
    const int nb = SPARSE ? (s.topk + kPage - 1) / kPage : (max(L, 0) + kPage - 1) / kPage;
    const int kfirst = (u == ub) ? kb0 : 0;
    const int kend = (u == ue) ? ke : nb;
    if (kfirst >= kend) continue;
    const int seg = (u == ub) ? split0 : 0;
    const int nsplit = a.num_splits[u + 1] - a.num_splits[u];

    // Q operand fragments of this lane's row: dims 16*st + 8*h .. +8
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

    // Row resolution.  Every wave resolves (redundantly, so that all waves
    // issue the same number of memory operations); wave 0 publishes.
    //   res_t:   logical position of key `lane` in tile kt+2
    //   res_off: cache byte offset of key `lane` in tile kt+1 (-1: masked)
    const int32_t* idx_row = SPARSE ? a.indices + (int64_t)u * s.topk : nullptr;
    const int32_t* bt_row = a.block_table + (int64_t)b * s.max_pages;
    auto position = [&](int tile) -> int {  // logical key position, or -1
      const int k = tile * kPage + lane;
      if constexpr (SPARSE) {
        const int t = idx_row[k < s.topk ? k : s.topk - 1];  // always one load
        return (tile < kend && k < s.topk) ? t : -1;
      }
      return tile < kend ? k : -1;
    };
    auto visible = [&](int t) { return t >= 0 && t < L; };
    auto page_of = [&](int t) -> int { return bt_row[visible(t) ? (t >> 6) : 0]; };  // one load
    auto offset_of = [&](int t, int page) -> int64_t {
      return visible(t) ? ((int64_t)page * kPage + (t & 63)) * kRowBytes : (int64_t)-1;
    };
    constexpr int kResolveLoads = SPARSE ? 2 : 1;  // per thread per tile
    auto publish = [&](int slot, int64_t off) {
      if (wave == 0) {
        rowoff[slot][lane] = off;
        const uint64_t bal = __ballot(off >= 0);
        if (lane == 0) { vmask[slot][0] = (uint32_t)bal; vmask[slot][1] = (uint32_t)(bal >> 32); }
      }
    };
    int res_t, pg2 = 0, t3 = -1;
    int64_t res_off;
    __syncthreads();  // the previous segment's last tile is fully consumed
    {
      const int t0 = position(kfirst);
      const int t1 = position(kfirst + 1);
      res_t = position(kfirst + 2);
      publish(0, offset_of(t0, page_of(t0)));
      res_off = offset_of(t1, page_of(t1));
    }
    __syncthreads();
    if constexpr (FMT == 0) {
      issue_tile_bf16(a.kv, rowoff[0], lds0, wave, lane);
    } else {
      issue_tile_fp8(a.kv, rowoff[0], lds1, wave, lane);
      MLA_WAIT_VMCNT(0);
      __syncthreads();
      dequant_stage(lds1, lds0);
    }
    // Everything loaded so far (Q, rows, the first tile) is needed before the
    // first compute anyway.  Waiting here also keeps the compiler from
    // placing its own waits for the Q loads inside the tile loop, where they
    // would stall on the next tile's copies that it cannot see.
    MLA_WAIT_VMCNT(0);

    // One tile: the copy of tile kt+1 and the row resolution of kt+2/kt+3
    // are issued, then tile kt is computed.  CUR is the tile buffer holding
    // tile kt (bf16 path; the loop is unrolled by two so it is static).
    auto tile_step = [&](auto cur_c, int kt) {
      constexpr int cur = decltype(cur_c)::value;
      const bool has_next = kt + 1 < kend;
      // 1. publish the rows of tile kt+1, then start copying it
      publish(cur ^ 1, res_off);
      __syncthreads();  // rows visible; FP8: dequantised tile kt visible
      if (has_next) {
        if constexpr (FMT == 0)
          issue_tile_bf16(a.kv, rowoff[cur ^ 1], cur ? lds0 : lds1, wave, lane);
        else
          issue_tile_fp8(a.kv, rowoff[cur ^ 1], lds1, wave, lane);
      }
      asm volatile("" ::: "memory");  // keep the resolve loads after the copies
      // 2. resolve tile kt+2 (page lookup) and kt+3 (index)
      pg2 = page_of(res_t);
      t3 = position(kt + 3);
      asm volatile("" ::: "memory");
      // 3. bf16: wait for this thread's copies of tile kt (issued one
      //    iteration earlier; the newer copies and resolve loads may stay in
      //    flight), then for every thread's
      if constexpr (FMT == 0) {
        if (has_next) MLA_WAIT_VMCNT(kTileLoads / 4 + kResolveLoads);
        else MLA_WAIT_VMCNT(kResolveLoads);
        MLA_BARRIER_NO_FENCE();
      }
      const uint8_t* ks = (FMT == 0 && cur) ? lds1 : lds0;
      const uint64_t vm = (uint64_t)vmask[cur][0] | ((uint64_t)vmask[cur][1] << 32);
      const int jlim = SPARSE ? 63 : min(63, tlim - kt * kPage);  // keys j <= jlim may count

      // The tile is consumed as two 32-key halves to bound register use.
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        // ---- S^T = K Q^T for keys 32*kb2 .. 32*kb2+31.  K operands are read
        // kPrefetch steps ahead of their MFMA so the LDS latency hides behind
        // the MFMA chain.
        f32x16 sacc;
        {
          const uint8_t* kb = ks + kb2 * 32 * 128;
          auto kload = [&](int st) {
            return *reinterpret_cast<const bf16x8*>(kb + k_off[st & 3] + 8192 * (st >> 2));
          };
          constexpr int kPrefetch = 3;
          bf16x8 kf[kPrefetch];
#pragma unroll
          for (int st = 0; st < kPrefetch; ++st) kf[st] = kload(st);
#pragma unroll
          for (int st = 0; st < kQSteps; ++st) {
            const bf16x8 cur_k = kf[st % kPrefetch];
            if (st + kPrefetch < kQSteps) kf[st % kPrefetch] = kload(st + kPrefetch);
            if (st == 0)
              mfma_s_first(sacc, cur_k, qf[st]);
            else
              mfma_s_acc(sacc, cur_k, qf[st]);
            __builtin_amdgcn_sched_barrier(0);
          }
          mfma_s_drain(sacc);
        }
        // ---- mask, scale, max over this half
        float tmax = -INFINITY;
        const uint32_t lanemask = SPARSE ? (uint32_t)(vm >> (kb2 * 32 + 4 * h)) : 0u;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb2 * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          // dense: visible keys are a prefix of the tile (tail and causal
          // limits folded into jlim); sparse: the per-key validity mask
          const bool ok = SPARSE ? ((lanemask >> (8 * (v >> 2) + (v & 3))) & 1) != 0 : key <= jlim;
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
        // ---- O^T += V^T P^T over 16 column blocks of 32.  Within each
        // 16-lane group, transpose read: lane j points at 4 consecutive
        // columns of one key row (key j/4 of the group's 4) and lane i
        // receives column i of those 4 keys.  k slot (h, e) <-> key
        // 32*kb2 + 16*sp + 8*(e/4) + 4*h + e%4.
        auto load_v = [&](int cb, i16x8* vv) {
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) {
            const uint8_t* vb = ks + 8192 * (cb >> 1) + 4096 * kb2 + 2048 * sp;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(vb + v_off[cb & 1][0]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(vb + v_off[cb & 1][1]));
            vv[sp] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
        };
        i16x8 vbuf[2][2];
        load_v(0, vbuf[0]);
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) {
          if (cb + 1 < 16) load_v(cb + 1, vbuf[(cb + 1) & 1]);
#pragma unroll
          for (int sp = 0; sp < 2; ++sp)
            o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vbuf[cb & 1][sp]),
                                                            pf[sp], o[cb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // 4. finish resolving tile kt+2
      res_off = offset_of(res_t, pg2);
      res_t = t3;
      if constexpr (FMT == 0) {
        MLA_BARRIER_NO_FENCE();  // tile kt consumed: its buffer may be refilled
      } else {
        if (has_next) {
          MLA_WAIT_VMCNT(0);
          __syncthreads();  // staged rows complete, bf16 tile consumed
          dequant_stage(lds1, lds0);
        }
      }
    };
    for (int kt = kfirst; kt < kend; kt += 2) {
      tile_step(std::integral_constant<int, 0>{}, kt);
      if (kt + 1 < kend) tile_step(std::integral_constant<int, 1>{}, kt + 1);
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
