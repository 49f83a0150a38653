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
// split-KV part was given by the scheduler.  The two products split the
// workgroup differently:
//   * scores: wave w owns rows 32w..32w+31; each lane keeps one row's Q (36
//     bf16x8 MFMA operands) in VGPRs and computes S^T = K Q^T, so it holds
//     32 keys of ONE row and the row max / row sum are lane-local plus one
//     exchange with lane^32;
//   * output: wave w owns output columns 128w..128w+127 of all 128 rows
//     (16 fp32 32x32 accumulator blocks in AGPRs) and computes
//     O^T += V^T P^T, with P^T of every row read from LDS.
// The output split makes each wave read only its quarter of V, so the V
// tile crosses the LDS once per workgroup instead of once per wave; V^T
// operands need transposing LDS reads, which move half the bytes of a plain
// 16-byte read, and they were the bottleneck of a row split.
//
// Per 64-token tile (two halves of 32 keys):
//   1. Rows are resolved two tiles ahead: position t -> page = table[t / 64],
//      slot = t % 64 ("Modular Platform 设计文档全景导读", section 四), or for
//      sparse units through the index list first.
//   2. The next tile is copied straight from global memory into LDS
//      (global_load_lds_dwordx4, no registers) while this one is computed.
//      bf16 tiles are double buffered; FP8 rows land in a staging buffer and
//      are dequantised into the bf16 tile: bf16(float(e4m3) * tile scale)
//      (FlashMLA page, section 设计 2).  Keys that are not visible are copied
//      from a zero row, so masked keys contribute exactly 0 to P*V.
//   3. S^T for half 0, then S^T for half 1 with the softmax of half 0
//      interleaved between its MFMAs: mask, scale, max, exp2, row sum, and
//      the bf16 P^T of the half written to LDS.
//   4. Barrier; O^T += V^T P^T for half 0 with the softmax of half 1
//      interleaved; barrier; O^T += V^T P^T for half 1.
//   Online softmax in base 2 with a lazily refreshed running max: the
//   running output is never rescaled in the loop; if some row's max grows by
//   more than 8, every wave parks its partial outputs in a per-lane flush
//   record and restarts them from zero (rare), merged back exactly at the end.
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
// 8 bytes per cycle) each touch the 16 groups once.  Chunk group 8 holds the
// 64 RoPE dims, which only the score product reads; once every wave is past
// the scores of a tile, it holds the P^T of the tile's second half.
//
// P^T layout.  Half a tile of probabilities is 128 rows x 32 keys of bf16,
// 4 chunks per row; chunk c of row r sits at chunk r*4 + (c ^ ((r/4)%4)),
// which keeps 16 consecutive rows at one chunk on 16 distinct bank groups.
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
constexpr int kRopeOffset = 8 * 512 * 16;      // chunk group 8: dims 512..575
constexpr int kStageGroups = 6;                // raw FP8 row: 41 chunks in 6 groups of 8
constexpr int kStageBytes = kStageGroups * 8 * 16 * kPage;  // 49152
constexpr int kStageLoads = kStageBytes / 1024;             // 48, 12 per wave
constexpr int kPHalfBytes = kRowsPerGroup * 32 * 2;         // 8192: P^T of half a tile

template <typename T>
__device__ inline __attribute__((address_space(3))) T* lds_ptr(const void* p) {
  return (__attribute__((address_space(3))) T*)(p);
}

// (x of this lane) combined with (x of lane ^ 32), as two swapped copies.
__device__ inline f32x2 swap_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ inline float wave_max_pair(float x) {
  const f32x2 p = swap_halves(x);
  return fmaxf(p[0], p[1]);
}
__device__ inline float wave_sum_pair(float x) {
  const f32x2 p = swap_halves(x);
  return p[0] + p[1];
}

// Two fp32 values rounded to bf16 (nearest even), lo in bits 0..15, in one
// paired conversion; converting them one by one takes two conversions and a
// pack.
__device__ inline uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
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

// Byte offset of 16-byte chunk c (< 4) of query row r in a P^T half buffer.
__device__ inline int p_chunk(int r, int c) { return (r * 4 + (c ^ ((r >> 2) & 3))) * 16; }

// Zero bytes that stand in for the cache row of a key that is not visible.
__device__ __attribute__((aligned(16))) const uint8_t g_zero_row[1168] = {};

// LDS byte address of a __shared__ object (wave-uniform).
__device__ inline uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane
// (lane layout checked on the device; no instruction offset, which would
// move the LDS destination too).  Issued from inline assembly so the
// compiler's wait-count bookkeeping does not see it: it would otherwise
// treat every later LDS read as unordered and wait for all of them.
// Completion is tracked by hand with MLA_WAIT_VMCNT.
__device__ inline void lds_dma16(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(m0) : "memory", "m0");
}

// Cache byte offset of key `row` of a tile, from the lane that resolved it
// (lane k of every wave holds the offset of key k; -1: not visible).
__device__ inline int64_t row_offset(int64_t off_lane, int row) {
  const int lo = __shfl((int)(uint32_t)off_lane, row);
  const int hi = __shfl((int)(uint32_t)((uint64_t)off_lane >> 32), row);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Copy of one tile, issued one 1 KiB copy at a time so the copies can be
// spread between MFMAs.  bf16: copy I = 4*t + wave (t < 18) fills chunk
// group g = t/2 of rows 8*(I%8) .. +7: lane L takes row 32*(t%2) + 8*wave +
// L/8 and tile position L%8 of that row's group, i.e. source chunk
// 8*g + ((L%8 - swz(row)) mod 8).  FP8: 64 raw 656-byte rows go to the
// staging buffer laid out as [group g < 6][row][8 chunks], chunk c of a row
// at g = c/8, slot c%8 (chunks 41..47 do not exist and are copied from the
// zero row); copy I = 4*t + wave (t < 12) covers group t/2 of the same rows.
template <int FMT>
struct TileCopy {
  static constexpr int kCopies = FMT == 0 ? kTileLoads / 4 : kStageLoads / 4;  // per wave
  const uint8_t* base[2];  // this lane's source for rows 8*wave + L/8 and 32 + 8*wave + L/8
  uint32_t dst;            // LDS address of copy 0 of this wave

  __device__ inline void prepare(const uint8_t* __restrict__ kv, int64_t off_lane, uint32_t buf,
                                 int wave, int lane) {
    asm volatile("" : "+v"(lane), "+v"(wave));  // keep the address math inside the tile loop
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 32 * half + 8 * wave + (lane >> 3);
      const int64_t off = row_offset(off_lane, row);
      const int c8 = FMT == 0 ? ((lane & 7) - swz(row)) & 7 : (lane & 7);
      base[half] = (off >= 0 ? kv + off : g_zero_row) + 16 * c8;
    }
    dst = __builtin_amdgcn_readfirstlane(buf + 1024 * wave);  // wave-uniform
  }
  // Dense tiles are pages: key row r of tile `tile` is row r of physical
  // page `page`, visible while tile*64 + r < vis (vis = the sequence length,
  // or 0 to copy zero rows only).  No cross-lane exchange is needed.
  __device__ inline void prepare_page(const uint8_t* __restrict__ kv, int page, int tile, int vis,
                                      uint32_t buf, int wave, int lane) {
    asm volatile("" : "+v"(lane), "+v"(wave));
    const uint8_t* pbase = kv + (int64_t)page * (kPage * RowBytes<FMT>::value);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 32 * half + 8 * wave + (lane >> 3);
      const int c8 = FMT == 0 ? ((lane & 7) - swz(row)) & 7 : (lane & 7);
      base[half] = (tile * kPage + row < vis ? pbase + row * RowBytes<FMT>::value : g_zero_row) + 16 * c8;
    }
    dst = __builtin_amdgcn_readfirstlane(buf + 1024 * wave);  // wave-uniform
  }
  // Copy t: source chunk group t/2 (128*(t/2) + 16*7 + 16 <= 1168, so a
  // masked row's source stays inside the zero row).
  template <int T>
  __device__ inline void issue(int lane) const {
    const uint8_t* src = base[T & 1] + 128 * (T >> 1);
    if (FMT == 1 && (T >> 1) == 5)  // chunk 40 only; 41..47 from the zero row
      src = (lane & 7) == 0 ? src : g_zero_row + 16 * (lane & 7);
    lds_dma16(src, dst + 4096 * T);
  }
  template <int T = 0>
  __device__ inline void issue_all(int lane) const {
    if constexpr (T < kCopies) {
      issue<T>(lane);
      issue_all<T + 1>(lane);
    }
  }
  // Copies are spread thinly over most of a tile: a CU holds only so many
  // copies in flight at HBM latency, and a burst stalls instruction issue
  // until the first ones return.  bf16: 7 copies in each score chain (after
  // the MFMAs of steps 2, 7, .., 32) and 4 early in the first P*V half
  // (after MFMAs 2, 7, 12, 17).  FP8: rows 0..31 of the stage (even
  // copies) in the first score chain, rows 32..63 (odd copies) in the
  // second, once the dequantisation of the current tile's rows 32..63 has
  // read them; copies 10 and 11 (the RoPE group, which needs the zero-row
  // source) go first, so that source is not held long.
  static constexpr int slot(int phase, int step) {
    if (FMT == 0) {
      if (step % 5 != 2) return -1;
      if (phase < 2) return 7 * phase + step / 5;
      return step / 5 < 4 ? 14 + step / 5 : -1;
    }
    if (phase == 2 || step % 6 != 2) return -1;
    return (2 * (step / 6) + 10) % kCopies + phase;
  }
  // every copy is issued exactly once (phases: 36, 36 and 32 steps)
  static constexpr bool slots_cover_copies() {
    int seen[kCopies] = {};
    for (int phase = 0; phase < 3; ++phase)
      for (int step = 0; step < (phase < 2 ? 36 : 32); ++step) {
        const int t = slot(phase, step);
        if (t >= kCopies) return false;
        if (t >= 0) ++seen[t];
      }
    for (int t = 0; t < kCopies; ++t)
      if (seen[t] != 1) return false;
    return true;
  }
  template <int PHASE, int STEP>
  __device__ inline void issue_at(int lane) const {
    constexpr int t = slot(PHASE, STEP);
    if constexpr (t >= 0) issue<t>(lane);
  }
  // Schedule of dense bf16 tiles, whose P*V runs half a tile behind the
  // scores.  During the first score chain: rows 0..31 of chunk groups 0..7
  // (copies 0, 2, .., 14, after MFMAs 2, 6, .., 30).  During the second:
  // the RoPE group of rows 0..31 (copy 16) first, then rows 32..63 of
  // groups 0..7 (copies 1, 3, .., 15) and their RoPE group (17), after
  // MFMAs 1, 4, .., 28.  Rows 0..31 of the tile are complete once at most
  // kLateCopies copies are in flight; all of it once at most kEarlyCopies
  // (those of the next tile's first chain) are.
  static constexpr int kEarlyCopies = 8;
  static constexpr int kLateCopies = 9;
  static constexpr int slot_split(int phase, int step) {
    if (phase == 0) return (step % 4 == 2 && step / 4 < kEarlyCopies) ? 2 * (step / 4) : -1;
    if (step % 3 != 1 || step / 3 > kLateCopies) return -1;
    const int i = step / 3;
    return i == 0 ? 16 : (i == kLateCopies ? 17 : 2 * i - 1);
  }
  static constexpr bool split_slots_cover_copies() {
    int seen[kCopies] = {};
    for (int phase = 0; phase < 2; ++phase)
      for (int step = 0; step < 36; ++step) {
        const int t = slot_split(phase, step);
        if (t >= kCopies) return false;
        if (t >= 0) ++seen[t];
      }
    for (int t = 0; t < kCopies; ++t)
      if (seen[t] != 1) return false;
    // rows 0..31 (even copies) before rows 32..63, and copy 16 first in the
    // second chain: exactly kLateCopies follow it
    int after16 = 0;
    bool past16 = false;
    for (int step = 0; step < 36; ++step) {
      const int t = slot_split(1, step);
      if (t < 0) continue;
      if (past16) ++after16;
      if (t == 16) past16 = true;
      else if (!past16) return false;
      else if (t % 2 == 0) return false;
    }
    return after16 == kLateCopies;
  }
  template <int PHASE, int STEP>
  __device__ inline void issue_split(int lane) const {
    constexpr int t = slot_split(PHASE, STEP);
    if constexpr (t >= 0) issue<t>(lane);
  }
};

static_assert(TileCopy<0>::slots_cover_copies() && TileCopy<1>::slots_cover_copies(),
              "copy schedule must issue every copy of a tile once");
static_assert(TileCopy<0>::split_slots_cover_copies(),
              "split copy schedule must issue every copy of a tile once, rows 0..31 first");

// f(integral_constant<I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ inline __attribute__((always_inline)) void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Dequantisation of 32 staged FP8 rows (row0 .. row0+31) into the bf16
// tile: value = bf16(float(e4m3) * scale of its 1x128 tile), RoPE bf16
// copied through (FlashMLA page, section 设计 2).  Thread t handles row
// row0 + t/8: code chunks sub + 8j (j < 4, dims 16*(sub+8j) .. +15, scale
// j) and RoPE chunk sub, sub = t%8.  Split into load(), 32 convert parts of
// four VALU instructions each (part p: chunk p/8, half of word (p/2)%4) with
// a store after every 8th, and store_rope(), so the work can be spread
// between MFMAs.
struct HalfDequant {
  u32x4 raw[2];  // code chunks j (in raw[j%2]); chunk j+1 is read while j is converted
  u32x4 rope;
  f32x4 scales;
  u32x4 out;     // bf16 pairs of the half chunk being converted
  const uint8_t* src;
  int row, sub;

  __device__ inline const uint8_t* stage_chunk(int c) const {
    return src + ((c >> 3) * 512 + row * 8 + (c & 7)) * 16;
  }
  __device__ inline void load(const uint8_t* stage, int row0) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    src = stage;
    row = row0 + (tid >> 3);
    sub = tid & 7;
    scales = *reinterpret_cast<const f32x4*>(stage_chunk(32));
    raw[0] = *reinterpret_cast<const u32x4*>(stage_chunk(sub));
  }
  __device__ inline void load_rope() { rope = *reinterpret_cast<const u32x4*>(stage_chunk(33 + sub)); }
  template <int P>
  __device__ inline void convert(uint8_t* ks) {
    constexpr int j = P >> 3, w = (P >> 1) & 3, hw = P & 1;
    if constexpr ((P & 7) == 0 && j + 1 < 4)
      raw[(j + 1) & 1] = *reinterpret_cast<const u32x4*>(stage_chunk(sub + 8 * (j + 1)));
    const float sc = scales[j];
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(raw[j & 1][w], hw != 0);
    const bf16x2 b = __builtin_convertvector(f32x2{f[0] * sc, f[1] * sc}, bf16x2);
    out[2 * (w & 1) + hw] = __builtin_bit_cast(uint32_t, b);
    if constexpr ((P & 3) == 3)  // words 0-1 (bf16 chunk 2cc) or 2-3 (2cc+1) done
      *reinterpret_cast<u32x4*>(ks + tile_chunk(row, 2 * (sub + 8 * j) + (w >> 1))) = out;
  }
  __device__ inline void store_rope(uint8_t* ks) {
    *reinterpret_cast<u32x4*>(ks + tile_chunk(row, 64 + sub)) = rope;  // bf16 chunks 64..71
  }
  __device__ inline void all(const uint8_t* stage, uint8_t* ks, int row0) {
    load(stage, row0);
    static_for<0, 32>([&](auto p) __attribute__((always_inline)) { convert<decltype(p)::value>(ks); });
    load_rope();
    store_rope(ks);
  }
};

// Workgroup barrier without a memory fence: the compiler's fence would wait
// for every outstanding global->LDS copy, including the next tile's.  LDS
// accesses issued before it are complete (lgkmcnt(0)); the asm memory
// clobber keeps the compiler from moving LDS accesses across it.
#define MLA_BARRIER_NO_FENCE() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
// The same barrier with the n most recent LDS reads of this wave still in
// flight.  LDS instructions of a wave complete in issue order, so every LDS
// access issued before those n is complete when the barrier is signalled
// (outstanding scalar loads, which also count here, only make it stricter).
#define MLA_BARRIER_NO_FENCE_KEEP(n) asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(n) : "memory")

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
// The leading s_nop 1 covers a VALU write of an operand register right
// before the MFMA (two wait states), which the compiler cannot see either.
__device__ inline void mfma_s_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_s_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_s_drain(f32x16& acc) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" : "+v"(acc));
}

// S^T for 32 keys (rows of the tile at kb) against this lane's Q row, with
// hook(integral_constant<st>) emitted after the MFMA of k-step st (independent VALU work that
// runs while the matrix core is busy).  K operands are read kKPrefetch steps
// ahead of their MFMA so the LDS latency hides behind the chain.
constexpr int kKPrefetch = 4;
struct KOperands {
  bf16x8 kf[kKPrefetch];
};
__device__ inline bf16x8 k_operand(const uint8_t* kb, const int* k_off, int st) {
  return *reinterpret_cast<const bf16x8*>(kb + k_off[st & 3] + 8192 * (st >> 2));
}
// The first kKPrefetch K operands of a chain (issued early, e.g. right after
// the barrier that makes the tile visible).
__device__ inline void score_chain_begin(KOperands& kp, const uint8_t* kb, const int* k_off) {
#pragma unroll
  for (int st = 0; st < kKPrefetch; ++st) kp.kf[st] = k_operand(kb, k_off, st);
}
template <class Hook>
__device__ inline __attribute__((always_inline)) void score_chain_run(f32x16& acc, KOperands& kp,
                                                                      const uint8_t* kb,
                                                                      const int* k_off,
                                                                      const bf16x8* qf, Hook&& hook) {
  static_for<0, kQSteps>([&](auto st_c) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value;
    const bf16x8 cur_k = kp.kf[st % kKPrefetch];
    if constexpr (st + kKPrefetch < kQSteps) kp.kf[st % kKPrefetch] = k_operand(kb, k_off, st + kKPrefetch);
    if constexpr (st == 0)
      mfma_s_first(acc, cur_k, qf[st]);
    else
      mfma_s_acc(acc, cur_k, qf[st]);
    hook(st_c);
    __builtin_amdgcn_sched_barrier(0);
  });
  mfma_s_drain(acc);
}
template <class Hook>
__device__ inline __attribute__((always_inline)) void score_chain(f32x16& acc, const uint8_t* kb,
                                                                  const int* k_off,
                                                                  const bf16x8* qf, Hook&& hook) {
  KOperands kp;
  score_chain_begin(kp, kb, k_off);
  score_chain_run(acc, kp, kb, k_off, qf, hook);
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

// exp2(x - M) for a merge of partial sums, 0 for a part that saw no key.
__device__ inline float merge_factor(float x, float M) {
  return x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x - M);
}

// Per-half softmax state of a lane (its row, its 16 keys of the half).
struct HalfSoftmax {
  float tmax;   // max of the masked raw scores, then of the scaled row
  float mnew;   // candidate running max
  bool grow;    // the row's max grew past the refresh threshold
  float mo;     // running max before this half's update
  float nmuse;  // minus the reference the probabilities are taken against
  float lh;     // this half's part of the row sum
  float x, e;   // scaled score and probability in flight between steps
  bf16x8 pf[2]; // bf16 probabilities, MFMA operand order
};
constexpr int kSoftmaxSteps = 29;
// P*V reads V^T this many column groups (4 MFMAs each) ahead of its use.
constexpr int kVAhead = 2;

template <int FMT, bool SPARSE>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(DecodeArgs a) {
  // bf16: two tile buffers (double buffering).  FP8: one bf16 tile plus a
  // staging buffer for the raw rows of the next tile.  Separate objects let
  // the compiler see that copies into one buffer never alias reads of the
  // other.
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[FMT == 0 ? kTileBytes : kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[kPHalfBytes];  // P^T of half 0
  // FP8: P^T of half 1 (bf16 keeps it in the tile's RoPE chunk group; FP8
  // overwrites rows 0..31 of the tile, RoPE chunks included, during the
  // second P*V half)
  __shared__ __attribute__((aligned(16))) uint8_t pbuf1[FMT == 1 ? kPHalfBytes : 16];
  __shared__ float mold_s[2][kRowsPerGroup];  // per row: running max before each half's update
  // per half, lane and wave: some row of the wave grew (every lane writes
  // the wave's value to its own word, so the write needs no branch; the
  // four waves' words of lane 0 are read as one 16-byte load)
  __shared__ __attribute__((aligned(16))) uint32_t gflag[2][64][4];
  __shared__ f32x4 oslots[kThreads];  // per-lane slot for copying accumulators
  f32x4* const oslot = &oslots[threadIdx.x];

  const Shape& s = a.s;
  constexpr int kRowBytes = RowBytes<FMT>::value;
  constexpr bool kPipelined = FMT == 0 && !SPARSE;  // tile loop order, below

  // Workgroup -> (part, row group).  Workgroups are dealt round-robin to
  // the 8 XCDs (XCD = id % 8).  XCD x takes the parts
  // [x * per, (x + 1) * per) with all their row groups: the row groups of a
  // part share that XCD's L2 for the tiles they all read, and consecutive
  // parts (the pieces of a split sequence) share it for the sequence's Q.
  // Every kernel argument is fetched in one round of scalar loads here,
  // rather than in a chain of rounds along their first uses.
  asm volatile("" ::"s"(a.q), "s"(a.kv), "s"(a.block_table), "s"(a.seqlens), "s"(a.indices),
               "s"(a.sched), "s"(a.num_splits), "s"(a.num_parts), "s"(a.ws_lse), "s"(a.ws_o),
               "s"(a.ws_flush), "s"(a.out), "s"(a.lse), "s"(s.units), "s"(s.rows), "s"(s.groups),
               "s"(s.s_q), "s"(s.h_q), "s"(s.topk), "s"(s.max_pages), "s"(s.is_causal),
               "s"(s.natural), "s"(s.scale_log2));
  // The schedule, sequence lengths, split counts and (dense) block table
  // are read-only here: scalar loads through the constant address space.
  using cint32 = const __attribute__((address_space(4))) int32_t;
  const int wg = blockIdx.x;
  const int per = (a.num_parts + 7) / 8;
  const int part = (wg % 8) * per + (wg / 8) / s.groups;
  const int grp = (wg / 8) % s.groups;
  if (part >= a.num_parts) return;
  cint32* sc = (cint32*)(a.sched + 8 * (size_t)part);
  const int ub = sc[0], kb0 = sc[1], ue = sc[2], ke = sc[3], split0 = sc[4];
  cint32* seqlens_c = (cint32*)a.seqlens;
  cint32* splits_c = (cint32*)a.num_splits;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;    // row within a 32-row block / key-slot group
  const int h = lane >> 5;    // half of the wave
  const int j16 = lane & 15;  // lane within its 16-lane group
  const int rs = wave * 32 + n;                 // score row of this lane, in the group
  const int r = grp * kRowsPerGroup + rs;       // ... in the unit
  const bool row_ok = r < s.rows;
  // per-lane flush record: 256 output values (block (cb, rb) at 16*(4cb+rb)),
  // the 4 output rows' maxima, the score row's sum and maximum
  // (recomputed where used, so no register holds it through the tile loop)
  const int64_t rec_wg = (int64_t)(part * s.groups + grp) * kThreads;
  auto flush_rec = [&]() -> float* {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    return a.ws_flush + (rec_wg + tid) * kFlushFloats;
  };

  // Lane-constant parts of the LDS operand addresses (tile layout above).
  // K operand, step st: row 32*kb2 + n, chunk 2*st + h.
  int k_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) k_off[i] = n * 128 + 16 * ((2 * i + h + swz(n)) & 7);
  // V^T operand (transpose read), column block cbg, key sub-block (kb2, sp,
  // e4): row 32*kb2 + 16*sp + 8*e4 + 4*h + j16/4, chunk 4*cbg + 2*(n/16) +
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
  // P^T operand / P^T store: row 32*rb + n, chunk 2*sp + h.
  int p_off[2];
#pragma unroll
  for (int sp = 0; sp < 2; ++sp) p_off[sp] = p_chunk(n, 2 * sp + h);

  for (int u = ub; u < s.units && (u < ue || (u == ue && ke > 0)); ++u) {
    // The previous segment is fully consumed (tiles, P^T, epilogue staging
    // in LDS).  No memory fence: Q and the first tile load in parallel below.
    MLA_BARRIER_NO_FENCE();
    const int b = SPARSE ? u / s.s_q : u;
    const int32_t* bt_row = a.block_table + (int64_t)b * s.max_pages;
    const int kfirst = (u == ub) ? kb0 : 0;
    // Q operand fragments of this lane's score row: dims 16*st + 8*h .. +8.
    // Dense: issued first, in flight while the scalar loads below resolve
    // the segment.  Sparse: issued after the first tile's copies, so that
    // the waits of the row resolution do not wait for them.  (The row is
    // recomputed from the thread index: a value kept through the previous
    // segment would come back as a spill reload, whose wait would also
    // wait for these loads.)
    bf16x8 qf[kQSteps];
    auto load_q = [&]() __attribute__((always_inline)) {
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int qr = grp * kRowsPerGroup + (tid >> 6) * 32 + (tid & 31);
      const uint16_t* qrow =
          a.q + ((int64_t)u * s.rows + (qr < s.rows ? qr : 0)) * kDqk + 8 * ((tid >> 5) & 1);
#pragma unroll
      for (int st = 0; st < kQSteps; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st);
    };
    if constexpr (!SPARSE) load_q();
    // One round of scalar loads: the sequence length, the split counts and
    // (dense) the first two pages of the segment, at in-range indices.
    const int L = seqlens_c[b];
    const int splits_u = splits_c[u], splits_u1 = splits_c[u + 1];
    int pg_first = 0, pg_second = 0;
    if constexpr (!SPARSE) {
      cint32* btc = (cint32*)bt_row;
      pg_first = btc[min(kfirst, s.max_pages - 1)];
      pg_second = btc[min(kfirst + 1, s.max_pages - 1)];
    }
    // all four waited for together, before the test below
    asm volatile("" ::"s"(L), "s"(splits_u), "s"(splits_u1), "s"(pg_first), "s"(pg_second));
    const int nb = SPARSE ? (s.topk + kPage - 1) / kPage : (max(L, 0) + kPage - 1) / kPage;
    const int kend = (u == ue) ? ke : nb;
    if (kfirst >= kend) {
      // (uses the Q loads on this path too, so that they are not moved
      // below the test, where they would wait for it)
      if constexpr (!SPARSE) {
      asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]),
                   "v"(qf[6]), "v"(qf[7]), "v"(qf[8]), "v"(qf[9]), "v"(qf[10]), "v"(qf[11]),
                   "v"(qf[12]), "v"(qf[13]), "v"(qf[14]), "v"(qf[15]), "v"(qf[16]), "v"(qf[17]));
      asm volatile("" ::"v"(qf[18]), "v"(qf[19]), "v"(qf[20]), "v"(qf[21]), "v"(qf[22]),
                   "v"(qf[23]), "v"(qf[24]), "v"(qf[25]), "v"(qf[26]), "v"(qf[27]), "v"(qf[28]),
                   "v"(qf[29]), "v"(qf[30]), "v"(qf[31]), "v"(qf[32]), "v"(qf[33]), "v"(qf[34]),
                   "v"(qf[35]));
      }
      continue;
    }
    const int seg = (u == ub) ? split0 : 0;
    const int nsplit = splits_u1 - splits_u;
    const float scale = s.scale_log2 == 0.0f ? 1.0f : fabsf(s.scale_log2);  // > 0
    // last visible position for this row (dense causal; the row is
    // recomputed from the thread index, as for Q above)
    int tlim = L - 1;
    if (!SPARSE && s.is_causal) {
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int qr = grp * kRowsPerGroup + (tid >> 6) * 32 + (tid & 31);
      // query position of the row = floor(qr / h_q), through the host's
      // reciprocal: (qr + 0.5) / h_q lies at least 0.5 / h_q from an
      // integer, far beyond the float rounding error for these sizes
      tlim = L - s.s_q + (int)(((float)qr + 0.5f) * s.inv_h_q);
    }

    float m = -INFINITY;  // running (possibly stale) max of the score row, log2 units
    float l = 0.0f;       // running sum of this lane's half of the keys
    bool flushed = false; // workgroup-uniform: outputs parked in the flush records
    f32x16 o[4][4];       // O^T block (column block cb of this wave, row block rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) o[cb][rb] = f32x16{};

    // Row resolution of sparse tiles.  Every wave resolves all 64 keys of a
    // tile (lane k: key k) and takes the rows it copies from the resolving
    // lanes.
    //   res_t:   logical position of key `lane` in tile kt+2
    //   res_off: cache byte offset of key `lane` in tile kt+1 (-1: masked)
    const int32_t* idx_row = SPARSE ? a.indices + (int64_t)u * s.topk : nullptr;
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
    // Dense: the page of tile kt+1 (wave-uniform, a scalar load issued one
    // tile ahead).  Sparse: the per-key resolution below.
    int pg_next = 0;
    constexpr int kResolveLoads = SPARSE ? 2 : 0;  // vector loads per thread per tile
    int res_t = -1, pg2 = 0, t3 = -1;
    bool t3_ok = false;  // sparse: tile kt+3's slot of this lane holds an index
    int64_t res_off = -1;
    uint64_t vm_cur = 0;  // keys of the current tile that are visible (sparse masking)
    {
      TileCopy<FMT> first;
      if constexpr (SPARSE) {
        const int t0 = position(kfirst);
        const int t1 = position(kfirst + 1);
        res_t = position(kfirst + 2);
        const int64_t off0 = offset_of(t0, page_of(t0));
        res_off = offset_of(t1, page_of(t1));
        vm_cur = __ballot(off0 >= 0);
        first.prepare(a.kv, off0, lds_addr(FMT == 0 ? lds0 : lds1), wave, lane);
      } else {
        // (past the segment's end the second page is not used: its rows
        // are copied from the zero row)
        first.prepare_page(a.kv, pg_first, kfirst, L, lds_addr(FMT == 0 ? lds0 : lds1), wave, lane);
        pg_next = pg_second;
      }
      first.issue_all(lane);
      if constexpr (SPARSE) load_q();
      if constexpr (FMT == 1) {
        MLA_WAIT_VMCNT(0);
        __syncthreads();
        HalfDequant dq;
        dq.all(lds1, lds0, 0);  // rows 32..63 are dequantised during the first score chain
      }
    }
    // Everything loaded so far (Q, rows, the first tile) is needed before the
    // first compute anyway.  Waiting here also keeps the compiler from
    // placing its own waits for the Q loads inside the tile loop, where they
    // would stall on the next tile's copies that it cannot see.
    MLA_WAIT_VMCNT(0);
    // The kernel works with a positive score scale: scale * (q.k) equals
    // |scale| * ((-q).k) for a negative scale (a sign flip of bf16 is exact)
    // and 1 * (0.k) = 0 for a zero scale.
    if (s.scale_log2 <= 0.0f) {
      const uint32_t flip = s.scale_log2 < 0.0f ? 0x80008000u : 0u;
      const uint32_t keep = s.scale_log2 < 0.0f ? 0xffffffffu : 0u;
#pragma unroll
      for (int st = 0; st < kQSteps; ++st) {
        u32x4 w = __builtin_bit_cast(u32x4, qf[st]);
        w = (w & keep) ^ flip;
        qf[st] = __builtin_bit_cast(bf16x8, w);
      }
    }

    // Park this lane's outputs (all 16 blocks) and its score row's sum in
    // the flush record and restart them from zero.  Two partial results
    // with references m1, m2 merge as M = max, each scaled by 2^(m_i - M).
    // Every party to a row applies the same sequence of maxima, so the
    // copies of a row's record maximum stay identical.
    auto flush = [&](int half, float mo_own) __attribute__((always_inline)) {
      float* rec = flush_rec();
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const float mo = mold_s[half][32 * rb + n];
        float M = mo, fa = 0.0f, fc = 1.0f;
        if (flushed) {
          const float mr = rec[256 + rb];
          M = fmaxf(mr, mo);
          fa = merge_factor(mr, M);
          fc = merge_factor(mo, M);
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4* dst = reinterpret_cast<f32x4*>(rec + (4 * cb + rb) * 16 + 4 * q4);
            const f32x4 old = flushed ? *dst * fa : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            *dst = old + acc_quad(o[cb][rb], q4, oslot) * fc;
          }
          // zero through the MFMA unit: keeps the accumulators in AGPRs
          o[cb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf16x8{}, bf16x8{}, f32x16{}, 0, 0, 0);
        }
        rec[256 + rb] = M;
      }
      float M = mo_own, fa = 0.0f, fc = 1.0f;
      if (flushed) {
        const float mr = rec[261];
        M = fmaxf(mr, mo_own);
        fa = merge_factor(mr, M);
        fc = merge_factor(mo_own, M);
      }
      rec[260] = (flushed ? rec[260] * fa : 0.0f) + l * fc;
      rec[261] = M;
      l = 0.0f;
      flushed = true;
    };

    // Per-tile state read by the softmax and P*V steps below.
    uint8_t* ks = lds0;               // buffer of the tile being scored
    uint64_t vm = 0;                  // sparse: visible keys of that tile
    uint32_t lanemask[2] = {0u, 0u};  // sparse: visibility of keys 32*kb2 + 4*h + (0..31)
    int jlim = 63;                    // dense: keys j <= jlim of that tile may count

    // The softmax of half kb2 (raw scores in sc; scores in log2 units are
    // scale * raw with scale > 0), cut into kSoftmaxSteps small steps of a
    // few VALU instructions each.  One step goes between two MFMAs: an
    // MFMA cannot issue while the matrix core is busy, and only the
    // independent instructions that precede it in program order run in
    // the shadow of the previous one.
    //   0..3   mask the half if any of its keys is not visible (step 0),
    //          max of the raw scores
    //   4..9   row max across the lane pair, running max update, publish
    //   9..26  probabilities, software-pipelined so no step waits on a
    //          result of the same step: step 10+v takes the exponential of
    //          score v, the scaled score v+1 and the row sum and bf16
    //          operand of probability v-1
    //   27, 28 store the half's P^T
    auto softmax_step = [&](int kb2, f32x16& sc, HalfSoftmax& hs, int u) __attribute__((always_inline)) {
      if (u == 0) {
        // dense: visible keys are a prefix of the tile (tail and causal
        // limits folded into jlim); sparse: the per-key validity mask
        // (bit 8*(v/4) + v%4 of the lane's mask word is key
        // 32*kb2 + 8*(v/4) + 4*h + v%4)
        bool full;
        if constexpr (SPARSE) {
          uint32_t word = (uint32_t)(vm >> (32 * kb2));
          asm volatile("" : "+s"(word));  // a 32-bit scalar test, not a 64-bit constant compare
          full = word == 0xffffffffu;
        } else {
          full = __builtin_amdgcn_readfirstlane(__all(jlim >= 32 * kb2 + 31) ? 1 : 0) != 0;
        }
        if (!full) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kb2 * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            const bool ok = SPARSE ? ((lanemask[kb2] >> (8 * (v >> 2) + (v & 3))) & 1) != 0 : key <= jlim;
            sc[v] = ok ? sc[v] : -INFINITY;
          }
        }
        hs.tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      } else if (u < 4) {
        hs.tmax = fmaxf(fmaxf(hs.tmax, sc[4 * u]), fmaxf(sc[4 * u + 1], fmaxf(sc[4 * u + 2], sc[4 * u + 3])));
      } else if (u == 4) {
        hs.tmax = wave_max_pair(hs.tmax) * scale;  // scale > 0 keeps the max; -inf stays -inf
      } else if (u == 5) {
        hs.mnew = fmaxf(m, hs.tmax);
        // A row that has seen no visible key yet holds O = 0 and l = 0:
        // it adopts the new max for free.
        if (m == -INFINITY) m = hs.mnew;
      } else if (u == 6) {
        hs.grow = hs.mnew > m + kRescaleThreshold;
        hs.mo = m;
        if (hs.grow) m = hs.mnew;
      } else if (u == 7) {
        hs.nmuse = (m == -INFINITY) ? 0.0f : -m;
        hs.lh = 0.0f;
      } else if (u == 8) {
        // the row index is recomputed here rather than kept in a register
        // (both lanes of a row pair hold the same maximum and write it)
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        mold_s[kb2][((tid >> 6) << 5) + (tid & 31)] = hs.mo;
      } else if (u == 9) {
        const bool any_grow = __ballot(hs.grow) != 0;
        int tid = threadIdx.x;  // (address recomputed, not kept in a register)
        asm volatile("" : "+v"(tid));
        gflag[kb2][tid & 63][tid >> 6] = any_grow ? 1u : 0u;
        hs.x = __builtin_fmaf(sc[0], scale, hs.nmuse);
      } else if (u < 27) {
        const int v = u - 10;  // 0..16
        float e = 0.0f;
        if (v < 16) e = __builtin_amdgcn_exp2f(hs.x);
        if (v < 15) hs.x = __builtin_fmaf(sc[v + 1], scale, hs.nmuse);
        if (v > 0) {
          hs.lh += hs.e;
          // keeps the add in this step: otherwise the compiler sinks all 16
          // into one dependent chain at the row-sum update, with every
          // probability held in a register until then
          asm volatile("" : "+v"(hs.lh));
          hs.pf[(v - 1) >> 3][(v - 1) & 7] = (__bf16)hs.e;
        }
        hs.e = e;
      } else if (u < 29) {
        const int sp = u - 27;
        uint8_t* pb = kb2 == 0 ? pbuf : (FMT == 1 ? pbuf1 : ks + kRopeOffset);
        // the address is recomputed from the thread index, not kept in a
        // register through the tile loop
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int pw = tid >> 6, pn = tid & 31, ph = (tid >> 5) & 1;
        *reinterpret_cast<bf16x8*>(pb + 2048 * pw + p_chunk(pn, 2 * sp + ph)) = hs.pf[sp];
      }
    };

    // Whether some row of the workgroup grew in half kb2 (readable once
    // the barrier after that half's softmax has passed): the LDS words, and
    // the wave-uniform answer.  Reading them well before the P*V half that
    // depends on them keeps the LDS round trip off its start.
    auto grew_word = [&](int kb2) -> u32x4 { return *reinterpret_cast<const u32x4*>(gflag[kb2][0]); };
    auto grew_any = [&](u32x4 w) -> bool {
      return __builtin_amdgcn_readfirstlane(w[0] | w[1] | w[2] | w[3]) != 0;
    };
    // Before the P*V of a half: if any wave saw a row grow, every wave
    // parks its outputs; then this lane's row sum takes the half's part.
    auto settle = [&](int kb2, float mo, float lh, bool grew) __attribute__((always_inline)) {
      if (grew) flush(kb2, mo);
      l += lh;
    };

    // O^T += V^T P^T for half kb2 of the tile in buffer vt, over this wave's
    // 4 column blocks and the 4 row blocks: 8 groups g = (key step sp = g/4, column block cb = g%4)
    // of 4 MFMAs, hook(j) after MFMA j (32 of them).  Within each 16-lane
    // group, transpose read: lane j points at 4 consecutive columns of one
    // key row (key j/4 of the group's 4) and lane i receives column i of
    // those 4 keys.  k slot (h, e) <-> key 32*kb2 + 16*sp + 8*(e/4) + 4*h +
    // e%4.  V^T operands rotate through kVAhead + 1 registers; the first
    // kVAhead groups' operands are tile data and are read before the
    // barrier that publishes the half's P^T (pv_prefetch).
    auto load_v = [&](const uint8_t* vt, int kb2, int g) {
      const int sp = g >> 2, cb = g & 3;
      const uint8_t* vb = vt + 8192 * (2 * wave + (cb >> 1)) + 4096 * kb2 + 2048 * sp;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(vb + v_off[cb & 1][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(vb + v_off[cb & 1][1]));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int kVRegs = kVAhead + 1;
    constexpr int kVPrefetchReads = 2 * kVAhead;  // LDS reads issued by pv_prefetch
    auto pv_prefetch = [&](const uint8_t* vt, int kb2, bf16x8* vf) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < kVAhead; ++g) vf[g] = load_v(vt, kb2, g);
    };
    auto load_p = [&](const uint8_t* pb, int sp, int rb) {
      return *reinterpret_cast<const bf16x8*>(pb + 2048 * rb + p_off[sp]);
    };
    // Every first operand of a half: V^T as pv_prefetch, and the P^T blocks
    // of the first key step (once the half's P^T is visible).
    constexpr int kPVBeginReads = kVPrefetchReads + 4;
    auto pv_begin = [&](const uint8_t* vt, int kb2, const uint8_t* pb, bf16x8* vf, bf16x8* pfr)
        __attribute__((always_inline)) {
      pv_prefetch(vt, kb2, vf);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) pfr[rb] = load_p(pb, 0, rb);
    };
    auto pv_run = [&](int kb2, const uint8_t* vt, const uint8_t* pb, bf16x8* vf, bf16x8* pfr,
                      auto&& pre, auto&& hook) __attribute__((always_inline)) {
      pre();  // runs while the first operands are in flight
      static_for<0, 8>([&](auto g_c) __attribute__((always_inline)) {
        constexpr int g = decltype(g_c)::value;
        constexpr int cb = g & 3;
        if constexpr (g + kVAhead < 8) vf[(g + kVAhead) % kVRegs] = load_v(vt, kb2, g + kVAhead);
        static_for<0, 4>([&](auto rb_c) __attribute__((always_inline)) {
          constexpr int rb = decltype(rb_c)::value;
          o[cb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[g % kVRegs], pfr[rb], o[cb][rb], 0, 0, 0);
          // the second key step's P^T block rb, right after its last use
          if constexpr (g == 3) pfr[rb] = load_p(pb, 1, rb);
          hook(std::integral_constant<int, 4 * g + rb>{});
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    };
    auto pv_half = [&](int kb2, const uint8_t* vt, const uint8_t* pb, bf16x8* vf, auto&& pre,
                       auto&& hook) __attribute__((always_inline)) {
      bf16x8 pfr[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) pfr[rb] = load_p(pb, 0, rb);
      pv_run(kb2, vt, pb, vf, pfr, pre, hook);
    };

    // Dense bf16 tiles run one P*V half behind the scores, so that both
    // softmax halves sit between P*V MFMAs (register-fed, with room for
    // VALU work) rather than between score MFMAs (which wait on LDS):
    //   B1 | scores 0 of kt (copies: rows 0..31 of kt+1)
    //      | P*V 1 of kt-1 + softmax 0 of kt
    //   B2 | scores 1 of kt (copies: RoPE group and rows 32..63 of kt+1)
    //   B3 | P*V 0 of kt + softmax 1 of kt (its P^T into kt's RoPE group)
    // The copies of rows 32..63 and of the RoPE group overwrite what P*V 1
    // of kt-1 reads, so they wait for B2; they need to land only by B1 / B2
    // of kt+1.
    if constexpr (kPipelined) {
      const __attribute__((address_space(4))) int32_t* bt_const =
          (const __attribute__((address_space(4))) int32_t*)bt_row;  // scalar loads
      float prev_mo = -INFINITY, prev_lh = 0.0f;  // softmax 1 of tile kt-1, for its P*V
      bf16x8 vf[kVRegs];
      for (int kt = kfirst; kt < kend; ++kt) {
        const bool odd = ((kt - kfirst) & 1) != 0;
        // 1. rows 0..31 (with their RoPE chunks) of tile kt have landed:
        //    only the copies issued after that RoPE group may still be in
        //    flight.  Every wave is done with P*V 0 of tile kt-1 (P^T half 0
        //    and its maxima are free); softmax 1 of tile kt-1 is published.
        MLA_WAIT_VMCNT(TileCopy<0>::kLateCopies);
        MLA_BARRIER_NO_FENCE();
        ks = odd ? lds1 : lds0;
        const uint8_t* kprev = odd ? lds0 : lds1;
        // the chain's first K reads go out before the copy address arithmetic
        KOperands kp;
        score_chain_begin(kp, ks, k_off);
        __builtin_amdgcn_sched_barrier(0);
        const u32x4 g1 = grew_word(1);  // softmax 1 of tile kt-1 (published by B1)
        __builtin_amdgcn_sched_barrier(0);
        TileCopy<0> next;
        const uint32_t next_buf = lds_addr(odd ? lds0 : lds1);
        next.prepare_page(a.kv, pg_next, kt + 1, kt + 1 < kend ? L : 0, next_buf, wave, lane);
        pg_next = bt_const[min(kt + 2, nb - 1)];  // for the next tile
        jlim = min(63, tlim - kt * kPage);
        const bool grew1 = grew_any(g1);

        HalfSoftmax hs0, hs1;
        f32x16 sacc0, sacc1;
        bf16x8 pfr[4];
        // P*V 1 of tile kt-1 reads operands published at B1: its first reads
        // go out during the last MFMAs of the chain (for the first tile of
        // a segment they read the idle buffer and are not used)
        score_chain_run(sacc0, kp, ks, k_off, qf, [&](auto st_c) __attribute__((always_inline)) {
          constexpr int st = decltype(st_c)::value;
          next.template issue_split<0, st>(lane);
          if constexpr (st == kQSteps - 3) pv_begin(kprev, 1, kprev + kRopeOffset, vf, pfr);
        });
        if (kt > kfirst) {
          pv_run(1, kprev, kprev + kRopeOffset, vf, pfr, [&] { settle(1, prev_mo, prev_lh, grew1); },
                 [&](auto j_c) __attribute__((always_inline)) {
                   constexpr int j = decltype(j_c)::value;
                   if constexpr (j < kSoftmaxSteps) softmax_step(0, sacc0, hs0, j);
                 });
        } else {
          static_for<0, kSoftmaxSteps>([&](auto u_c) __attribute__((always_inline)) {
            softmax_step(0, sacc0, hs0, decltype(u_c)::value);
          });
        }
        // 2. half 0's P^T and maxima visible; the other buffer (tile kt-1)
        //    is free; rows 32..63 of tile kt have landed (only the copies
        //    issued during scores 0 may still be in flight)
        MLA_WAIT_VMCNT(TileCopy<0>::kEarlyCopies);
        MLA_BARRIER_NO_FENCE();
        const u32x4 g0 = grew_word(0);  // softmax 0 of tile kt (published by B2)
        __builtin_amdgcn_sched_barrier(0);
        bool grew0 = false;
        score_chain(sacc1, ks + 32 * 128, k_off, qf, [&](auto st_c) __attribute__((always_inline)) {
          constexpr int st = decltype(st_c)::value;
          next.template issue_split<1, st>(lane);
          if constexpr (st == 6) grew0 = grew_any(g0);
        });
        // 3. every wave is past the scores of tile kt: its RoPE chunk group
        //    takes half 1's P^T.  (Half 0's P^T is visible since B2, so
        //    all first operands are read before this barrier.)
        pv_begin(ks, 0, pbuf, vf, pfr);
        MLA_BARRIER_NO_FENCE_KEEP(kPVBeginReads);
        pv_run(0, ks, pbuf, vf, pfr, [&] { settle(0, hs0.mo, hs0.lh, grew0); },
                [&](auto j_c) __attribute__((always_inline)) {
                  constexpr int j = decltype(j_c)::value;
                  if constexpr (j < kSoftmaxSteps) softmax_step(1, sacc1, hs1, j);
                });
        prev_mo = hs1.mo;
        prev_lh = hs1.lh;
      }
      // P*V 1 of the last tile
      pv_prefetch(ks, 1, vf);
      MLA_BARRIER_NO_FENCE_KEEP(kVPrefetchReads);
      pv_half(1, ks, ks + kRopeOffset, vf, [&] { settle(1, prev_mo, prev_lh, grew_any(grew_word(1))); }, [](auto) {});
    }

    // One tile: the copy of tile kt+1 and the row resolution of kt+2/kt+3
    // are issued, then tile kt is computed.  bf16 tiles alternate between
    // the two buffers, starting with lds0.
    for (int kt = kfirst; kt < kend && !kPipelined; ++kt) {
      const bool odd = ((kt - kfirst) & 1) != 0;
      // 1. tile kt has landed (this thread's copies, then everyone's); every
      //    wave is done with tile kt-1, its buffer and both P^T halves
      if constexpr (FMT == 0) MLA_WAIT_VMCNT(kResolveLoads);
      MLA_BARRIER_NO_FENCE();
      vm = vm_cur;
      // Sparse: address of tile kt+2's page-table entry.  res_t was loaded
      // during the previous tile; using it here, where only that tile's two
      // resolve loads can still be in flight, keeps the wait the compiler
      // places for it from also waiting for this tile's copies.  (Dense
      // positions are arithmetic: no wait, no early address needed.)
      int pg_idx = 0;
      if constexpr (SPARSE) {
        pg_idx = visible(res_t) ? (res_t >> 6) : 0;
        asm volatile("" : "+v"(pg_idx));
      }
      // 2. sources of tile kt+1's copy; the copies themselves are issued
      //    between the MFMAs of the first score chain (res_off is -1 for
      //    every key past the unit's last tile)
      TileCopy<FMT> next;
      const uint32_t next_buf = lds_addr(FMT == 1 ? lds1 : (odd ? lds0 : lds1));
      if constexpr (SPARSE) {
        next.prepare(a.kv, res_off, next_buf, wave, lane);
        vm_cur = __ballot(res_off >= 0);
      } else {
        // tile kt+1 past the segment: zero rows
        next.prepare_page(a.kv, pg_next, kt + 1, kt + 1 < kend ? L : 0, next_buf, wave, lane);
        pg_next = bt_row[min(kt + 2, nb - 1)];  // for the next tile; a scalar load
      }

      ks = (FMT == 0 && odd) ? lds1 : lds0;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) lanemask[kb2] = SPARSE ? (uint32_t)(vm >> (kb2 * 32 + 4 * h)) : 0u;
      jlim = SPARSE ? 63 : min(63, tlim - kt * kPage);

      HalfSoftmax hs0, hs1;
      f32x16 sacc0, sacc1;
      // 3. scores of half 0; scores of half 1 with the softmax of half 0
      // Issued unconditionally: after a unit's last tile every key of "tile
      // kt+1" resolves to the zero row, so the copies fill the free buffer
      // with zeros, which nothing reads; the next unit starts with a barrier
      // that waits for them.  No branch keeps the chain's registers simple.
      // FP8: rows 32..63 of tile kt are dequantised from the stage between
      // the MFMAs of the first chain, which reads rows 0..31 only (they were
      // dequantised during the previous tile's second P*V half)
      HalfDequant dqh;
      score_chain(sacc0, ks, k_off, qf, [&](auto st_c) __attribute__((always_inline)) {
        constexpr int st = decltype(st_c)::value;
        next.template issue_at<0, st>(lane);
        if constexpr (FMT == 1) {
          if constexpr (st == 0) dqh.load(lds1, 32);
          if constexpr (st >= 1 && st <= 32) dqh.template convert<st - 1>(ks);
          if constexpr (st == 20) dqh.load_rope();
          if constexpr (st == 34) dqh.store_rope(ks);
        }
      });
      // FP8: rows 32..63 of tile kt are in place; the stage rows they came
      // from are free for the next tile's copies
      if constexpr (FMT == 1) MLA_BARRIER_NO_FENCE();
      score_chain(sacc1, ks + 32 * 128, k_off, qf, [&](auto st_c) __attribute__((always_inline)) {
        constexpr int st = decltype(st_c)::value;
        next.template issue_at<1, st>(lane);
        if constexpr (st < kSoftmaxSteps) softmax_step(0, sacc0, hs0, st);
      });

      // 4. half 0's P^T and maxima visible; every wave is past the scores,
      //    so the RoPE chunk group is free for half 1's P^T
      bf16x8 vf[kVRegs];
      pv_prefetch(ks, 0, vf);
      MLA_BARRIER_NO_FENCE_KEEP(kVPrefetchReads);
      pv_half(0, ks, pbuf, vf, [&] { settle(0, hs0.mo, hs0.lh, grew_any(grew_word(0))); }, [&](auto j_c) __attribute__((always_inline)) {
        constexpr int j = decltype(j_c)::value;
        next.template issue_at<2, j>(lane);
        if constexpr (j < kSoftmaxSteps) softmax_step(1, sacc1, hs1, j);
      });
      // resolve kt+2 (page lookup) and kt+3 after the last copy: the wait at
      // the top of the next tile counts these loads as the only ones newer
      // than the copies
      asm volatile("" ::: "memory");
      if constexpr (SPARSE) {
        pg2 = bt_row[pg_idx];
        // The raw index of tile kt+3.  Its only reader until the end of the
        // tile is an empty asm statement there, so the compiler's wait for
        // it lands at the end of the tile; a select next to the load would
        // be waited for here, and with it every copy issued before it.
        // Validity is applied at the end of the tile.
        const int k = (kt + 3) * kPage + lane;
        t3 = idx_row[k < s.topk ? k : s.topk - 1];
        t3_ok = kt + 3 < kend && k < s.topk;
      }
      asm volatile("" ::: "memory");
      // FP8: this thread's copies of tile kt+1 are complete (only the
      // resolve loads may be newer), so after the barrier every staged row
      // is visible to the dequantisation below
      if constexpr (FMT == 1) MLA_WAIT_VMCNT(kResolveLoads);
      pv_prefetch(ks, 1, vf);
      MLA_BARRIER_NO_FENCE_KEEP(kVPrefetchReads);  // half 1's P^T and maxima visible
      if constexpr (FMT == 0) {
        pv_half(1, ks, ks + kRopeOffset, vf, [&] { settle(1, hs1.mo, hs1.lh, grew_any(grew_word(1))); }, [](auto) {});
      } else {
        // rows 0..31 of tile kt are no longer read (half 0 is done): the
        // staged rows 0..31 of tile kt+1 are dequantised into them between
        // the MFMAs of half 1 (after a unit's last tile they are zero rows
        // written into a tile nothing reads any more)
        HalfDequant dq;
        pv_half(1, ks, pbuf1, vf, [&] { dq.load(lds1, 0); settle(1, hs1.mo, hs1.lh, grew_any(grew_word(1))); },
                [&](auto j_c) __attribute__((always_inline)) {
                  dq.template convert<decltype(j_c)::value>(ks);
                  if constexpr (decltype(j_c)::value == 24) dq.load_rope();
                  if constexpr (decltype(j_c)::value == 31) dq.store_rope(ks);
                });
      }

      // 5. finish resolving tile kt+2
      if constexpr (SPARSE) {
        res_off = offset_of(res_t, pg2);
        asm volatile("" : "+v"(t3));
        res_t = t3_ok ? t3 : -1;
      }
    }

    // ---- epilogue.  The score-row owner folds in its flush record and
    // publishes the row's output factors; every wave then normalises and
    // stores its column blocks.
    float fa = 0.0f, fc = 1.0f, mfin = m, lfin = l;
    float* rec = flush_rec();
    if (flushed) {
      const float mf = rec[261];
      mfin = fmaxf(mf, m);
      fa = merge_factor(mf, mfin);
      fc = merge_factor(m, mfin);
      lfin = rec[260] * fa + l * fc;
    }
    const float ltot = wave_sum_pair(lfin);
    const float lse2 = ltot > 0.0f ? mfin + log2f(ltot) : -INFINITY;
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    // half 0's P^T buffer is free: every wave is past the last tile's final barrier
    f32x2* epi = reinterpret_cast<f32x2*>(pbuf);
    if (h == 0) epi[rs] = f32x2{fc * inv, fa * inv};
    MLA_BARRIER_NO_FENCE();
    const bool direct = nsplit == 1;
    // Output rows and columns come from the thread index again rather than
    // from values kept through the tile loop: those come back as spill
    // reloads, and a reload waits for every store issued before it.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int ow = tid >> 6, on = tid & 31, oh = (tid >> 5) & 1;
    const int64_t orow0 = direct ? (int64_t)u * s.rows : ((int64_t)a.num_splits[u] + seg) * s.rows;
    // Rows go out through LDS so that each store writes one whole 1 KiB
    // output row: per row block, every wave writes its 32 x 128 slice
    // (normalised, bf16) into a staging area of the last tile's buffer (free
    // after the barrier above; two areas in turn), then wave w stores rows
    // 8w .. 8w+7 of the block.  16-byte chunk c of staged row r sits at chunk
    // c ^ (r % 16), which spreads both the slice writes and the row reads
    // over all banks.
    uint16_t* const obase = direct ? a.out : a.ws_o;  // final rows or bf16 split partials
    auto store_rows = [&](auto flushed_c) __attribute__((always_inline)) {
      constexpr bool kFlushed = decltype(flushed_c)::value;
      const float* recp = flush_rec();
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        uint8_t* const stg = ks + 32768 * (rb & 1);
        {
          const f32x2 f = epi[32 * rb + on];
          f32x4 fr[16];  // the row block's parked values, loaded before use
          if constexpr (kFlushed) {
#pragma unroll
            for (int k = 0; k < 16; ++k)
              fr[k] = *reinterpret_cast<const f32x4*>(recp + (4 * (k >> 2) + rb) * 16 + 4 * (k & 3));
          }
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              f32x4 v = f32x4{o[cb][rb][4 * q4], o[cb][rb][4 * q4 + 1], o[cb][rb][4 * q4 + 2],
                              o[cb][rb][4 * q4 + 3]} * f[0];
              if constexpr (kFlushed) v += fr[4 * cb + q4] * f[1];
              const uint32_t w0 = pk_bf16(v[0], v[1]);
              const uint32_t w1 = pk_bf16(v[2], v[3]);
              const int chunk = (16 * ow + 4 * cb + q4) ^ (on & 15);  // columns 128ow + 32cb + 8q4 ..
              *reinterpret_cast<uint2*>(stg + on * 1024 + chunk * 16 + 8 * oh) = make_uint2(w0, w1);
            }
          }
        }
        MLA_BARRIER_NO_FENCE();  // the block is staged; the other area is free again
        const int ln = tid & 63;
        const int ows = __builtin_amdgcn_readfirstlane(ow);  // wave-uniform row tests below
        const int ro8 = grp * kRowsPerGroup + 32 * rb + 8 * ows;  // first output row in the unit
        auto row_chunk = [&](int i) {
          const int rr = 8 * ows + i;  // row in the block
          return *reinterpret_cast<const uint4*>(stg + rr * 1024 + ((ln ^ (rr & 15)) * 16));
        };
        if (ro8 + 8 <= s.rows) {  // all 8 rows exist: every read before any store
          uint4 rowv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) rowv[i] = row_chunk(i);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint4*>(obase + (orow0 + ro8 + i) * kDv + 8 * ln) = rowv[i];
        } else {
          for (int i = 0; i < 8 && ro8 + i < s.rows; ++i) {
            const uint4 v = row_chunk(i);
            *reinterpret_cast<uint4*>(obase + (orow0 + ro8 + i) * kDv + 8 * ln) = v;
          }
        }
      }
    };
    if (flushed) store_rows(std::integral_constant<bool, true>{});
    else store_rows(std::integral_constant<bool, false>{});
    if (row_ok && h == 0) {
      const int64_t row = (int64_t)u * s.rows + r;
      if (direct)
        a.lse[row] = s.natural ? lse2 * 0.69314718055994531f : lse2;
      else
        a.ws_lse[((int64_t)a.num_splits[u] + seg) * s.rows + r] = lse2;
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
