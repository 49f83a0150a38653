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
//      (FlashMLA page, section 设计 2).  Keys that are not visible are
//      masked to -inf before the softmax; their rows are copied from a zero
//      row (FP8, sparse) or from the tile's last visible row (dense bf16), so
//      they hold finite values and contribute exactly 0 to P*V.
//   3. S^T for half 0, then S^T for half 1 with the softmax of half 0
//      interleaved between its MFMAs: mask, scale, max, exp2, row sum, and
//      the bf16 P^T of the half written to LDS.
//   4. Barrier; O^T += V^T P^T for half 0 with the softmax of half 1
//      interleaved; barrier; O^T += V^T P^T for half 1.
//   The dense bf16 kernel runs P*V half a tile behind the scores (the
//   schedule is spelled out at its tile loop).
//   Online softmax in base 2 against a fixed reference: a row's
//   probabilities are taken against the first finite maximum the row sees,
//   so the running output is never rescaled in the loop (the correction
//   factor of section 六 is 1 throughout).  Probabilities may exceed 1 by up
//   to 2^kRestartMargin, far inside fp32.  If some row of the workgroup climbs
//   further, the workgroup runs its segment again against the exact row
//   maxima the first pass found (rare: scores that grow along the sequence).
// Epilogue: a unit processed in one segment writes bf16 out and lse; a split
// unit writes its normalised bf16 partial and fp32 lse to the workspace for
// the combine kernel.
//
// LDS tile layout of the FP8 and sparse kernels (the dense bf16 layout is
// described at nope_row below).  A key row of 576 bf16 is 72 chunks of 16
// bytes; chunk c of row r sits at chunk position
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
constexpr int kTileBytes = kPage * kDqk * 2;  // 73728: 72 chunk groups of 1 KiB
constexpr int kTileLoads = kTileBytes / 1024;  // 72 direct copies, 18 per wave
constexpr int kStageGroups = 6;                // raw FP8 row: 41 chunks in 6 groups of 8
constexpr int kStageBytes = kStageGroups * 8 * 16 * kPage;  // 49152
constexpr int kStageLoads = kStageBytes / 1024;             // 48, 12 per wave
constexpr int kPHalfBytes = kRowsPerGroup * 32 * 2;         // 8192: P^T of half a tile
// Dense bf16 tile (the pipelined kernel).  The 1 KiB NoPE part of a key
// row is copied by one contiguous copy; rows sit at a 1040-byte pitch in
// groups of 16, row q of a group in slot nope_slot(q); the RoPE parts (64
// rows x 128 B) follow in the 16-byte chunk rotation of the tile layout.
constexpr int kNopeSlot = 1040;
constexpr int kNopeGroup = 16 * kNopeSlot;                  // 16640
constexpr int kDenseRope = 4 * kNopeGroup;                  // 66560
constexpr int kDenseTileBytes = kDenseRope + kPage * 128;   // 74752

template <typename T>
__device__ inline __attribute__((address_space(3))) T* lds_ptr(const void* p) {
  return (__attribute__((address_space(3))) T*)(p);
}

// (x of this lane) combined with (x of lane ^ 32), as two swapped copies.
__device__ inline f32x2 swap_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Maxima of scores in plain v_max3/v_max instructions: fmaxf would first
// quiet possible signalling NaNs (an extra instruction per operand), which
// MFMA results never are.
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float wave_max_pair(float x) {
  const f32x2 p = swap_halves(x);
  return max2f(p[0], p[1]);
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

// Dense layout: byte offset of the NoPE part of key row r, and of RoPE chunk
// c (< 8) of row r.  Slot s(q) = 4*(q%4) + q/4 puts the 16 rows of a group
// on 16 distinct bank groups (K operand reads: 16 rows at one chunk) and any
// 4 consecutive rows 4 bank groups apart (transposed V reads: 4 rows x 4
// adjacent chunks).
__device__ inline int nope_slot(int q) { return 4 * (q & 3) + (q >> 2); }
__device__ inline int nope_row(int r) { return kNopeGroup * (r >> 4) + kNopeSlot * nope_slot(r & 15); }
__device__ inline int rope_chunk(int r, int c) { return kDenseRope + 128 * r + 16 * ((c + swz(r)) & 7); }

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
};

static_assert(TileCopy<0>::slots_cover_copies() && TileCopy<1>::slots_cover_copies(),
              "copy schedule must issue every copy of a tile once");
// Copy of one dense bf16 tile in the layout of the pipelined kernel, 18
// copies per wave: copies 0..15 take the NoPE parts of key rows 4i + wave
// (i = copy), one contiguous 1 KiB read each; copies 16 and 17 take the
// RoPE parts of rows 8j .. 8j+7 for j = wave and wave + 4 (lane L: row
// 8j + L/8, LDS slot L%8, which holds chunk (L%8 - swz(row)) mod 8).  A copy
// whose source is one contiguous range moves far faster than one gathered
// from eight rows.  Rows past the tile's visible range read the last visible
// row instead: finite values whose probabilities are zero.
struct DenseCopy {
  const uint8_t* page;  // cache address of the tile's page (wave-uniform)
  uint32_t mbase;       // LDS address of the tile buffer + 4 * kNopeSlot * wave (wave-uniform)
  uint32_t rbase;       // LDS address of the buffer's RoPE region (wave-uniform)
  int nvm1;             // last row of the tile to read (0..63)
  uint32_t nlane;       // byte offset of this lane's 16 bytes in row `wave` of the page
  uint32_t ncap;        // the same in row nvm1
  __device__ inline void prepare(const uint8_t* __restrict__ kv, int pg, int tile, int vis,
                                 uint32_t buf) {
    // A tile with no visible row (the one past a segment's end) is copied
    // from page 0 of the pool: its block-table entry may lie past the
    // sequence's pages (an unused slot), and nothing reads the copy.
    page = kv + (vis > tile * kPage ? (int64_t)pg * (kPage * 1152) : (int64_t)0);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // nope_row(4i + w) = kNopeGroup * (i / 4) + kNopeSlot * (4w + i % 4)
    mbase = buf + 4 * kNopeSlot * w;
    rbase = buf + kDenseRope;
    nvm1 = __builtin_amdgcn_readfirstlane(min(kPage - 1, max(vis - tile * kPage - 1, 0)));
    const uint32_t l16 = 16 * (threadIdx.x & 63);
    nlane = (uint32_t)w * 1152 + l16;
    ncap = (uint32_t)nvm1 * 1152 + l16;
  }
  template <int I>
  __device__ inline void issue() const {
    if constexpr (I < 16) {
      // row min(4I + wave, nvm1); the LDS destination is an immediate offset
      // from this wave's base (M0 set by one scalar add)
      const uint32_t voff = min(nlane + 4 * 1152 * I, ncap);
      asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff), "s"(page), "s"(mbase), "n"(kNopeGroup * (I >> 2) + kNopeSlot * (I & 3))
                   : "memory", "m0", "scc");
    } else {
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));  // recomputed here rather than kept in registers
      const int lane = tid & 63;
      const int j = 4 * (I - 16) + (tid >> 6);
      const int rd = 8 * j + (lane >> 3);  // row in the tile
      const uint32_t voff = (uint32_t)(min(rd, nvm1) * 1152 + 1024 + 16 * (((lane & 7) - swz(rd)) & 7));
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(rbase + 1024 * j);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff), "s"(page), "s"(m0) : "memory", "m0");
    }
  }
  template <int I = 0>
  __device__ inline void issue_all() const {
    if constexpr (I < 18) {
      issue<I>();
      issue_all<I + 1>();
    }
  }
};
// Copies of tile kt+1 per phase of tile kt (18 per wave), all between P*V
// MFMAs (the score chains keep the LDS busy with their K operand reads):
//   B (P*V 1 of kt-1): NoPE rows 0..31      D (P*V 0): RoPE, rows 32..63
// B1 of tile kt+1 needs B's copies and D's two RoPE copies (D's 8 NoPE
// copies may be in flight); B2 of tile kt+1 needs D's (the 8 of B of tile
// kt+1 may be in flight).
constexpr int kDenseB1InFlight = 8;
constexpr int kDenseB2InFlight = 8;

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
// below pads the chain before any VALU reads or writes the result (an MFMA
// result read by the VALU needs wait states the compiler cannot see through
// asm: for this 8-pass MFMA on gfx950 the compiler's own padding is 12, a
// build check confirms it; the drain gives 16).
// Their operands come from LDS reads (K) or are set once per segment (Q),
// so no VALU instruction writes one within the two wait states before an
// MFMA that the hardware would need; a build check verifies this on the
// generated code of every instance.
__device__ inline void mfma_s_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_s_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ inline void mfma_s_drain(f32x16& acc) {
  asm volatile("s_nop 15" : "+v"(acc));
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

// Per-half softmax state of a lane (its row, its 16 keys of the half).
struct HalfSoftmax {
  float tmax;   // max of the masked raw scores, then of the scaled row
  float nmuse;  // minus the reference the probabilities are taken against
  float lh;     // this half's part of the row sum
  float x;      // scaled score in flight between steps
  float e[2];   // the last two probabilities (paired for the bf16 conversion)
  u32x4 pw[2];  // bf16 probability pairs, MFMA operand order
};
constexpr int kSoftmaxSteps = 25;
// The probabilities of a row are taken against a fixed reference: the row's
// first finite maximum.  A row whose scores climb more than this (log2
// units) above it sends the segment to a second pass against the exact row
// maximum, so no probability ever exceeds 2^kRestartMargin.
constexpr float kRestartMargin = 20.0f;
// P*V reads V^T this many column groups (4 MFMAs each) ahead of its use.
constexpr int kVAhead = 2;

template <int FMT, bool SPARSE>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(DecodeArgs a) {
  // bf16: two tile buffers (double buffering).  FP8: one bf16 tile plus a
  // staging buffer for the raw rows of the next tile.  Separate objects let
  // the compiler see that copies into one buffer never alias reads of the
  // other.  P^T of the two halves of a tile have buffers of their own, so
  // the copies of the next tile never wait for them.
  constexpr bool kPipelined = FMT == 0 && !SPARSE;  // tile loop order and layout, below
  __shared__ __attribute__((aligned(256))) uint8_t lds0[kPipelined ? kDenseTileBytes : kTileBytes];
  __shared__ __attribute__((aligned(256))) uint8_t
      lds1[kPipelined ? kDenseTileBytes : (FMT == 0 ? kTileBytes : kStageBytes)];
  __shared__ __attribute__((aligned(256))) uint8_t pbuf[kPHalfBytes];  // P^T of half 0
  // P^T of half 1 (the pipelined kernel keeps it in the RoPE region of the
  // tile it belongs to, dead once the tile's scores are done)
  __shared__ __attribute__((aligned(256))) uint8_t pbuf1[kPipelined ? 16 : kPHalfBytes];

  const Shape& s = a.s;
  constexpr int kRowBytes = RowBytes<FMT>::value;

  // Workgroup -> (part, row group).  Workgroups are dealt round-robin to
  // the 8 XCDs (XCD = id % 8).  XCD x takes the parts
  // [x * per, (x + 1) * per) with all their row groups: the row groups of a
  // part share that XCD's L2 for the tiles they all read, and consecutive
  // parts (the pieces of a split sequence) share it for the sequence's Q.
  // Every kernel argument is fetched in one round of scalar loads here,
  // rather than in a chain of rounds along their first uses.
  asm volatile("" ::"s"(a.q), "s"(a.kv), "s"(a.block_table), "s"(a.seqlens), "s"(a.indices),
               "s"(a.sched), "s"(a.num_splits), "s"(a.num_parts), "s"(a.ws_lse), "s"(a.ws_o),
               "s"(a.out), "s"(a.lse), "s"(s.units), "s"(s.rows), "s"(s.groups),
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
  // Dense layout (pipelined kernel).  K operand of row 32*kb2 + n, chunk
  // 2*st + h: NoPE at kbase + 33280*kb2 + 32*st (st < 32), RoPE at
  // rope_off[st - 32] + 4096*kb2.  V^T operand of row 32*kb2 + 16*sp + 8*e4
  // + 4*h + j16/4, chunk 16*wave + 4*cb + 2*(n/16) + (j16%4)/2, byte
  // 8*(j16%2): vbase + 2080*e4 + 16640*(2*kb2 + sp) + 64*cb.
  const int kbase = nope_row(n) + 16 * h;
  int rope_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rope_off[i] = rope_chunk(n, 2 * i + h);
  const int vbase = kNopeSlot * (4 * (j16 >> 2) + h) +
                    16 * (16 * wave + 2 * (n >> 4) + ((j16 & 3) >> 1)) + 8 * (j16 & 1);

  for (int u = ub; u < s.units && (u < ue || (u == ue && ke > 0)); ++u) {
    // The previous segment is fully consumed (tiles, P^T, epilogue staging
    // in LDS).  No memory fence: Q and the first tile load in parallel below.
    MLA_BARRIER_NO_FENCE();
    const int b = SPARSE ? u / s.s_q : u;
    const int32_t* bt_row = a.block_table + (int64_t)b * s.max_pages;
    const int kfirst = (u == ub) ? kb0 : 0;
    // Q operand fragments of this lane's score row: dims 16*st + 8*h .. +8.
    // Dense: issued first, in flight while the scalar loads below resolve
    // the segment.  Sparse: issued in two halves behind the two rounds of
    // row lookups of the first tiles (below), so that each round waits only
    // for the loads issued before it.  (The row is recomputed from the
    // thread index: a value kept through the previous segment would come
    // back as a spill reload, whose wait would also wait for these loads.)
    bf16x8 qf[kQSteps];
    auto load_q_steps = [&](auto lo_c, auto hi_c) __attribute__((always_inline)) {
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int qr = grp * kRowsPerGroup + (tid >> 6) * 32 + (tid & 31);
      const uint16_t* qrow =
          a.q + ((int64_t)u * s.rows + (qr < s.rows ? qr : 0)) * kDqk + 8 * ((tid >> 5) & 1);
#pragma unroll
      for (int st = decltype(lo_c)::value; st < decltype(hi_c)::value; ++st)
        qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st);
    };
    auto load_q = [&]() __attribute__((always_inline)) {
      load_q_steps(std::integral_constant<int, 0>{}, std::integral_constant<int, kQSteps>{});
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

    float m;              // reference of the row's probabilities, log2 units
    float l;              // running sum of this lane's half of the keys
    float rmax;           // running maximum of the row's scaled scores
    f32x16 o[4][4];       // O^T block (column block cb of this wave, row block rb)
    uint8_t* ks = lds0;   // buffer of the tile being scored
    // Second pass: the exact row maximum of the first, parked in LDS (thread
    // slot, behind the restart votes) so that no register carries it across
    // the pass.  It is read back before the first barrier of the pass, and
    // no P^T store reaches this part of pbuf before that barrier.
    float* mref_slot = reinterpret_cast<float*>(pbuf + 4096 + 256);
    for (int pass = 0;; ++pass) {
      m = pass == 0 ? -INFINITY : mref_slot[threadIdx.x];
      l = 0.0f;
      rmax = -INFINITY;
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
          // The first three tiles' indices, then the first two tiles'
          // table entries, each round issued together (every load at an
          // in-range address, its result selected afterwards) and each
          // followed by half of Q.  The empty asm statements keep the
          // compiler from turning the loads into branches with a wait each
          // and keep the rounds in this order.
          int ix[3];
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            const int k = (kfirst + j) * kPage + lane;
            ix[j] = idx_row[k < s.topk ? k : s.topk - 1];
          }
          load_q_steps(std::integral_constant<int, 0>{}, std::integral_constant<int, kQSteps / 2>{});
          asm volatile("" : "+v"(ix[0]), "+v"(ix[1]), "+v"(ix[2])::"memory");
          auto pos = [&](int j) {
            const int k = (kfirst + j) * kPage + lane;
            return (kfirst + j < kend && k < s.topk) ? ix[j] : -1;
          };
          const int t0 = pos(0), t1 = pos(1);
          res_t = pos(2);
          int pg0 = bt_row[visible(t0) ? (t0 >> 6) : 0];
          int pg1 = bt_row[visible(t1) ? (t1 >> 6) : 0];
          load_q_steps(std::integral_constant<int, kQSteps / 2>{}, std::integral_constant<int, kQSteps>{});
          asm volatile("" : "+v"(pg0), "+v"(pg1)::"memory");
          const int64_t off0 = offset_of(t0, pg0);
          res_off = offset_of(t1, pg1);
          vm_cur = __ballot(off0 >= 0);
          first.prepare(a.kv, off0, lds_addr(FMT == 0 ? lds0 : lds1), wave, lane);
        } else if constexpr (kPipelined) {
          DenseCopy fd;
          fd.prepare(a.kv, pg_first, kfirst, L, lds_addr(lds0));
          fd.issue_all();
          pg_next = pg_second;
        } else {
          // (past the segment's end the second page is not used: its rows
          // are copied from the zero row)
          first.prepare_page(a.kv, pg_first, kfirst, L, lds_addr(FMT == 0 ? lds0 : lds1), wave, lane);
          pg_next = pg_second;
        }
        if constexpr (!kPipelined) first.issue_all(lane);
        if (!SPARSE && pass > 0) load_q();
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

      // Per-tile state read by the softmax and P*V steps below.
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
      //   4, 5   row max across the lane pair, running maximum; a row that
      //          has seen no finite score yet adopts this half's maximum as
      //          its reference (its output and sum are still zero)
      //   6..22  probabilities, software-pipelined so no step waits on a
      //          result of the same step: step 6+v takes the exponential of
      //          score v, the scaled score v+1, the row sum of probability
      //          v-1 and, at even v, the bf16 pair of probabilities v-2, v-1
      //   23, 24 store the half's P^T
      auto softmax_step = [&](int kb2, f32x16& sc, HalfSoftmax& hs, int u, int jl, uint8_t* pdst)
          __attribute__((always_inline)) {
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
            full = __builtin_amdgcn_readfirstlane(__all(jl >= 32 * kb2 + 31) ? 1 : 0) != 0;
          }
          if (!full) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int key = kb2 * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
              const bool ok = SPARSE ? ((lanemask[kb2] >> (8 * (v >> 2) + (v & 3))) & 1) != 0 : key <= jl;
              sc[v] = ok ? sc[v] : -INFINITY;
            }
          }
          hs.tmax = max3f(max3f(sc[0], sc[1], sc[2]), sc[3], sc[4]);
        } else if (u < 4) {
          // scores 5u .. 5u+4 (u = 3: 15 only)
          hs.tmax = u < 3 ? max3f(max3f(hs.tmax, sc[5 * u], sc[5 * u + 1]), sc[5 * u + 2], max2f(sc[5 * u + 3], sc[5 * u + 4]))
                          : max2f(hs.tmax, sc[15]);
        } else if (u == 4) {
          hs.tmax = wave_max_pair(hs.tmax) * scale;  // scale > 0 keeps the max; -inf stays -inf
          rmax = max2f(rmax, hs.tmax);
        } else if (u == 5) {
          if (m == -INFINITY) m = hs.tmax;
          hs.nmuse = (m == -INFINITY) ? 0.0f : -m;
          hs.lh = 0.0f;
          hs.x = __builtin_fmaf(sc[0], scale, hs.nmuse);
        } else if (u < 23) {
          const int v = u - 6;  // 0..16
          if (v >= 2 && (v & 1) == 0) {
            const int w = (v - 2) >> 1;  // bf16 pair of probabilities v-2, v-1
            hs.pw[w >> 2][w & 3] = pk_bf16(hs.e[0], hs.e[1]);
          }
          if (v > 0) {
            hs.lh += hs.e[(v - 1) & 1];
            // keeps the add in this step: otherwise the compiler sinks all 16
            // into one dependent chain at the end, with every probability
            // held in a register until then
            asm volatile("" : "+v"(hs.lh));
          }
          if (v < 16) hs.e[v & 1] = __builtin_amdgcn_exp2f(hs.x);
          if (v < 15) hs.x = __builtin_fmaf(sc[v + 1], scale, hs.nmuse);
          if (v == 16) l += hs.lh;
        } else if (u < 25) {
          const int sp = u - 23;
          // the address is recomputed from the thread index, not kept in a
          // register through the tile loop
          int tid = threadIdx.x;
          asm volatile("" : "+v"(tid));
          const int pw = tid >> 6, pn = tid & 31, ph = (tid >> 5) & 1;
          asm volatile("" ::: "memory");  // LDS accesses stay in program order around the store
          *reinterpret_cast<u32x4*>(pdst + 2048 * pw + p_chunk(pn, 2 * sp + ph)) = hs.pw[sp];
          asm volatile("" ::: "memory");
        }
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
        i16x4 lo, hi;
        if constexpr (kPipelined) {
          const uint8_t* vb = vt + vbase + kNopeGroup * (2 * kb2 + sp) + 64 * cb;
          lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(vb));
          hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(vb + 2 * kNopeSlot));
        } else {
          const uint8_t* vb = vt + 8192 * (2 * wave + (cb >> 1)) + 4096 * kb2 + 2048 * sp;
          lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(vb + v_off[cb & 1][0]));
          hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(vb + v_off[cb & 1][1]));
        }
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int kVRegs = kVAhead + 1;
      constexpr int kVPrefetchReads = 2 * kVAhead;  // LDS reads issued by pv_prefetch
      auto pv_prefetch = [&](const uint8_t* vt, int kb2, bf16x8* vf) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < kVAhead; ++g) vf[g] = load_v(vt, kb2, g);
      };
      // (the lane's address is formed once per key step and kept opaque, so
      // the row blocks are immediate offsets rather than one VALU add each:
      // P^T buffers lie beyond the 64 KiB an immediate offset reaches)
      using lds_u8 = const __attribute__((address_space(3))) uint8_t;
      auto p_lane = [&](const uint8_t* pb, int sp) {
        lds_u8* b = lds_ptr<const uint8_t>(pb + p_off[sp]);  // an LDS pointer: ds_read, not flat
        asm volatile("" : "+v"(b));
        return b;
      };
      auto load_p = [&](lds_u8* pl, int rb) {
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(pl + 2048 * rb);
      };
      auto pv_run = [&](int kb2, const uint8_t* vt, const uint8_t* pb, bf16x8* vf, bf16x8* pfr,
                        auto&& hook) __attribute__((always_inline)) {
        lds_u8* pl1 = p_lane(pb, 1);
        static_for<0, 8>([&](auto g_c) __attribute__((always_inline)) {
          constexpr int g = decltype(g_c)::value;
          constexpr int cb = g & 3;
          if constexpr (g + kVAhead < 8) vf[(g + kVAhead) % kVRegs] = load_v(vt, kb2, g + kVAhead);
          static_for<0, 4>([&](auto rb_c) __attribute__((always_inline)) {
            constexpr int rb = decltype(rb_c)::value;
            o[cb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[g % kVRegs], pfr[rb], o[cb][rb], 0, 0, 0);
            // the second key step's P^T block rb, right after its last use
            if constexpr (g == 3) pfr[rb] = load_p(pl1, rb);
            hook(std::integral_constant<int, 4 * g + rb>{});
            __builtin_amdgcn_sched_barrier(0);
          });
        });
      };
      auto pv_half = [&](int kb2, const uint8_t* vt, const uint8_t* pb, bf16x8* vf, auto&& pre,
                         auto&& hook) __attribute__((always_inline)) {
        bf16x8 pfr[4];
        lds_u8* pl = p_lane(pb, 0);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) pfr[rb] = load_p(pl, rb);
        pre();  // runs while the first operands are in flight
        pv_run(kb2, vt, pb, vf, pfr, hook);
      };

      // Dense bf16 tiles run one P*V half behind the scores.  The score
      // chains are bound by their K operand reads from LDS (one 1 KiB read
      // per MFMA and wave); the P*V halves are fed from registers and two
      // LDS reads per MFMA.  The softmax of a half is spread over both
      // kinds of phase: its first steps (mask, maxima, the first
      // exponentials) run between the MFMAs of the P*V half that follows
      // the half's scores, the rest between the MFMAs of the next score
      // chain, which publishes the half's P^T with a barrier of its own and
      // then reads the first operands of the P*V half after it.  Tile kt:
      //   B1 | A: scores 0 of kt; softmax 1 of kt-1, second part (P^T into
      //      |    the RoPE region of kt-1's buffer) | barrier |     (copies)
      //      | B: P*V 1 of kt-1; softmax 0 of kt, first part       (copies)
      //   B2 | C: scores 1 of kt; softmax 0 of kt, second part (P^T into
      //      |    pbuf) | barrier |                                (copies)
      //      | D: P*V 0 of kt; softmax 1 of kt, first part         (copies)
      // B1 waits for rows 0..31 and the RoPE region of tile kt and frees
      // rows 0..31 of the other buffer (P*V 0 of kt-1 is done) and pbuf;
      // B2 waits for rows 32..63 of tile kt and frees rows 32..63 and the
      // RoPE region of the other buffer (P*V 1 of kt-1 is done).
      if constexpr (kPipelined) {
        const __attribute__((address_space(4))) int32_t* bt_const =
            (const __attribute__((address_space(4))) int32_t*)bt_row;  // scalar loads
        bf16x8 vf[kVRegs];
        bf16x8 pfr[4];
        // Softmax 1 of the tile before, carried into the next tile's first
        // chain.  The first tile of a segment has none: scores of -inf and a
        // cleared state make its second part add nothing.
        f32x16 sacc1;
        HalfSoftmax hs1;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc1[i] = -INFINITY;
        hs1.tmax = -INFINITY;
        hs1.nmuse = 0.0f;
        hs1.lh = 0.0f;
        hs1.x = -INFINITY;
        hs1.e[0] = hs1.e[1] = 0.0f;
        hs1.pw[0] = hs1.pw[1] = u32x4{0u, 0u, 0u, 0u};
        int jl_prev = 63;
        // K operand of step st of the chain over rows 32*kb2 .. +31 of buffer kb
        auto k_dense = [&](const uint8_t* kb, int kb2, int st) {
          return *reinterpret_cast<const bf16x8*>(
              kb + (st < 32 ? kbase + 33280 * kb2 + 32 * st : rope_off[st - 32] + 4096 * kb2));
        };
        // 36 score MFMAs of half kb2 with hook(st) after MFMA st; K operands
        // are read kKPrefetch steps ahead
        auto chain = [&](f32x16& acc, const uint8_t* kb, int kb2, auto&& hook) __attribute__((always_inline)) {
          bf16x8 kf[kKPrefetch];
#pragma unroll
          for (int st = 0; st < kKPrefetch; ++st) kf[st] = k_dense(kb, kb2, st);
          static_for<0, kQSteps>([&](auto st_c) __attribute__((always_inline)) {
            constexpr int st = decltype(st_c)::value;
            const bf16x8 cur_k = kf[st % kKPrefetch];
            if constexpr (st + kKPrefetch < kQSteps) kf[st % kKPrefetch] = k_dense(kb, kb2, st + kKPrefetch);
            if constexpr (st == 0)
              mfma_s_first(acc, cur_k, qf[st]);
            else
              mfma_s_acc(acc, cur_k, qf[st]);
            hook(st_c);
            __builtin_amdgcn_sched_barrier(0);
          });
          mfma_s_drain(acc);
        };
        // Softmax steps 0 .. kSplit-1 go after P*V MFMAs 3, 5, .., steps
        // kSplit .. 24 after score MFMAs 1, 2, ..; the P^T stores (steps 23,
        // 24, after MFMAs 11 and 12) precede the chain's barrier (after MFMA
        // 16) by exactly four LDS reads, the K operands of steps 17 to 20.
        constexpr int kSplit = 13;
        constexpr int kChainBarrierStep = kSoftmaxSteps - kSplit + 4;  // 16
        constexpr int kReadsAfterStores = 4;
        auto in_pv = [](int j) { return j >= 3 && (j & 1) == 1 && (j - 3) / 2 < kSplit; };
        for (int kt = kfirst; kt < kend; ++kt) {
          const bool odd = ((kt - kfirst) & 1) != 0;
          // B1
          MLA_WAIT_VMCNT(kDenseB1InFlight);
          MLA_BARRIER_NO_FENCE();
          ks = odd ? lds1 : lds0;
          uint8_t* const kprev = odd ? lds0 : lds1;
          DenseCopy next;
          next.prepare(a.kv, pg_next, kt + 1, kt + 1 < kend ? L : 0, lds_addr(kprev));
          const int jl = min(63, tlim - kt * kPage);

          HalfSoftmax hs0;
          f32x16 sacc0;
          // A.
          chain(sacc0, ks, 0, [&](auto st_c) __attribute__((always_inline)) {
            constexpr int st = decltype(st_c)::value;
            if constexpr (st >= 1 && st <= kSoftmaxSteps - kSplit)
              softmax_step(1, sacc1, hs1, kSplit + st - 1, jl_prev, kprev + kDenseRope);
            if constexpr (st == kChainBarrierStep) MLA_BARRIER_NO_FENCE_KEEP(kReadsAfterStores);
            if constexpr (st == kChainBarrierStep + 1 || st == kChainBarrierStep + 2)
              vf[st - kChainBarrierStep - 1] = load_v(kprev, 1, st - kChainBarrierStep - 1);
            if constexpr (st == kChainBarrierStep + 3 || st == kChainBarrierStep + 4) {
              constexpr int r0 = 2 * (st - kChainBarrierStep - 3);
              lds_u8* pl = p_lane(kprev + kDenseRope, 0);
              pfr[r0] = load_p(pl, r0);
              pfr[r0 + 1] = load_p(pl, r0 + 1);
            }
          });
          // B. (the first tile of a segment has no P*V 1 of a previous tile)
          if (kt > kfirst) {
            pv_run(1, kprev, kprev + kDenseRope, vf, pfr, [&](auto j_c) __attribute__((always_inline)) {
              constexpr int j = decltype(j_c)::value;
              if constexpr (j % 4 == 2) next.template issue<j / 4>();  // copies 0..7
              if constexpr (in_pv(j)) softmax_step(0, sacc0, hs0, (j - 3) / 2, jl, pbuf);
            });
          } else {
            static_for<0, 8>([&](auto i_c) __attribute__((always_inline)) {
              next.template issue<decltype(i_c)::value>();
            });
            static_for<0, kSplit>([&](auto u_c) __attribute__((always_inline)) {
              softmax_step(0, sacc0, hs0, decltype(u_c)::value, jl, pbuf);
            });
          }
          // B2
          MLA_WAIT_VMCNT(kDenseB2InFlight);
          MLA_BARRIER_NO_FENCE();
          // C.
          chain(sacc1, ks, 1, [&](auto st_c) __attribute__((always_inline)) {
            constexpr int st = decltype(st_c)::value;
            if constexpr (st >= 1 && st <= kSoftmaxSteps - kSplit)
              softmax_step(0, sacc0, hs0, kSplit + st - 1, jl, pbuf);
            if constexpr (st == kChainBarrierStep) MLA_BARRIER_NO_FENCE_KEEP(kReadsAfterStores);
            if constexpr (st == kChainBarrierStep + 1 || st == kChainBarrierStep + 2)
              vf[st - kChainBarrierStep - 1] = load_v(ks, 0, st - kChainBarrierStep - 1);
            if constexpr (st == kChainBarrierStep + 3 || st == kChainBarrierStep + 4) {
              constexpr int r0 = 2 * (st - kChainBarrierStep - 3);
              lds_u8* pl = p_lane(pbuf, 0);
              pfr[r0] = load_p(pl, r0);
              pfr[r0 + 1] = load_p(pl, r0 + 1);
            }
          });
          // D.
          pv_run(0, ks, pbuf, vf, pfr, [&](auto j_c) __attribute__((always_inline)) {
            constexpr int j = decltype(j_c)::value;
            // the RoPE copies first (needed at the end of the next tile's first chain)
            if constexpr (j == 0 || j == 1) next.template issue<16 + j>();
            if constexpr (j % 3 == 2 && j / 3 < 8) next.template issue<8 + j / 3>();  // copies 8..15
            if constexpr (in_pv(j)) softmax_step(1, sacc1, hs1, (j - 3) / 2, jl, ks + kDenseRope);
          });
          jl_prev = jl;
          // the page of tile kt+2, for the next tile's copies (a scalar load,
          // waited for by the barrier that starts the next tile)
          pg_next = bt_const[min(kt + 2, nb - 1)];
        }
        // Second part of softmax 1 and P*V 1 of the last tile.  Its P^T goes
        // into the RoPE region of the tile, which other waves may still read
        // at the end of their second score chain: a barrier first.
        MLA_BARRIER_NO_FENCE();
        static_for<kSplit, kSoftmaxSteps>([&](auto u_c) __attribute__((always_inline)) {
          softmax_step(1, sacc1, hs1, decltype(u_c)::value, jl_prev, ks + kDenseRope);
        });
        pv_prefetch(ks, 1, vf);
        MLA_BARRIER_NO_FENCE_KEEP(kVPrefetchReads);
        pv_half(1, ks, ks + kDenseRope, vf, [] {}, [](auto) {});
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
          if constexpr (st < kSoftmaxSteps) softmax_step(0, sacc0, hs0, st, jlim, pbuf);
        });

        // 4. half 0's P^T visible
        bf16x8 vf[kVRegs];
        pv_prefetch(ks, 0, vf);
        MLA_BARRIER_NO_FENCE_KEEP(kVPrefetchReads);
        pv_half(0, ks, pbuf, vf, [] {}, [&](auto j_c) __attribute__((always_inline)) {
          constexpr int j = decltype(j_c)::value;
          next.template issue_at<2, j>(lane);
          if constexpr (j < kSoftmaxSteps) softmax_step(1, sacc1, hs1, j, jlim, pbuf1);
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
        MLA_BARRIER_NO_FENCE_KEEP(kVPrefetchReads);  // half 1's P^T visible
        if constexpr (FMT == 0) {
          pv_half(1, ks, pbuf1, vf, [] {}, [](auto) {});
        } else {
          // rows 0..31 of tile kt are no longer read (half 0 is done): the
          // staged rows 0..31 of tile kt+1 are dequantised into them between
          // the MFMAs of half 1 (after a unit's last tile they are zero rows
          // written into a tile nothing reads any more)
          HalfDequant dq;
          pv_half(1, ks, pbuf1, vf, [&] { dq.load(lds1, 0); },
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

      // Restart test: a row whose scores climbed more than kRestartMargin
      // above its reference sends the whole workgroup through the segment
      // again, against the exact row maxima this pass found.  Every wave
      // publishes its vote after its last P*V (pbuf is free: the last reads
      // of it were before the final barrier), then reads all four.
      uint32_t* votes = reinterpret_cast<uint32_t*>(pbuf + 4096);
      if (pass == 0) {
        const bool over = __ballot(rmax > m + kRestartMargin) != 0;
        if (lane == 0) votes[wave] = over ? 1u : 0u;
      }
      MLA_BARRIER_NO_FENCE();
      if (pass == 0) {
        const u32x4 vw = *reinterpret_cast<const u32x4*>(votes);
        if (__builtin_amdgcn_readfirstlane(vw[0] | vw[1] | vw[2] | vw[3]) != 0) {
          mref_slot[threadIdx.x] = rmax;
          MLA_BARRIER_NO_FENCE();  // every wave has read the votes
          continue;
        }
      }
      break;
    }

    // ---- epilogue.  The score-row owner publishes the row's output factor;
    // every wave then normalises and stores its column blocks.
    const float ltot = wave_sum_pair(l);
    const float lse2 = ltot > 0.0f ? m + log2f(ltot) : -INFINITY;
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    // half 0's P^T buffer is free: every wave is past the last tile's final barrier
    float* epi = reinterpret_cast<float*>(pbuf);
    if (h == 0) epi[rs] = inv;
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
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      uint8_t* const stg = ks + 32768 * (rb & 1);
      {
        const float f = epi[32 * rb + on];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v = f32x4{o[cb][rb][4 * q4], o[cb][rb][4 * q4 + 1], o[cb][rb][4 * q4 + 2],
                                  o[cb][rb][4 * q4 + 3]} * f;
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
