// FP8 top-k indexer for gfx950: per query token, the cached rows of largest
// head-summed FP8 score ("max.nn.kernels 内核封装模块全解析", section
// 稀疏注意力（MSA）与 MLA 索引内核, mla_fp8_index_top_k).  The definition and
// its readings are in include/mla_index.h.
//
// The sum over heads is linear, so it can be taken before the dot products:
//   S_j = sum_t s_j[t] * sum_{d in tile t} e4m3(c_j[d]) * Qsum[d],
//   Qsum[d] = sum_h qs[h][t(d)] * e4m3(q[h][d]),
// which is the definition's value with the sums regrouped.  Scoring a row
// then costs 512 multiply-adds per query token instead of 512 per head, and
// the kernels are bound by the stream of cache rows.  Three kernels on the
// caller's stream:
//   index_query_kernel  Qsum of every query token (fp32, into the workspace);
//   index_score_kernel  S[b][i][j] for every row j of the pages that hold
//                       visible rows (fp32, into the workspace);
//   index_topk_kernel   per (b, i): the top-k visible rows by S, ascending j,
//                       -1 fill.
//
// Scores.  A workgroup (8 waves) owns one sequence b, up to kMaxTokens of its
// query tokens and a chunk of kChunkPages pages.  Sixteen lanes share a row:
// lane c holds Qsum of dims [16c, 16c + 16) and [256 + 16c, 256 + 16c + 16)
// of each token in registers, converts the row's codes of those dims to fp32
// (exactly), takes its two partial dot products, scales each by its tile's
// scale and sums with the other fifteen lanes in four DPP rotations.
//
// Cache rows are staged whole-page, 528 bytes per row (the 512 codes and
// the four scales; the bf16 RoPE part is not read) at a 528-byte pitch, so
// the 16 lanes of a row read 16 distinct 16-byte bank groups.  A page is 33
// direct global->LDS copies of 1 KiB, spread over the eight waves, into a
// ring of kRing pages kept kRing - 1 pages ahead.
#include "../../include/mla_index.h"
#include "internal.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kIdxThreads = 512;         // 8 waves
constexpr int kIdxWaves = kIdxThreads / 64;
constexpr int kRowBytes = 656;           // cache row (MLA_KV_FP8_656)
constexpr int kStageRow = 528;           // staged part: codes + scales
constexpr int kStagePage = kPage * kStageRow;  // 33792
constexpr int kPageCopies = kStagePage / 1024;  // 33
constexpr int kRing = 4;
constexpr int kCopiesPerWave = 4;        // waves 1..7; wave 0 issues 5
static_assert(kPageCopies == kIdxWaves * kCopiesPerWave + 1, "copy split");
constexpr int kMaxTokens = 4;            // query tokens of a workgroup
constexpr int kChunkPages = kIndexChunkPages;

// Waits and barriers that leave the direct copies alone (the compiler does
// not see them; see the decode kernel for the same rules).
#define IDX_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
#define IDX_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

__device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Visible (pooled) rows of query token i of a sequence of L tokens.
__device__ inline int visible_rows(int L, int s_q, int i, int kpool, int causal) {
  const int t_max = causal ? L - s_q + i : L - 1;
  return t_max < 0 ? 0 : t_max / kpool + 1;
}

// LDS address of a __shared__ object (wave-uniform).
__device__ inline uint32_t lds_u32(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

// x rotated right by N lanes within each row of 16 lanes (DPP).
template <int N>
__device__ inline float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row, in every lane of it.
__device__ inline float row_sum16(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  return x;
}

struct IndexArgs {
  int32_t batch, s_q, h, tokens_per_group, groups;
  int32_t kpool, is_causal, max_pages, chunks, n_max;
  const uint8_t* q;
  const float* qs;
  const uint8_t* kv;
  const int32_t* block_table;
  const int32_t* seqlens;
  float* ws;    // scores [B, s_q, n_max]
  float* qsum;  // [B, s_q, 512]
  int32_t topk;
  int32_t* indices;
  float* scores;
};

// Four e4m3 codes (one 32-bit word) to fp32, exactly.
__device__ inline void codes4(uint32_t w, float* out) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// Qsum of query token blockIdx.x.  Lane l of wave w holds dims 8l .. 8l + 7
// (one 8-byte load per head row) and sums heads w, w + 4, .. in head order;
// the four wave partials are added in wave order through LDS.
__global__ void __launch_bounds__(256) index_query_kernel(IndexArgs a) {
  __shared__ __attribute__((aligned(16))) float part[4][512];
  const int64_t tok = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d0 = 8 * lane;
  const uint8_t* q = a.q + tok * a.h * 512 + d0;
  const float* qs = a.qs + tok * a.h * 4 + (d0 >> 7);
  float acc[8] = {};
  int h = wave;
  // four heads in flight per step: independent loads, then the fmas in order
  for (; h + 12 < a.h; h += 16) {
    uint64_t codes[4];
    float sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      codes[u] = *reinterpret_cast<const uint64_t*>(q + (int64_t)(h + 4 * u) * 512);
      sc[u] = qs[(int64_t)(h + 4 * u) * 4];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float f[8];
      codes4((uint32_t)codes[u], f);
      codes4((uint32_t)(codes[u] >> 32), f + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(sc[u], f[e], acc[e]);
    }
  }
  for (; h < a.h; h += 4) {
    const uint64_t c8 = *reinterpret_cast<const uint64_t*>(q + (int64_t)h * 512);
    const float sc = qs[(int64_t)h * 4];
    float f[8];
    codes4((uint32_t)c8, f);
    codes4((uint32_t)(c8 >> 32), f + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(sc, f[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[wave][d0 + e] = acc[e];
  __syncthreads();
  const int d = 2 * (int)threadIdx.x;
  f32x2 r;
#pragma unroll
  for (int e = 0; e < 2; ++e) r[e] = ((part[0][d + e] + part[1][d + e]) + part[2][d + e]) + part[3][d + e];
  *reinterpret_cast<f32x2*>(a.qsum + tok * 512 + d) = r;
}

template <int TG>
__global__ void __launch_bounds__(kIdxThreads, 1) index_score_kernel(IndexArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * kStagePage];

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; XCD x
  // takes a contiguous run of (sequence, group, chunk) items, so the chunks
  // of one sequence share that XCD's L2.
  const int total = a.batch * a.groups * a.chunks;
  const int per_xcd = (total + 7) / 8;
  const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= total) return;
  const int chunk = item % a.chunks;
  const int g = (item / a.chunks) % a.groups;
  const int b = item / (a.chunks * a.groups);

  using cint32 = const __attribute__((address_space(4))) int32_t;
  const int L = ((cint32*)a.seqlens)[b];
  const int i0 = g * a.tokens_per_group;
  const int ntok = min(a.tokens_per_group, a.s_q - i0);
  // the group's most visible rows, at most the rows the table holds (as in
  // the selection), so a length beyond the table reads nothing past its row
  const int nvis = min(visible_rows(L, a.s_q, i0 + ntok - 1, a.kpool, a.is_causal), a.n_max);
  const int p_begin = chunk * kChunkPages;
  const int p_end = min(p_begin + kChunkPages, ceil_div(nvis, kPage));
  if (p_begin >= p_end) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15;  // dim chunk of the lane
  cint32* bt = (cint32*)(a.block_table + (int64_t)b * a.max_pages);

  // Direct copies of page p into ring slot p % kRing.  Copy k (of 33) fills
  // LDS bytes [1024k, 1024k + 1024) of the slot: lane L's 16 bytes are byte
  // o = 1024k + 16L of the staged page, row o / 528, offset o % 528.  Wave w
  // issues copies w, w + 8, ..; wave 0 also the 33rd, which the waits below
  // count as if it belonged to the next page (a slightly longer wait on
  // wave 0, exact on the others).
  const uint32_t ring_base = lds_u32(ring);
  auto issue_page = [&](int p) {
    const int pg = bt[p];
    const uint8_t* src = a.kv + (int64_t)pg * (kPage * kRowBytes);
    const uint32_t slot = ring_base + (uint32_t)(p % kRing) * kStagePage;
    const int ncopy = wave == 0 ? kCopiesPerWave + 1 : kCopiesPerWave;
    for (int k = 0; k < ncopy; ++k) {
      const int cp = wave + kIdxWaves * k;
      const uint32_t o = 1024u * cp + 16u * lane;
      const uint32_t r = (o * 7944u) >> 22;  // o / 528 for o < 33792
      const uint32_t voff = r * kRowBytes + (o - r * kStageRow);
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(slot + 1024u * cp);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff), "s"(src), "s"(m0) : "memory", "m0");
    }
  };

  // Qsum of the lane's 32 dims for each token of the group (0 past ntok).
  float qlo[TG][16], qhi[TG][16];
#pragma unroll
  for (int tk = 0; tk < TG; ++tk) {
    const float* qv = a.qsum + ((int64_t)b * a.s_q + i0 + min(tk, ntok - 1)) * 512;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      f32x4 lo = *reinterpret_cast<const f32x4*>(qv + 16 * c + 4 * e4);
      f32x4 hi = *reinterpret_cast<const f32x4*>(qv + 256 + 16 * c + 4 * e4);
      if (tk >= ntok) lo = hi = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qlo[tk][4 * e4 + e] = lo[e];
        qhi[tk][4 * e4 + e] = hi[e];
      }
    }
  }
  // the query loads must land before the first copy is counted
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");

  const int npages = p_end - p_begin;
  for (int k = 0; k < kRing - 1 && k < npages; ++k) issue_page(p_begin + k);

  float* ws_b = a.ws + ((int64_t)b * a.s_q + i0) * a.n_max;
  for (int k = 0; k < npages; ++k) {
    const int p = p_begin + k;
    // page p landed (the pages after it may still be in flight)
    const int ahead = min(npages - 1 - k, kRing - 2);
    if (ahead >= 2) IDX_WAIT_VMCNT(2 * kCopiesPerWave);
    else if (ahead == 1) IDX_WAIT_VMCNT(kCopiesPerWave);
    else IDX_WAIT_VMCNT(0);
    IDX_BARRIER();
    if (k + kRing - 1 < npages) issue_page(p + kRing - 1);

    const uint8_t* st = ring + (p % kRing) * kStagePage;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int row = 8 * wave + 4 * m + (lane >> 4);
      const uint8_t* kr = st + row * kStageRow;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(kr + 16 * c);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(kr + 256 + 16 * c);
      const f32x4 sc = *reinterpret_cast<const f32x4*>(kr + 512);
      const float s_lo = c < 8 ? sc[0] : sc[1];  // tile of dims 16c..
      const float s_hi = c < 8 ? sc[2] : sc[3];  // tile of dims 256 + 16c..
      float klo[16], khi[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        codes4(lo[w], klo + 4 * w);
        codes4(hi[w], khi + 4 * w);
      }
      float v[TG];
#pragma unroll
      for (int tk = 0; tk < TG; ++tk) {
        float p1 = 0.f, p2 = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p1 = __builtin_fmaf(qlo[tk][e], klo[e], p1);
          p2 = __builtin_fmaf(qhi[tk][e], khi[e], p2);
        }
        v[tk] = row_sum16(__builtin_fmaf(s_lo, p1, s_hi * p2));
      }
#pragma unroll
      for (int tk = 0; tk < TG; ++tk)
        if (c == tk && tk < ntok) ws_b[(int64_t)tk * a.n_max + p * kPage + row] = v[tk];
    }
  }
}

// Order-preserving key of an fp32 score (larger score, larger key); NaN
// maps to 1, below every other value; 0 marks a row that is not visible.
__device__ inline uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f);
  if (f != f) return 1u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;
constexpr int kPerThread = 64;  // rows per thread: 65536 per sequence at most

// Inclusive prefix sum over the 64 lanes of a wave in six DPP adds: within
// each row of 16 lanes by shifts of 1, 2, 4 and 8, then the last lane of
// rows 0 and 2 into rows 1 and 3 (row_bcast:15) and lane 31 into rows 2 and
// 3 (row_bcast:31).
__device__ inline int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}
__device__ inline int wave_total(int x) { return __builtin_amdgcn_readlane(wave_incl_scan(x), 63); }

// Workgroup sum of one int per thread: the wave sums, then the 16 of them
// through LDS (in wave order).  The two halves of red[] alternate between
// calls, so one barrier per call suffices: a wave can write the other half
// while slower waves still read this one, and a half is written again only
// after a later barrier that every reader of it has passed.
__device__ inline int block_sum(int v, int* red, int& parity, int wave, int lane) {
  const int t = wave_total(v);
  int* r = red + parity * (kTopkThreads / 64);
  parity ^= 1;
  if (lane == 0) r[wave] = t;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) s += r[w];
  return s;
}

// Bits of the threshold found over all rows before the candidates that
// share them are compacted into LDS, and the most candidates compacted.
constexpr int kTopBits = 12;
constexpr int kLowBits = 32 - kTopBits;
constexpr int kMaxCand = 8192;
constexpr int kWaveRows = 64 * kPerThread;  // rows of one wave: 4096
constexpr int kQuads = kPerThread / 4;       // 16-byte loads per lane

// Selection of the top-k rows of one query token.  Wave w owns rows
// [4096w, 4096w + 4096); its load e4 covers rows 4096w + 256e4 + [0, 256),
// four per lane (rows 4l .. 4l + 3 of the 256), so every load reads 1 KiB
// contiguous and row order is (wave, e4, lane, element).  Ranks in row order
// come from lane prefix sums per load plus the totals of the waves before.
__global__ void __launch_bounds__(kTopkThreads, 1) index_topk_kernel(IndexArgs a) {
  __shared__ int red[2 * (kTopkThreads / 64)];
  __shared__ int wred[kTopkThreads / 64];
  __shared__ uint32_t cand[kMaxCand];  // low bits of the keys that share the threshold's top bits
  int parity = 0;
  const int row = blockIdx.x;  // (b, i)
  const int b = row / a.s_q, i = row % a.s_q;
  const int L = a.seqlens[b];
  const int n = min(visible_rows(L, a.s_q, i, a.kpool, a.is_causal), a.n_max);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* src = a.ws + (int64_t)row * a.n_max;
  const int jw = kWaveRows * wave + 4 * lane;  // row of element (e4, q): jw + 256 e4 + q

  uint32_t key[kPerThread];
#pragma unroll
  for (int e4 = 0; e4 < kQuads; ++e4) {
    const int j = jw + 256 * e4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (j < n) v = *reinterpret_cast<const f32x4*>(src + j);  // j + 3 < n_max: inside the row
#pragma unroll
    for (int q = 0; q < 4; ++q) key[4 * e4 + q] = (j + q < n) ? score_key(v[q]) : 0u;
  }

  // Sum over the waves before this one of one wave-uniform value per wave.
  auto waves_before = [&](int wave_value) {
    if (lane == 0) wred[wave] = wave_value;
    __syncthreads();
    int s0 = 0;
    for (int w = 0; w < wave; ++w) s0 += wred[w];
    __syncthreads();
    return s0;
  };

  // Threshold: the largest T with #{key >= T} >= k (n > k), else take all.
  // Bisection, one bit at a time from the top.  After the top kTopBits bits
  // the keys that still share them are usually few: they are compacted into
  // LDS and the low bits are found on them alone (the keys above their band
  // counted once); a band too wide for LDS keeps bisecting over all rows.
  const int k = a.topk;
  uint32_t T = 1u;
  int need_eq = 0;
  if (n > k) {
    T = 0u;
    for (int bit = 31; bit >= kLowBits; --bit) {
      const uint32_t c1 = T | (1u << bit);
      int c = 0;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) c += key[e] >= c1 ? 1 : 0;
      if (block_sum(c, red, parity, wave, lane) >= k) T = c1;
    }
    constexpr uint32_t kBand = 1u << kLowBits;
    int in_band = 0, above = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      in_band += (key[e] - T) < kBand ? 1 : 0;  // T <= key < T + kBand (T <= 2^32 - kBand: no wrap)
      above += key[e] > (T | (kBand - 1)) ? 1 : 0;
    }
    const int m = block_sum(in_band, red, parity, wave, lane);
    const int above_all = block_sum(above, red, parity, wave, lane);
    if (m <= kMaxCand) {
      // compaction, in any order: the lane's slots after the lanes and waves before it
      const int incl = wave_incl_scan(in_band);
      int at = waves_before(__builtin_amdgcn_readlane(incl, 63)) + incl - in_band;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e)
        if ((key[e] - T) < kBand) cand[at++] = key[e] - T;
      __syncthreads();
      // the low bits on the m candidates, by all waves (at most 8 a thread)
      uint32_t U = 0u;
      for (int bit = kLowBits - 1; bit >= 0; --bit) {
        const uint32_t c1 = U | (1u << bit);
        int c = 0;
        for (int ci = tid; ci < m; ci += kTopkThreads) c += cand[ci] >= c1 ? 1 : 0;
        if (block_sum(c, red, parity, wave, lane) + above_all >= k) U = c1;
      }
      T += U;
    } else {
      for (int bit = kLowBits - 1; bit >= 0; --bit) {
        const uint32_t c1 = T | (1u << bit);
        int c = 0;
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) c += key[e] >= c1 ? 1 : 0;
        if (block_sum(c, red, parity, wave, lane) >= k) T = c1;
      }
    }
    int cg = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) cg += key[e] > T ? 1 : 0;
    need_eq = k - block_sum(cg, red, parity, wave, lane);
  }

  // Selection in row order: keys above T, and the first need_eq keys equal
  // to T (ties go to the smallest rows).
  uint32_t selw[kPerThread / 32] = {};  // bit e % 32 of word e / 32: element e selected
  if (n > k) {
    int eq_lane = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) eq_lane += key[e] == T ? 1 : 0;
    int run = waves_before(wave_total(eq_lane));  // ties in earlier waves
#pragma unroll
    for (int e4 = 0; e4 < kQuads; ++e4) {
      int c = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) c += key[4 * e4 + q] == T ? 1 : 0;
      const int incl = wave_incl_scan(c);
      int r = run + incl - c;  // ties before this lane's four rows
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t kk = key[4 * e4 + q];
        const bool sel = kk > T || (kk == T && r < need_eq);
        r += kk == T ? 1 : 0;
        selw[(4 * e4 + q) >> 5] |= (uint32_t)sel << ((4 * e4 + q) & 31);
      }
      run += __builtin_amdgcn_readlane(incl, 63);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) selw[e >> 5] |= (uint32_t)(key[e] != 0u) << (e & 31);
  }
  int nsel = 0;
#pragma unroll
  for (int w = 0; w < kPerThread / 32; ++w) nsel += __builtin_popcount(selw[w]);
  int pos = waves_before(wave_total(nsel));
  int32_t* out_i = a.indices + (int64_t)row * k;
  float* out_s = a.scores ? a.scores + (int64_t)row * k : nullptr;
  // With k <= kMaxCand the selected rows are ranked into LDS (cand is free
  // once the threshold is known) and then written out by all threads in
  // order, coalesced; beyond that each lane stores its own rows.
  const int filled = min(k, n);
  // the lane's first row, recomputed from the thread index: values kept from
  // the loads would be held (spilled) through the whole selection
  int tid_o = threadIdx.x;
  asm volatile("" : "+v"(tid_o));
  const int jo = kWaveRows * (tid_o >> 6) + 4 * (tid_o & 63);
  if (k <= kMaxCand) {
#pragma unroll
    for (int e4 = 0; e4 < kQuads; ++e4) {
      const uint32_t quad = (selw[(4 * e4) >> 5] >> ((4 * e4) & 31)) & 15u;
      const int c = __builtin_popcount(quad);
      const int incl = wave_incl_scan(c);
      int at = pos + incl - c;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if ((quad >> q) & 1u) cand[at++] = (uint32_t)(jo + 256 * e4 + q);
      pos += __builtin_amdgcn_readlane(incl, 63);
    }
    __syncthreads();
    for (int q = tid; q < filled; q += kTopkThreads) {
      const int j = (int)cand[q];
      out_i[q] = j;
      if (out_s) out_s[q] = src[j];
    }
  } else {
#pragma unroll
    for (int e4 = 0; e4 < kQuads; ++e4) {
      const uint32_t quad = (selw[(4 * e4) >> 5] >> ((4 * e4) & 31)) & 15u;
      const int c = __builtin_popcount(quad);
      const int incl = wave_incl_scan(c);
      int at = pos + incl - c;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if ((quad >> q) & 1u) {
          const int j = jo + 256 * e4 + q;
          out_i[at] = j;
          if (out_s) out_s[at] = src[j];
          ++at;
        }
      }
      pos += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  for (int q = filled + tid; q < k; q += kTopkThreads) {
    out_i[q] = -1;
    if (out_s) out_s[q] = -INFINITY;
  }
}

}  // namespace

void index_groups(int32_t s_q, int32_t* tokens_per_group, int32_t* groups) {
  *groups = (s_q + kMaxTokens - 1) / kMaxTokens;
  *tokens_per_group = (s_q + *groups - 1) / *groups;
}

namespace {

IndexArgs index_args(const IndexLaunch& l) {
  IndexArgs a;
  a.batch = l.batch;
  a.s_q = l.s_q;
  a.h = l.h;
  index_groups(l.s_q, &a.tokens_per_group, &a.groups);
  a.kpool = l.kpool;
  a.is_causal = l.is_causal;
  a.max_pages = l.max_pages;
  a.chunks = (l.max_pages + kChunkPages - 1) / kChunkPages;
  a.n_max = l.max_pages * kPage;
  a.q = l.q;
  a.qs = l.qs;
  a.kv = l.kv;
  a.block_table = l.block_table;
  a.seqlens = l.seqlens;
  a.ws = l.ws;
  a.qsum = l.ws + (int64_t)l.batch * l.s_q * a.n_max;
  a.topk = l.topk;
  a.indices = l.indices;
  a.scores = l.scores;
  return a;
}

}  // namespace

size_t index_workspace_bytes(int32_t batch, int32_t s_q, int32_t max_pages) {
  const size_t tokens = (size_t)batch * (size_t)s_q;
  return align256(tokens * (size_t)max_pages * kPage * sizeof(float)) + align256(tokens * 512 * sizeof(float));
}

hipError_t launch_index_scores(const IndexLaunch& l, hipStream_t stream) {
  if (l.batch == 0) return hipSuccess;
  const IndexArgs a = index_args(l);
  hipLaunchKernelGGL(index_query_kernel, dim3(a.batch * a.s_q), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = a.batch * a.groups * a.chunks;
  const int grid = (total + 7) / 8 * 8;
  switch (a.tokens_per_group) {
    case 1: hipLaunchKernelGGL(index_score_kernel<1>, dim3(grid), dim3(kIdxThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(index_score_kernel<2>, dim3(grid), dim3(kIdxThreads), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(index_score_kernel<3>, dim3(grid), dim3(kIdxThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL(index_score_kernel<4>, dim3(grid), dim3(kIdxThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_index_select(const IndexLaunch& l, hipStream_t stream) {
  if (l.batch == 0) return hipSuccess;
  const IndexArgs a = index_args(l);
  hipLaunchKernelGGL(index_topk_kernel, dim3(a.batch * a.s_q), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
