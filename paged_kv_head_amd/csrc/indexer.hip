// FP8 top-k indexer for gfx950: per query token, the cached rows of largest
// head-summed FP8 score ("max.nn.kernels 内核封装模块全解析", section
// 稀疏注意力（MSA）与 MLA 索引内核, mla_fp8_index_top_k).  The definition and
// its readings are in include/mla_index.h.
//
// Two kernels on the caller's stream:
//   index_score_kernel  S[b][i][j] for every row j of the pages that hold
//                       visible rows (fp32, into the workspace);
//   index_topk_kernel   per (b, i): the top-k visible rows by S, ascending j,
//                       -1 fill.
//
// Scores.  A workgroup (4 waves) owns one sequence b, a group of query
// tokens (their heads padded to a multiple of 16 rows, at most 256 rows) and
// a chunk of kChunkPages pages.  Q rows are the A operand of
// v_mfma_f32_32x32x64_f8f6f4 (32 query rows x 64 dims of e4m3 codes, eight
// VGPRs per lane; all 512 dims of the wave's row blocks stay in registers);
// the cache rows are the B operand (64 dims x 32 keys), read from LDS.  The
// fp32 result of a 128-dim tile (two MFMAs) is scaled per row by the query's
// tile scale and summed over the lane's 16 rows, then scaled by the key's
// tile scale: S_j += s_j[t] * sum_rows qs[row][t] * P_t[row][j].  A lane of
// a 32x32 result holds 16 rows of one key: rows 0..15 of the block in
// elements 0..7 (both lane halves), rows 16..31 in 8..15, so with heads
// padded to 16 every half block belongs to one query token.
//
// Cache rows are staged whole-page, 528 bytes per row (the 512 codes and
// the four scales; the bf16 RoPE part is not read) at a 528-byte pitch:
// 16 consecutive rows start on 16 distinct 16-byte bank groups, so the B
// operand reads (16 rows at one offset) are conflict-free.  A page is 33
// direct global->LDS copies of 1 KiB, spread over the four waves, into a
// ring of kRing pages kept kRing - 1 pages ahead.
#include "../../include/mla_index.h"
#include "internal.h"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kIdxThreads = 256;
constexpr int kRowBytes = 656;           // cache row (MLA_KV_FP8_656)
constexpr int kStageRow = 528;           // staged part: codes + scales
constexpr int kStagePage = kPage * kStageRow;  // 33792
constexpr int kPageCopies = kStagePage / 1024;  // 33
constexpr int kRing = 4;
constexpr int kMaxRows = 256;            // query rows of a workgroup
constexpr int kCopiesPerWave = 8;        // waves 1..3; wave 0 issues 9
static_assert(kPageCopies == 4 * kCopiesPerWave + 1, "copy split");

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

struct IndexArgs {
  int32_t batch, s_q, h, h16, tokens_per_group, groups, rows, row_blocks;
  int32_t kpool, is_causal, max_pages, chunks, n_max;
  const uint8_t* q;
  const float* qs;
  const uint8_t* kv;
  const int32_t* block_table;
  const int32_t* seqlens;
  float* ws;  // [B, s_q, n_max]
  int32_t topk;
  int32_t* indices;
  float* scores;
};

constexpr int kChunkPages = 32;

__global__ void __launch_bounds__(kIdxThreads, 1) index_score_kernel(IndexArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * kStagePage];
  __shared__ __attribute__((aligned(16))) float qs_lds[4 * kMaxRows];  // [tile][row]
  __shared__ __attribute__((aligned(16))) float part[16 * kPage];       // [16-row group][key]

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; XCD x
  // takes a contiguous run of (sequence, group, chunk) items, so the chunks
  // of one sequence share that XCD's L2 for their query.
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
  const int nvis = visible_rows(L, a.s_q, i0 + ntok - 1, a.kpool, a.is_causal);  // the group's most
  const int p_begin = chunk * kChunkPages;
  const int p_end = min(p_begin + kChunkPages, ceil_div(nvis, kPage));
  if (p_begin >= p_end) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;  // lane half
  cint32* bt = (cint32*)(a.block_table + (int64_t)b * a.max_pages);

  // Direct copies of page p into ring slot p % kRing.  Copy c (of 33) fills
  // LDS bytes [1024c, 1024c + 1024) of the slot: lane L's 16 bytes are byte
  // o = 1024c + 16L of the staged page, row o / 528, offset o % 528.
  const uint32_t ring_base = lds_u32(ring);
  auto issue_page = [&](int p) {
    const int pg = bt[p];
    const uint8_t* src = a.kv + (int64_t)pg * (kPage * kRowBytes);
    const uint32_t slot = ring_base + (uint32_t)(p % kRing) * kStagePage;
    const int ncopy = wave == 0 ? kCopiesPerWave + 1 : kCopiesPerWave;
    for (int k = 0; k < ncopy; ++k) {
      const int c = wave + 4 * k;
      const uint32_t o = 1024u * c + 16u * lane;
      const uint32_t r = (o * 7944u) >> 22;  // o / 528 for o < 33792
      const uint32_t voff = r * kRowBytes + (o - r * kStageRow);
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(slot + 1024u * c);
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff), "s"(src), "s"(m0) : "memory", "m0");
    }
    // wave 0's ninth copy is accounted for as if it were one of the next
    // page's: waiting for all but 2 * kCopiesPerWave copies then waits for a
    // little more than the page on wave 0, exactly the page on the others
  };

  // Query: scales into LDS ([tile][row], 0 for padding rows), codes of the
  // wave's row blocks (w and w + 4) into registers.
  for (int rr = tid; rr < kMaxRows; rr += kIdxThreads) {
    const int tl = rr / a.h16, head = rr % a.h16;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (rr < a.rows && tl < ntok && head < a.h)
      v = *reinterpret_cast<const f32x4*>(a.qs + (((int64_t)b * a.s_q + i0 + tl) * a.h + head) * 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) qs_lds[t * kMaxRows + rr] = v[t];
  }
  i32x8 qf[2][8];
#pragma unroll
  for (int lb = 0; lb < 2; ++lb) {
    const int rb = wave + 4 * lb;
    const int rr = 32 * rb + (lane & 31);
    const int tl = rr / a.h16, head = rr % a.h16;
    const bool ok = rb < a.row_blocks && rr < a.rows && tl < ntok && head < a.h;
    const uint8_t* qrow = a.q + (((int64_t)b * a.s_q + i0 + (ok ? tl : 0)) * a.h + (ok ? head : 0)) * 512 + 32 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      i32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (ok) {
        lo = *reinterpret_cast<const i32x4*>(qrow + 64 * s);
        hi = *reinterpret_cast<const i32x4*>(qrow + 64 * s + 16);
      }
      qf[lb][s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  const bool has0 = wave < a.row_blocks, has1 = wave + 4 < a.row_blocks;  // wave-uniform
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
    float acc[2][2][2] = {};  // [local row block][key block][row half]
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 qv[2][4];
#pragma unroll
      for (int lb = 0; lb < 2; ++lb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          qv[lb][gq] = *reinterpret_cast<const f32x4*>(
              &qs_lds[t * kMaxRows + 32 * (wave + 4 * lb) + 8 * gq + 4 * hh]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint8_t* krow = st + (32 * kb + (lane & 31)) * kStageRow;
        const float ks = *reinterpret_cast<const float*>(krow + 512 + 4 * t);
        i32x8 kf[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(krow + 128 * t + 64 * u + 32 * hh);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(krow + 128 * t + 64 * u + 32 * hh + 16);
          kf[u] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int lb = 0; lb < 2; ++lb) {
          if ((lb == 0 && !has0) || (lb == 1 && !has1)) continue;
          f32x16 pr = {};
          pr = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[lb][2 * t], kf[0], pr, 0, 0, 0, 0, 0, 0);
          pr = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[lb][2 * t + 1], kf[1], pr, 0, 0, 0, 0, 0, 0);
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int v = 0; v < 8; ++v) s0 = __builtin_fmaf(qv[lb][v >> 2][v & 3], pr[v], s0);
#pragma unroll
          for (int v = 8; v < 16; ++v) s1 = __builtin_fmaf(qv[lb][v >> 2][v & 3], pr[v], s1);
          acc[lb][kb][0] = __builtin_fmaf(ks, s0, acc[lb][kb][0]);
          acc[lb][kb][1] = __builtin_fmaf(ks, s1, acc[lb][kb][1]);
        }
      }
    }
    // Both lane halves hold 8 of the 16 rows of a half block: add them, then
    // lanes 0..31 publish row half 0 and lanes 32..63 row half 1.
#pragma unroll
    for (int lb = 0; lb < 2; ++lb) {
      if ((lb == 0 && !has0) || (lb == 1 && !has1)) continue;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float v[2];
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[lb][kb][rh]),
                                                          __float_as_uint(acc[lb][kb][rh]), false, false);
          v[rh] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
        const int grp = 2 * (wave + 4 * lb) + hh;
        part[grp * kPage + 32 * kb + (lane & 31)] = hh ? v[1] : v[0];
      }
    }
    IDX_BARRIER();
    // Sum the 16-row groups of each token and store the page's scores.
    const int gpt = a.h16 / 16;  // 16-row groups per token
    for (int e = tid; e < ntok * kPage; e += kIdxThreads) {
      const int tl = e / kPage, key = e % kPage;
      float sum = 0.f;
      for (int q = 0; q < gpt; ++q) sum += part[(tl * gpt + q) * kPage + key];
      ws_b[(int64_t)tl * a.n_max + p * kPage + key] = sum;
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

// Workgroup sum of one int per wave (16 waves), through LDS.
__device__ inline int block_sum16(int wave_value, int* red, int wave, int lane) {
  if (lane == 0) red[wave] = wave_value;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

__global__ void __launch_bounds__(kTopkThreads, 1) index_topk_kernel(IndexArgs a) {
  __shared__ int red[kTopkThreads / 64];
  __shared__ int wave_base[kTopkThreads / 64];
  const int row = blockIdx.x;  // (b, i)
  const int b = row / a.s_q, i = row % a.s_q;
  const int L = a.seqlens[b];
  const int n = min(visible_rows(L, a.s_q, i, a.kpool, a.is_causal), a.n_max);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* src = a.ws + (int64_t)row * a.n_max;
  const int j0 = tid * kPerThread;

  uint32_t key[kPerThread];
#pragma unroll
  for (int e4 = 0; e4 < kPerThread / 4; ++e4) {
    const int j = j0 + 4 * e4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (j < n) v = *reinterpret_cast<const f32x4*>(src + j);  // rows past n are never read
#pragma unroll
    for (int q = 0; q < 4; ++q) key[4 * e4 + q] = (j + q < n) ? score_key(v[q]) : 0u;
  }

  // Threshold: the largest T with #{key >= T} >= k (n > k), else take all.
  const int k = a.topk;
  uint32_t T = 1u;
  int need_eq = 0;
  if (n > k) {
    T = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int c = 0;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[e] >= cand));
      if (block_sum16(c, red, wave, lane) >= k) T = cand;
    }
    int cg = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) cg += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[e] > T));
    need_eq = k - block_sum16(cg, red, wave, lane);
  }

  // Ties at T go to the smallest rows: rank them in row order (a thread's
  // rows are contiguous, threads in order).
  int eq = 0;
  if (n > k) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) eq += key[e] == T ? 1 : 0;
  }
  auto exclusive_scan = [&](int v) {
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    if (tid == 0) {
      int s = 0;
      for (int w = 0; w < kTopkThreads / 64; ++w) {
        wave_base[w] = s;
        s += red[w];
      }
    }
    __syncthreads();
    const int r = wave_base[wave] + incl - v;
    __syncthreads();
    return r;
  };
  int eq_before = exclusive_scan(eq);
  int nsel = 0;
  uint64_t selmask = 0;  // bit e: row j0 + e selected
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    bool sel;
    if (n > k) {
      sel = key[e] > T;
      if (key[e] == T) {
        sel = eq_before < need_eq;
        ++eq_before;
      }
    } else {
      sel = key[e] != 0u;
    }
    if (sel) {
      selmask |= 1ull << e;
      ++nsel;
    }
  }
  int pos = exclusive_scan(nsel);
  int32_t* out_i = a.indices + (int64_t)row * k;
  float* out_s = a.scores ? a.scores + (int64_t)row * k : nullptr;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if ((selmask >> e) & 1ull) {
      out_i[pos] = j0 + e;
      if (out_s) out_s[pos] = src[j0 + e];
      ++pos;
    }
  }
  const int filled = min(k, n);
  for (int q = filled + tid; q < k; q += kTopkThreads) {
    out_i[q] = -1;
    if (out_s) out_s[q] = -INFINITY;
  }
}

}  // namespace

bool index_shape(int32_t h, int32_t s_q, int32_t* h16, int32_t* tokens_per_group, int32_t* groups) {
  if (h < 1 || h > kMaxRows) return false;
  *h16 = (h + 15) / 16 * 16;
  *tokens_per_group = max(1, min(s_q, kMaxRows / *h16));
  *groups = (s_q + *tokens_per_group - 1) / *tokens_per_group;
  return true;
}

hipError_t launch_index(const IndexLaunch& l, hipStream_t stream) {
  IndexArgs a;
  a.batch = l.batch;
  a.s_q = l.s_q;
  a.h = l.h;
  index_shape(l.h, l.s_q, &a.h16, &a.tokens_per_group, &a.groups);
  a.rows = a.tokens_per_group * a.h16;
  a.row_blocks = (a.rows + 31) / 32;
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
  a.topk = l.topk;
  a.indices = l.indices;
  a.scores = l.scores;
  if (l.batch == 0) return hipSuccess;
  const int total = a.batch * a.groups * a.chunks;
  const int grid = (total + 7) / 8 * 8;
  hipLaunchKernelGGL(index_score_kernel, dim3(grid), dim3(kIdxThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(index_topk_kernel, dim3(a.batch * a.s_q), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
