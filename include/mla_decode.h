/*
 * mla_decode.h -- C ABI of the paged MLA decode library (libmla_decode.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * Operation (multi-head latent attention decode over a paged latent cache).
 * For every batch entry b, new query token i < s_q and head h < h_q:
 *
 *   q[b,i,h,:]   576 values: 512 "NoPE" latent dims then 64 RoPE dims.
 *   K_t          the cached 576-value latent row of logical token t of b; the
 *                only KV head (h_kv = 1) is shared by every query head, and
 *                the value row is its first 512 values (V = K[:, :512]).
 *                Source: "Modular Platform 设计文档全景导读", section 九
 *                (Multi-Head Latent Attention): absorbed MLA reduces to MQA
 *                with Q [heads, 576], one K head of 576 and V = K[..., :512].
 *   paging       logical t -> (t / page_size, t % page_size); the block table
 *                row of b maps the first to a physical page.  Same guide,
 *                section 四 (PagedAttention): divmod then table lookup.
 *   visible set  dense: t < L_b (with is_causal, query i sees t <= L_b-s_q+i);
 *                sparse: the listed indices of (b, i) that lie in [0, L_b).
 *   P_t          softmax_scale * dot(q, K_t)
 *   lse          log2( sum over visible t of 2^P_t )
 *   out          sum over visible t of 2^(P_t - lse) * K_t[0:512]
 *                Source: "为什么 FlashMLA 的解码内核能跑到 660 TFLOPS——内核里的
 *                5 个关键设计", section 上手示例 (the sparse semantics: gather,
 *                scaled scores, base-2 log-sum-exp, base-2 weights).
 *   An empty visible set gives lse = -inf and out = 0.
 *   With MLA_FLAG_NATURAL_BASE the exponent base is e instead of 2 (ordinary
 *   softmax), and lse is the natural log-sum-exp.
 *
 * Work is split across the GPU in three calls per decode step, following the
 * same FlashMLA page's usage section (schedule once per step, decode once
 * per layer) and section 设计 5 (a separate combine kernel merges split
 * results; a tile scheduler spreads requests and blocks over the cores):
 *   mla_decode_get_metadata  (once per step)  -> sched, num_splits
 *   mla_decode_paged         (once per layer) -> out/lse, or split partials
 *   mla_decode_combine       (once per layer) -> merges split partials
 *
 * Conventions for every call:
 *  - All pointers except `p` are device pointers to caller-owned memory; the
 *    library never allocates, frees, copies between host and device or
 *    synchronises.  Kernels are enqueued on `stream` (a hipStream_t; NULL =
 *    the default stream), so the calls can be captured in a hipGraph.
 *  - `p` points to host memory and is read during the call only.
 *  - Arguments are checked on the host before any HIP call.  On failure the
 *    call returns a nonzero mla_status, launches nothing, and
 *    mla_last_error() (per calling thread) names the offending argument.
 *  - Values that live in device memory (cache_seqlens, block_table entries,
 *    indices) are not checked: cache_seqlens[b] must lie in
 *    [0, max_pages_per_seq * page_size] and every block-table entry the
 *    visible tokens reach must lie in [0, num_pages).  Sparse indices outside
 *    [0, L_b) are not errors: they are skipped by definition.
 *  - Calls are thread-safe.  The only library state is a per-device cache
 *    of the compute-unit count and the per-thread error string.
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1, /* malformed argument (named by mla_last_error) */
  MLA_ERR_UNSUPPORTED = 2,      /* well-formed but outside what the kernels do */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4               /* a HIP runtime call failed (message has the HIP error) */
} mla_status;

/* Layout of one cached latent token row. */
enum {
  /* 576 bf16 values, 1152 bytes. */
  MLA_KV_BF16 = 0,
  /* 656 bytes: [0,512) float8 e4m3fn codes of dims 0..511; [512,528) four
   * little-endian float32 scales, scale k covering dims [128k, 128k+128);
   * [528,656) 64 bf16 RoPE values (dims 512..575).  Dequantised value of
   * dim d < 512: bf16_rne(float(code) * scale[d/128]), product in float32.
   * Source: FlashMLA page above, section 设计 2 (FP8 KV cache): 512 e4m3
   * codes with four fp32 per-1x128-tile scales plus 64 bf16 RoPE values,
   * dequantised to bf16 before the bf16 matrix products. */
  MLA_KV_FP8_656 = 1
};

enum {
  MLA_FLAG_NATURAL_BASE = 1 /* softmax in base e; lse in natural-log units */
};

/* Problem description (host memory, plain data). */
typedef struct mla_problem {
  int32_t batch;             /* B >= 0 */
  int32_t s_q;               /* new query tokens per sequence, >= 1 */
  int32_t h_q;               /* query heads, >= 1 */
  int32_t h_kv;              /* must be 1 */
  int32_t d_qk;              /* must be 576 */
  int32_t d_v;               /* must be 512 */
  int32_t page_size;         /* tokens per page; must be 64 */
  int32_t num_pages;         /* pages in the pool, >= 1 */
  int32_t max_pages_per_seq; /* block_table row stride, >= 1 */
  int32_t topk;              /* 0 = dense; > 0 = sparse with `indices` */
  int32_t kv_format;         /* MLA_KV_BF16 or MLA_KV_FP8_656 */
  int32_t is_causal;         /* 0 or 1; must be 0 when topk > 0 */
  int32_t flags;             /* MLA_FLAG_* */
  float softmax_scale;       /* any finite value */
} mla_problem;

/* Number of work units U: dense -> B (each covers s_q*h_q query rows);
 * sparse -> B*s_q (each covers h_q rows, one query token's index list).
 * Returns -1 if `p` is NULL.  Source: the FlashMLA page above, section
 * 上手示例 (the metadata call is sized by the query rows per KV head,
 * s_q*h_q/h_kv, and, for sparse decode, by topk per query token). */
int32_t mla_decode_num_units(const mla_problem* p);

/* Recommended number of split-KV parts for `device` (one workgroup per
 * compute unit for each 128-row group of a unit).  Any value in
 * [1, 65536] may be passed to the calls below instead.  Source: the FlashMLA
 * page above, section 设计 5 (the tile scheduler spreads the requests' blocks
 * evenly over the compute units). */
mla_status mla_decode_num_parts(const mla_problem* p, int device, int32_t* num_parts);

/* Device memory the caller provides for the metadata:
 *   sched       int32 [num_parts * 8]
 *   num_splits  int32 [U + 1]
 * Source: the FlashMLA page above, section 上手示例 (the metadata call
 * returns the tile-scheduler metadata and the per-sequence split counts
 * that every decode call of the step then reads). */
mla_status mla_decode_metadata_size(const mla_problem* p, int32_t num_parts,
                                    size_t* sched_ints, size_t* num_splits_ints);

/* Bytes of device workspace mla_decode_paged/mla_decode_combine need for
 * split partial results (an upper bound computed from host values only).
 * Source: the FlashMLA page above, section 设计 5 (a sequence split over
 * several compute units leaves partial results, each with its log-sum-exp,
 * for a merge step). */
mla_status mla_decode_workspace_bytes(const mla_problem* p, int32_t num_parts, size_t* bytes);

/* Split-KV tile scheduler.  Reads cache_seqlens (int32 [B], device) and
 * writes a balanced assignment of (unit, 64-token block) ranges to
 * `num_parts` parts:
 *   sched[8*part + 0..4] = {begin_unit, begin_block, end_unit, end_block,
 *                           split index of the first segment};
 *     [5] = blocks-per-part budget, [6] = per-segment cost in blocks, [7] = 0.
 *     A part covers blocks from (begin_unit, begin_block) up to, not
 *     including, (end_unit, end_block) in (unit, block) order.
 *   num_splits[u] = number of segments of units before u (num_splits[U] =
 *     total); a unit with one segment is written directly by
 *     mla_decode_paged, a unit with none (empty visible range) by
 *     mla_decode_combine.
 * Run once per decode step; reuse the result for every layer. */
mla_status mla_decode_get_metadata(const mla_problem* p, const int32_t* cache_seqlens,
                                   int32_t num_parts, int32_t* sched, int32_t* num_splits,
                                   void* stream);

/* Decode.  Layouts (row-major, contiguous):
 *   q            bf16  [B, s_q, h_q, 576]           (16-byte aligned)
 *   kv_pool      bytes [num_pages, 64, row bytes]   (16-byte aligned; row
 *                bytes 1152 for MLA_KV_BF16, 656 for MLA_KV_FP8_656)
 *   block_table  int32 [B, max_pages_per_seq]
 *   cache_seqlens int32 [B]
 *   indices      int32 [B, s_q, topk] logical positions; NULL iff topk == 0
 *   sched, num_splits  from mla_decode_get_metadata with the same num_parts
 *   workspace    >= mla_decode_workspace_bytes (16-byte aligned)
 *   out          bf16  [B, s_q, h_q, 512]           (16-byte aligned)
 *   lse          float [B, s_q, h_q]
 * Rows of units with exactly one segment are final after this call; the
 * others need mla_decode_combine.
 * Dense units of at most 32 query rows (s_q * h_q), either cache format,
 * run on a streaming kernel that keeps a whole unit in one workgroup;
 * larger units and sparse calls run on the 128-row tile kernel.  For a given
 * num_parts the results are deterministic: the same bits on every run and
 * under any permutation of the physical pages.
 * With the environment variable MLA_DEBUG_CHECKS set to anything but "" or
 * "0" (read at every call), this call and those built on it first run
 * mla_decode_check_inputs on `stream`, wait for it, and return
 * MLA_ERR_INVALID_ARGUMENT naming the first bad sequence instead of
 * launching the decode.  That mode synchronises the stream (not for graph
 * capture), and its result words live in a static per-GPU array, so such
 * calls that overlap on one GPU race. */
mla_status mla_decode_paged(const mla_problem* p, const void* q, const void* kv_pool,
                            const int32_t* block_table, const int32_t* cache_seqlens,
                            const int32_t* indices, const int32_t* sched, int32_t num_parts,
                            const int32_t* num_splits, void* workspace, size_t workspace_bytes,
                            void* out, float* lse, void* stream);

/* Same as mla_decode_paged, for dense decode over the 656-byte FP8 layout
 * (requires kv_format == MLA_KV_FP8_656 and topk == 0). */
mla_status mla_decode_paged_fp8(const mla_problem* p, const void* q, const void* kv_pool,
                                const int32_t* block_table, const int32_t* cache_seqlens,
                                const int32_t* sched, int32_t num_parts,
                                const int32_t* num_splits, void* workspace,
                                size_t workspace_bytes, void* out, float* lse, void* stream);

/* Same as mla_decode_paged, for top-k sparse decode over the 656-byte FP8
 * layout (requires kv_format == MLA_KV_FP8_656, topk > 0 and indices). */
mla_status mla_decode_sparse_fp8(const mla_problem* p, const void* q, const void* kv_pool,
                                 const int32_t* block_table, const int32_t* cache_seqlens,
                                 const int32_t* indices, const int32_t* sched,
                                 int32_t num_parts, const int32_t* num_splits, void* workspace,
                                 size_t workspace_bytes, void* out, float* lse, void* stream);

/* Size of the static device scratch behind mla_decode_paged_noalloc: 96 MiB.
 * The split partials take 1,028 bytes per (segment slot, row), with
 * num_parts + units slots of s_q * h_q rows (topk > 0: h_q rows); e.g. batch
 * 128, s_q 2, h_q 128 over 128 parts needs (128 + 128) x 256 x 1,028 bytes
 * = 64.3 MiB. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/* Decode and combine in one call that allocates nothing, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments are those of
 * mla_decode_paged without the workspace; `out` and `lse` are final on
 * return of the launched work (the combine runs on the same stream).  The
 * split partials go to a static device array of MLA_NOALLOC_SCRATCH_BYTES
 * bytes inside the library, one per GPU, held until the process ends; the
 * call makes no allocation of any kind.  Results equal those of
 * mla_decode_paged followed by mla_decode_combine with the same metadata,
 * bit for bit.
 *   Errors: as mla_decode_paged; MLA_ERR_WORKSPACE_TOO_SMALL when
 *   mla_decode_workspace_bytes for (p, num_parts) exceeds the scratch (a
 *   smaller num_parts or the workspace entry point then applies).
 *   Nothing in the scratch has to start at zero: every partial the combine
 *   reads is written by the decode launch of the same call.
 *   All calls on one GPU share that GPU's scratch, which keeps the last
 *   call's contents: calls that overlap on one GPU (several streams or host
 *   threads) race, and the caller must order them.
 *   The first call on a device takes the array's device address
 *   (hipGetSymbolAddress, with the stream's device current) and keeps it. */
mla_status mla_decode_paged_noalloc(const mla_problem* p, const void* q, const void* kv_pool,
                                    const int32_t* block_table, const int32_t* cache_seqlens,
                                    const int32_t* indices, const int32_t* sched, int32_t num_parts,
                                    const int32_t* num_splits, void* out, float* lse, void* stream);

/* Merge split partial results by their log-sum-exp:
 *   M = max_s lse_s,  lse = M + log2(sum_s 2^(lse_s - M)),
 *   out = sum_s 2^(lse_s - lse) * out_s.
 * Source: "Modular Platform 设计文档全景导读", sections 六 and 七 (online
 * softmax: results over disjoint key ranges merge through the running max
 * and a correction factor).  Writes out/lse of every unit that has zero or
 * at least two segments. */
mla_status mla_decode_combine(const mla_problem* p, int32_t num_parts, const int32_t* num_splits,
                              const void* workspace, size_t workspace_bytes, void* out,
                              float* lse, void* stream);

/* Device-side check of the preconditions the decode calls leave unchecked
 * (they read device memory): every cache_seqlens[b] in
 * [0, max_pages_per_seq * 64], and every block-table entry a visible
 * position can reach (block_table[b][j] for j < ceil(L_b / 64)) in
 * [0, num_pages).  For sparse problems the same pages bound what listed
 * indices can reach.  Writes result[0] = number of sequences that violate
 * either, result[1] = the first such sequence (-1 if none); result is a
 * device int32[2].  Meant for debugging and input validation outside the
 * hot loop (one workgroup; cost grows with batch * pages).  Source: the
 * MAX kernels guide, "max.nn.kernels 内核封装模块全解析", section 输入校验
 * (inputs are validated and the offending argument reported). */
mla_status mla_decode_check_inputs(const mla_problem* p, const int32_t* block_table,
                                   const int32_t* cache_seqlens, int32_t* result, void* stream);

/* FP8 KV writer: quantises new latent tokens into the 656-byte layout
 * (MLA_KV_FP8_656) and stores each at its paged slot.
 *   kv_new       bf16  [batch, n_new, 576]  (16-byte aligned; device)
 *   start_pos    int32 [batch]  logical position of token 0 of each sequence
 *   block_table  int32 [batch, max_pages_per_seq]
 *   kv_pool      bytes [num_pages, 64, 656]  (16-byte aligned; written in place)
 * Token j of sequence b goes to logical position t = start_pos[b] + j, i.e.
 * slot t % 64 of page block_table[b][t / 64] ("Modular Platform 设计文档全景
 * 导读", section 四: divmod of the token index by the page size, then the
 * block table).  Per 1x128 tile k of the 512 NoPE values: amax = max |x|,
 * scale_k = amax / 448 (fp32 division), code = e4m3fn(x / scale_k) (fp32
 * division, nearest code with ties to even, saturated to +-448); a tile with
 * amax = 0 gets scale 0 and code 0x00 throughout.  The 64 RoPE values are
 * copied as bf16.  Layout source: the FlashMLA page above, section 设计 2
 * (1x128-tile fp32 scales, e4m3 codes, bf16 RoPE); the rounding and the
 * amax/448 scale are this library's reading of it.
 * Inputs must be finite.  Tokens whose position is negative, whose page
 * index t / 64 is >= max_pages_per_seq or whose block-table entry lies
 * outside [0, num_pages) are skipped (not errors; device values are not
 * checked on the host).  If two tokens map to the same slot, which one is
 * stored is unspecified.  Only the addressed rows are written; the call
 * neither allocates nor synchronises.  page_size must be 64. */
mla_status mla_kv_quantize_fp8(int32_t batch, int32_t n_new, int32_t page_size,
                               int32_t num_pages, int32_t max_pages_per_seq, const void* kv_new,
                               const int32_t* start_pos, const int32_t* block_table,
                               void* kv_pool, void* stream);

/* Sparse prefill.  Source: the FlashMLA page above, section 上手示例: the
 * sparse prefill call takes q [s_q, h_q, 576], a flat latent cache
 * kv [s_kv, 1, 576] (no batch dimension, no block table; one KV head) and
 * indices [s_q, 1, topk]; per query token i it gathers the rows
 * kv[indices[i][k]], scores P = scale * q.K, and returns
 * lse = log2(sum 2^P) and out = sum 2^(P - lse) * K[0:512] (base e with
 * MLA_FLAG_NATURAL_BASE).  Entries outside [0, s_kv) are skipped;
 * duplicates count with multiplicity; an empty list gives lse = -inf and
 * out = 0.
 *   q        bf16  [s_q, h_q, 576]        (16-byte aligned; device)
 *   kv       bytes [s_kv, row bytes]      (16-byte aligned; 1152 for
 *            MLA_KV_BF16, 656 for MLA_KV_FP8_656)
 *   indices  int32 [s_q, topk]
 *   workspace >= mla_sparse_prefill_workspace_bytes (256-byte aligned)
 *   out      bf16  [s_q, h_q, 512]        (16-byte aligned)
 *   lse      float [s_q, h_q]
 *   num_parts  split-KV parts per launch, in [1, 65536]; the value
 *            mla_decode_num_parts gives for a batch-1 sparse problem with
 *            the same h_q fills the GPU.
 * It runs the sparse decode kernels (batch 1, one work unit per query
 * token, chunks of at most 2048 query tokens) with an identity block table
 * (page p = rows 64p..64p+63) that it writes into the workspace first.  All
 * work is enqueued on `stream`; nothing is allocated. */
mla_status mla_sparse_prefill_workspace_bytes(int32_t s_q, int32_t h_q, int32_t s_kv, int32_t topk,
                                              int32_t kv_format, int32_t num_parts, size_t* bytes);
mla_status mla_sparse_prefill(int32_t s_q, int32_t h_q, int32_t s_kv, int32_t topk,
                              int32_t kv_format, int32_t flags, float softmax_scale,
                              const void* q, const void* kv, const int32_t* indices,
                              int32_t num_parts, void* workspace, size_t workspace_bytes,
                              void* out, float* lse, void* stream);

/* Message of the last failed call on this thread ("" if none); it names
 * the offending argument.  Source: "max.nn.kernels 内核封装模块全解析",
 * section 输入校验 (the kernel wrappers reject malformed inputs before any
 * kernel runs and report which argument is wrong). */
const char* mla_last_error(void);

/* Name of the kernel mla_decode_paged launches for this problem
 * ("decode_kernel": 128-row tiles; "decode_small_kernel": dense units of at
 * most 32 query rows), or NULL if the problem is invalid.  A helper for
 * profiling tools that look kernels up by name; it reads host memory only. */
const char* mla_decode_kernel_name(const mla_problem* p);

/* Shader-clock probe, a measurement helper (not part of the decode path).
 * Launches `workgroups` workgroups that keep the matrix cores busy for
 * `spins` iterations of four bf16 MFMAs per wave and writes, per workgroup w,
 * out[2w] = elapsed shader-clock cycles (s_memtime) and out[2w+1] = elapsed
 * ticks of the 100 MHz constant-rate counter (s_memrealtime) over the same
 * interval; cycles / ticks * 100 MHz is the shader clock under that load.
 * `out` is a device int64 [2 * workgroups], 8-byte aligned. */
mla_status mla_clock_probe(int64_t* out, int32_t workgroups, int32_t spins, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
