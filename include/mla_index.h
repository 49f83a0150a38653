/* FP8 top-k indexer of libmla_decode.so: the step that picks, for every
 * query token, the cached rows a top-k sparse decode (mla_decode_sparse_fp8)
 * then attends to.
 *
 * Source: "max.nn.kernels 内核封装模块全解析", section 稀疏注意力（MSA）与
 * MLA 索引内核 (mla_fp8_index_top_k): an FP8 query is scored against the
 * quantised K cache with their scales, the scores are aggregated over heads
 * and masked, and the call returns per query token the int32 indices of the
 * top-k keys, -1 where there is no valid key; with kpool > 1 the cache keeps
 * one pooled key per kpool tokens and the indices are pool ids.
 *
 * Definition.  The passage leaves several steps open; this library reads
 * them as follows.
 *   - Quantised K.  Row j of the cache is a 656-byte row of the
 *     MLA_KV_FP8_656 layout.  Its quantised part is the 512 e4m3fn codes
 *     c_j[d] and the four fp32 tile scales s_j[t], tile t covering dims
 *     [128t, 128t + 128).  The 64 bf16 RoPE values are not quantised and take
 *     no part in the FP8 score.
 *   - FP8 query.  Token (b, i) has, per index head h, 512 e4m3fn codes
 *     q[b][i][h][d] and four fp32 tile scales qs[b][i][h][t] on the same
 *     tiling (the layout of the cache's quantised part).
 *   - Score of row j for token (b, i), summed over the heads:
 *       S = sum_h sum_t qs[b][i][h][t] * s_j[t]
 *                       * sum_{d in tile t} e4m3(q[b][i][h][d]) * e4m3(c_j[d]).
 *   - Rows.  Row j of sequence b is slot j % 64 of page
 *     block_table[b][j / 64] (with kpool > 1, the rows of the pooled cache).
 *   - Mask.  With t_max = L_b - 1, or L_b - s_q + i when is_causal (the
 *     bottom-right alignment of the decode calls), the visible rows are
 *     j < ceil((t_max + 1) / kpool): a pooled row is visible once a token
 *     it covers is.  No row is visible when t_max < 0.
 *   - Selection.  The min(topk, visible) visible rows of largest S; equal
 *     scores are broken toward the smaller j; a NaN score ranks below every
 *     other score.
 *   - Output.  indices[b][i][0..] holds the selected rows in ascending j,
 *     then -1 up to topk.  scores (optional) holds S of each selected row,
 *     -inf beside each -1.
 * The sum over heads is linear, so the kernels take it first: per query
 * token Qsum[d] = sum_h qs[h][t(d)] * e4m3(q[h][d]) (fp32, in a fixed order),
 * then S_j = sum_t s_j[t] * sum_{d in tile t} e4m3(c_j[d]) * Qsum[d] (fp32;
 * every code converts to fp32 exactly).  Selection is made on those fp32
 * scores.  For a given problem the results are the same bits on every run.
 */
#ifndef MLA_INDEX_H_
#define MLA_INDEX_H_

#include "mla_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mla_index_problem {
  int32_t batch;             /* B >= 0 */
  int32_t s_q;               /* query tokens per sequence, >= 1 */
  int32_t h;                 /* index heads, 1..4096 */
  int32_t d;                 /* must be 512: the quantised part of a row */
  int32_t page_size;         /* must be 64 */
  int32_t num_pages;         /* pages in the pool, >= 1 */
  int32_t max_pages_per_seq; /* block_table row stride; 64 * this <= 65536 */
  int32_t topk;              /* 1 .. 64 * max_pages_per_seq */
  int32_t kpool;             /* tokens per cached (pooled) row, >= 1 */
  int32_t is_causal;         /* 0 or 1 */
} mla_index_problem;

/* Bytes of device workspace mla_fp8_index_top_k needs: fp32 scores of every
 * row a sequence can hold, [B, s_q, 64 * max_pages_per_seq], then the
 * head-summed query of every token, [B, s_q, 512] fp32 (each part 256-byte
 * aligned).  Host values only.  Errors: MLA_ERR_INVALID_ARGUMENT / MLA_ERR_UNSUPPORTED as for the
 * call below. */
mla_status mla_fp8_index_workspace_bytes(const mla_index_problem* p, size_t* bytes);

/* The indexer.  Layouts (row-major, contiguous):
 *   q_fp8         uint8 [B, s_q, h, 512] e4m3fn codes   (16-byte aligned)
 *   q_scale       float [B, s_q, h, 4] tile scales      (16-byte aligned)
 *   kv_pool       bytes [num_pages, 64, 656], MLA_KV_FP8_656 rows (16-byte aligned)
 *   block_table   int32 [B, max_pages_per_seq]; the entries of the pages that
 *                 hold visible rows must lie in [0, num_pages)
 *   cache_seqlens int32 [B], tokens per sequence, in [0, 64 * kpool *
 *                 max_pages_per_seq] (mla_decode_check_inputs checks the
 *                 kpool = 1 case on the device); the kernels read at most
 *                 the 64 * max_pages_per_seq rows a table row holds
 *   workspace     >= mla_fp8_index_workspace_bytes (16-byte aligned)
 *   indices       int32 [B, s_q, topk]                 (output)
 *   scores        float [B, s_q, topk] or NULL         (output)
 * All device memory is the caller's; two kernels run on `stream` (scores,
 * then selection) and the call returns without waiting for them.
 * Errors: MLA_ERR_INVALID_ARGUMENT (named argument), MLA_ERR_UNSUPPORTED
 * (d != 512, page_size != 64, h > 4096, more than 65536 rows per sequence),
 * MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP (launch failure). */
mla_status mla_fp8_index_top_k(const mla_index_problem* p, const void* q_fp8, const float* q_scale,
                               const void* kv_pool, const int32_t* block_table,
                               const int32_t* cache_seqlens, void* workspace,
                               size_t workspace_bytes, int32_t* indices, float* scores,
                               void* stream);

/* The two phases of mla_fp8_index_top_k, for callers that want every row's
 * score or time the phases apart.  mla_fp8_index_scores writes the fp32 score
 * S of every row of the pages that hold visible rows into the workspace,
 * [B, s_q, 64 * max_pages_per_seq] (entries of rows that are not visible are
 * unspecified); mla_fp8_index_select then writes indices and scores from it
 * exactly as mla_fp8_index_top_k does.  Arguments, layouts and errors as
 * there; the workspace must be the one the score phase filled, with the same
 * problem and cache_seqlens. */
mla_status mla_fp8_index_scores(const mla_index_problem* p, const void* q_fp8, const float* q_scale,
                                const void* kv_pool, const int32_t* block_table,
                                const int32_t* cache_seqlens, void* workspace,
                                size_t workspace_bytes, void* stream);
mla_status mla_fp8_index_select(const mla_index_problem* p, const int32_t* cache_seqlens,
                                const void* workspace, size_t workspace_bytes, int32_t* indices,
                                float* scores, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_INDEX_H_ */
