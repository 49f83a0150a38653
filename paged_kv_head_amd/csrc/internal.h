// Internal declarations shared by the translation units of libmla_decode.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kPage = 64;          // tokens per page == keys per tile
constexpr int kRowsPerGroup = 128; // query rows one workgroup owns
// Dense units of at most kSmallMaxRows rows (bf16 cache) or
// kSmallMaxRowsFp8 rows (FP8 cache) run on the small-head kernel (one
// workgroup per part, all rows of the unit in it).
constexpr int kSmallMaxRows = 32;
constexpr int kSmallMaxRowsFp8 = 32;
constexpr int kSplitPenalty = 3;   // scheduler cost of one segment, in blocks (measured: a
                                    // segment's prologue + epilogue ~ 3 tiles)
constexpr int kMaxUnits = 16384;   // metadata kernel keeps per-unit arrays in LDS
constexpr int kMaxParts = 65536;

struct Shape {
  int32_t batch, s_q, h_q, topk, kv_format, is_causal, natural;
  int32_t num_pages, max_pages;
  int32_t units;  // U
  int32_t rows;   // query rows per unit (R)
  int32_t groups; // row groups per unit: ceil(R / rows per workgroup of the kernel that runs it)
  float scale_log2;  // exponent multiplier: softmax_scale, times log2(e) for base e
  float inv_h_q;     // 1 / h_q (query position of a row without an integer division)
};

struct DecodeArgs {
  Shape s;
  const uint16_t* q;
  const uint8_t* kv;
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* indices;
  const int32_t* sched;
  const int32_t* num_splits;
  int32_t num_parts;
  float* ws_lse;  // [slots * R]
  uint16_t* ws_o;  // [slots * R * 512] bf16, normalised split outputs
  uint16_t* out;
  float* lse;
};

// Workspace layout: split lse block (fp32), then split output block (bf16);
// both for num_parts + U slots of R rows, each block 256-byte aligned.
inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
inline size_t ws_slots(int32_t num_parts, int32_t units) { return (size_t)num_parts + (size_t)units; }
inline size_t ws_lse_bytes(size_t slots, int32_t rows) {
  return align256(slots * (size_t)rows * sizeof(float));
}
inline size_t ws_o_bytes(size_t slots, int32_t rows) {
  return align256(slots * (size_t)rows * kDv * sizeof(uint16_t));
}
inline size_t ws_total_bytes(int32_t num_parts, int32_t units, int32_t rows) {
  const size_t slots = ws_slots(num_parts, units);
  return ws_lse_bytes(slots, rows) + ws_o_bytes(slots, rows);
}

hipError_t launch_metadata(const Shape& s, const int32_t* seqlens, int32_t num_parts,
                           int32_t* sched, int32_t* num_splits, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Dense units of at most kSmallMaxRows query rows (either cache format) run on a
// kernel built for the HBM-bound small-head shape; same inputs, outputs and
// workspace.
bool small_decode_applies(const Shape& s);
hipError_t launch_decode_small(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_combine(const Shape& s, const int32_t* num_splits, const float* ws_lse,
                          const uint16_t* ws_o, uint16_t* out, float* lse, hipStream_t stream);
hipError_t launch_kv_quantize_fp8(int32_t batch, int32_t n_new, int32_t num_pages,
                                  int32_t max_pages, const uint16_t* kv_new,
                                  const int32_t* start_pos, const int32_t* block_table,
                                  uint8_t* kv_pool, hipStream_t stream);
hipError_t launch_check_inputs(const Shape& s, const int32_t* block_table, const int32_t* seqlens,
                               int32_t* result, hipStream_t stream);
hipError_t launch_clock_probe(int64_t* out, int32_t workgroups, int32_t spins, hipStream_t stream);
hipError_t launch_identity_table(int32_t* table, int32_t pages, int32_t* seqlen, int32_t s_kv,
                                 hipStream_t stream);

// FP8 top-k indexer (indexer.hip).
struct IndexLaunch {
  int32_t batch, s_q, h, kpool, is_causal, max_pages, topk;
  const uint8_t* q;
  const float* qs;
  const uint8_t* kv;
  const int32_t* block_table;
  const int32_t* seqlens;
  float* ws;  // index_workspace_bytes: scores, then head-summed queries
  int32_t* indices;
  float* scores;  // may be null
};
// Pages of one sequence a score workgroup of the indexer covers.
constexpr int kIndexChunkPages = 32;
// Query tokens per score workgroup and workgroups per sequence.
void index_groups(int32_t s_q, int32_t* tokens_per_group, int32_t* groups);
// Workspace of the indexer: fp32 scores [batch, s_q, 64 * max_pages], then
// the head-summed queries [batch, s_q, 512] (fp32), each 256-byte aligned.
size_t index_workspace_bytes(int32_t batch, int32_t s_q, int32_t max_pages);
// Scores of every row of the pages holding visible rows into l.ws, then the
// selection from l.ws (the two kernels of the indexer).
hipError_t launch_index_scores(const IndexLaunch& l, hipStream_t stream);
hipError_t launch_index_select(const IndexLaunch& l, hipStream_t stream);

// Sparse prefill runs the decode path over chunks of at most this many query
// tokens (each a decode unit), which bounds the split workspace.
constexpr int kPrefillChunk = 2048;

}  // namespace mla
