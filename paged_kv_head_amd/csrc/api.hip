// C ABI of libmla_decode.so: host-side validation and kernel launches.
// Every check runs before any HIP call; a failed check returns a status and
// records a message naming the argument (the wrappers in the MAX kernels
// guide, "max.nn.kernels 内核封装模块全解析", section 输入校验, reject bad
// tensors by argument name before the kernel runs; scalars such as the
// softmax scale travel as host float32 values, same section).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/mla_decode.h"
#include "../../include/mla_index.h"
#include "internal.h"

// Scratch of mla_decode_paged_noalloc: the split partials (lse block, then
// bf16 output block, as in a caller's workspace) of its decode and combine
// launches.  Every GPU the library runs on holds its own copy until the
// process ends.  In host code this name is a host-side stand-in: only the
// device address taken by scratch_address() below may reach a kernel.
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];
// Result words of the input check that MLA_DEBUG_CHECKS runs before a decode
// launch (one pair per GPU; reached only through symbol_address() below).
static __device__ __align__(256) int32_t check_words[2];

namespace {

thread_local char g_err[512] = "";

mla_status fail(mla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

mla_status ok() {
  g_err[0] = '\0';
  return MLA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Validates the problem and fills the kernel-side shape.
mla_status check_problem(const mla_problem* p, mla::Shape* s) {
  if (!p) return fail(MLA_ERR_INVALID_ARGUMENT, "p: NULL problem");
  if (p->batch < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "batch: must be >= 0 (got %d)", p->batch);
  if (p->s_q < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "s_q: must be >= 1 (got %d)", p->s_q);
  if (p->h_q < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "h_q: must be >= 1 (got %d)", p->h_q);
  if (p->h_kv != 1) return fail(MLA_ERR_UNSUPPORTED, "h_kv: only 1 latent KV head is supported (got %d)", p->h_kv);
  if (p->d_qk != mla::kDqk) return fail(MLA_ERR_UNSUPPORTED, "d_qk: must be 576 (got %d)", p->d_qk);
  if (p->d_v != mla::kDv) return fail(MLA_ERR_UNSUPPORTED, "d_v: must be 512 (got %d)", p->d_v);
  if (p->page_size != mla::kPage) return fail(MLA_ERR_UNSUPPORTED, "page_size: must be 64 (got %d)", p->page_size);
  if (p->num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages: must be >= 1 (got %d)", p->num_pages);
  if (p->max_pages_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq: must be >= 1 (got %d)", p->max_pages_per_seq);
  if (p->topk < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "topk: must be >= 0 (got %d)", p->topk);
  if (p->kv_format != MLA_KV_BF16 && p->kv_format != MLA_KV_FP8_656)
    return fail(MLA_ERR_INVALID_ARGUMENT, "kv_format: unknown value %d", p->kv_format);
  if (p->is_causal != 0 && p->is_causal != 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "is_causal: must be 0 or 1 (got %d)", p->is_causal);
  if (p->is_causal && p->topk > 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "is_causal: sparse decode (topk > 0) takes visibility from indices; is_causal must be 0");
  if (p->flags & ~MLA_FLAG_NATURAL_BASE)
    return fail(MLA_ERR_INVALID_ARGUMENT, "flags: unknown bits 0x%x", (unsigned)(p->flags & ~MLA_FLAG_NATURAL_BASE));
  if (!isfinite(p->softmax_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale: must be finite");
  const int64_t units = p->topk > 0 ? (int64_t)p->batch * p->s_q : p->batch;
  const int64_t rows = p->topk > 0 ? p->h_q : (int64_t)p->s_q * p->h_q;
  if (units > mla::kMaxUnits)
    return fail(MLA_ERR_UNSUPPORTED, "batch: %lld work units exceed the scheduler limit %d",
                (long long)units, mla::kMaxUnits);
  if (rows * 512 > INT32_MAX / 8)
    return fail(MLA_ERR_UNSUPPORTED, "h_q: %lld query rows per unit is too many", (long long)rows);
  const int64_t blocks_per_unit =
      p->topk > 0 ? (p->topk + mla::kPage - 1) / mla::kPage : p->max_pages_per_seq;
  if (units * (blocks_per_unit + mla::kSplitPenalty) + mla::kMaxParts >= INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "max_pages_per_seq/topk: total work exceeds the scheduler's int32 range");
  const int64_t table = (int64_t)p->batch * p->max_pages_per_seq;
  if (table >= INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "block_table: more than 2^31 entries");
  s->batch = p->batch;
  s->s_q = p->s_q;
  s->h_q = p->h_q;
  s->topk = p->topk;
  s->kv_format = p->kv_format;
  s->is_causal = p->is_causal;
  s->natural = (p->flags & MLA_FLAG_NATURAL_BASE) ? 1 : 0;
  s->num_pages = p->num_pages;
  s->max_pages = p->max_pages_per_seq;
  s->units = (int32_t)units;
  s->rows = (int32_t)rows;
  s->groups = mla::small_decode_applies(*s)
                  ? 1
                  : (int32_t)((rows + mla::kRowsPerGroup - 1) / mla::kRowsPerGroup);
  s->scale_log2 = s->natural ? (float)((double)p->softmax_scale * 1.4426950408889634) : p->softmax_scale;
  s->inv_h_q = 1.0f / (float)p->h_q;
  return MLA_OK;
}

mla_status check_parts(int32_t num_parts) {
  if (num_parts < 1 || num_parts > mla::kMaxParts)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts: must be in [1, %d] (got %d)", mla::kMaxParts, num_parts);
  return MLA_OK;
}

std::mutex g_cu_mutex;
std::vector<int> g_cu_count;  // per device, 0 = unknown

mla_status cu_count(int device, int* cus) {
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (device < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "device: must be >= 0 (got %d)", device);
  if ((size_t)device < g_cu_count.size() && g_cu_count[device] > 0) {
    *cus = g_cu_count[device];
    return MLA_OK;
  }
  int v = 0;
  hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess)
    return fail(MLA_ERR_HIP, "hipDeviceGetAttribute(device=%d): %s", device, hipGetErrorString(e));
  if ((size_t)device >= g_cu_count.size()) g_cu_count.resize(device + 1, 0);
  g_cu_count[device] = v;
  *cus = v;
  return MLA_OK;
}

mla_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define MLA_CHECK(expr)              \
  do {                               \
    mla_status st_ = (expr);         \
    if (st_ != MLA_OK) return st_;   \
  } while (0)

mla_status check_ptr(const void* ptr, const char* name, size_t align) {
  if (!ptr) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: NULL pointer", name);
  if (!aligned(ptr, align)) return fail(MLA_ERR_INVALID_ARGUMENT, "%s: must be %zu-byte aligned", name, align);
  return MLA_OK;
}

// Device address of a static device array (`scratch`, `check_words`) on
// each GPU, taken once per device, with that device current, on the first
// call that needs it there.
constexpr int kScratchDevices = 64;
enum DeviceSymbol { kScratch = 0, kCheckWords = 1 };
std::mutex g_scratch_mutex;
void* g_symbol_addr[2][kScratchDevices] = {};

mla_status symbol_address(hipStream_t stream, DeviceSymbol which, void** addr) {
  const char* name = which == kScratch ? "scratch" : "check_words";
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MLA_ERR_UNSUPPORTED, "stream: device %d is beyond the %d devices the static %s serves",
                dev, kScratchDevices, name);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  void*& slot = g_symbol_addr[which][dev];
  if (!slot) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(MLA_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* a = nullptr;
    e = which == kScratch ? hipGetSymbolAddress(&a, HIP_SYMBOL(scratch))
                          : hipGetSymbolAddress(&a, HIP_SYMBOL(check_words));
    if (dev != cur) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess)
      return fail(MLA_ERR_HIP, "hipGetSymbolAddress(%s) on device %d: %s", name, dev, hipGetErrorString(e));
    if (!a || !aligned(a, 256))
      return fail(MLA_ERR_HIP, "hipGetSymbolAddress(%s) on device %d: unusable address %p", name, dev, a);
    slot = a;
  }
  *addr = slot;
  return MLA_OK;
}

mla_status scratch_address(hipStream_t stream, void** addr) { return symbol_address(stream, kScratch, addr); }

// MLA_DEBUG_CHECKS set to anything but "" or "0" (read at every call): the
// decode calls first run the device-side input check on their stream, wait
// for it, and fail naming the first bad sequence instead of launching.
bool debug_checks() {
  const char* v = getenv("MLA_DEBUG_CHECKS");
  return v && v[0] && strcmp(v, "0") != 0;
}

mla_status debug_check(const mla::Shape& s, const int32_t* block_table, const int32_t* seqlens,
                       hipStream_t stream) {
  void* words = nullptr;
  MLA_CHECK(symbol_address(stream, kCheckWords, &words));
  MLA_CHECK(hip_status(mla::launch_check_inputs(s, block_table, seqlens, (int32_t*)words, stream),
                       "MLA_DEBUG_CHECKS: input check kernel launch"));
  int32_t host[2] = {0, -1};
  hipError_t e = hipMemcpyAsync(host, words, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(MLA_ERR_HIP, "MLA_DEBUG_CHECKS: reading the input check: %s", hipGetErrorString(e));
  if (host[0] != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "cache_seqlens/block_table: %d sequence(s) have a length outside [0, 64 * max_pages_per_seq] "
                "or a reachable block-table entry outside [0, num_pages); first: sequence %d (MLA_DEBUG_CHECKS)",
                host[0], host[1]);
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_decode_num_units(const mla_problem* p) {
  if (!p) return -1;
  return p->topk > 0 ? p->batch * p->s_q : p->batch;
}

mla_status mla_decode_num_parts(const mla_problem* p, int device, int32_t* num_parts) {
  mla::Shape s;
  MLA_CHECK(check_problem(p, &s));
  if (!num_parts) return fail(MLA_ERR_INVALID_ARGUMENT, "num_parts: NULL pointer");
  int cus = 0;
  MLA_CHECK(cu_count(device, &cus));
  int parts = cus / s.groups;
  if (parts < 1) parts = 1;
  *num_parts = parts;
  return ok();
}

const char* mla_decode_kernel_name(const mla_problem* p) {
  mla::Shape s;
  if (check_problem(p, &s) != MLA_OK) return nullptr;
  ok();
  return mla::small_decode_applies(s) ? "decode_small_kernel" : "decode_kernel";
}

mla_status mla_clock_probe(int64_t* out, int32_t workgroups, int32_t spins, void* stream) {
  if (workgroups < 1 || workgroups > 65536)
    return fail(MLA_ERR_INVALID_ARGUMENT, "workgroups: must be in [1, 65536] (got %d)", workgroups);
  if (spins < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "spins: must be >= 1 (got %d)", spins);
  MLA_CHECK(check_ptr(out, "out", 8));
  return hip_status(mla::launch_clock_probe(out, workgroups, spins, (hipStream_t)stream),
                    "clock probe kernel launch");
}

mla_status mla_decode_metadata_size(const mla_problem* p, int32_t num_parts, size_t* sched_ints,
                                    size_t* num_splits_ints) {
  mla::Shape s;
  MLA_CHECK(check_problem(p, &s));
  MLA_CHECK(check_parts(num_parts));
  if (!sched_ints || !num_splits_ints)
    return fail(MLA_ERR_INVALID_ARGUMENT, "sched_ints/num_splits_ints: NULL pointer");
  *sched_ints = (size_t)num_parts * 8;
  *num_splits_ints = (size_t)s.units + 1;
  return ok();
}

mla_status mla_decode_workspace_bytes(const mla_problem* p, int32_t num_parts, size_t* bytes) {
  mla::Shape s;
  MLA_CHECK(check_problem(p, &s));
  MLA_CHECK(check_parts(num_parts));
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes: NULL pointer");
  *bytes = mla::ws_total_bytes(num_parts, s.units, s.rows);
  return ok();
}

mla_status mla_decode_get_metadata(const mla_problem* p, const int32_t* cache_seqlens,
                                   int32_t num_parts, int32_t* sched, int32_t* num_splits,
                                   void* stream) {
  mla::Shape s;
  MLA_CHECK(check_problem(p, &s));
  MLA_CHECK(check_parts(num_parts));
  MLA_CHECK(check_ptr(cache_seqlens, "cache_seqlens", 4));
  MLA_CHECK(check_ptr(sched, "sched", 4));
  MLA_CHECK(check_ptr(num_splits, "num_splits", 4));
  return hip_status(mla::launch_metadata(s, cache_seqlens, num_parts, sched, num_splits,
                                         (hipStream_t)stream),
                    "metadata kernel launch");
}

mla_status mla_decode_paged(const mla_problem* p, const void* q, const void* kv_pool,
                            const int32_t* block_table, const int32_t* cache_seqlens,
                            const int32_t* indices, const int32_t* sched, int32_t num_parts,
                            const int32_t* num_splits, void* workspace, size_t workspace_bytes,
                            void* out, float* lse, void* stream) {
  mla::Shape s;
  MLA_CHECK(check_problem(p, &s));
  MLA_CHECK(check_parts(num_parts));
  MLA_CHECK(check_ptr(q, "q", 16));
  MLA_CHECK(check_ptr(kv_pool, "kv_pool", 16));
  MLA_CHECK(check_ptr(block_table, "block_table", 4));
  MLA_CHECK(check_ptr(cache_seqlens, "cache_seqlens", 4));
  if (p->topk > 0) {
    MLA_CHECK(check_ptr(indices, "indices", 4));
  } else if (indices) {
    return fail(MLA_ERR_INVALID_ARGUMENT, "indices: must be NULL when topk == 0");
  }
  MLA_CHECK(check_ptr(sched, "sched", 4));
  MLA_CHECK(check_ptr(num_splits, "num_splits", 4));
  MLA_CHECK(check_ptr(workspace, "workspace", 16));
  MLA_CHECK(check_ptr(out, "out", 16));
  MLA_CHECK(check_ptr(lse, "lse", 4));
  const size_t need = mla::ws_total_bytes(num_parts, s.units, s.rows);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes: %zu given, %zu needed", workspace_bytes, need);
  if (s.units == 0) return ok();
  if (debug_checks()) MLA_CHECK(debug_check(s, block_table, cache_seqlens, (hipStream_t)stream));
  mla::DecodeArgs a;
  a.s = s;
  a.q = (const uint16_t*)q;
  a.kv = (const uint8_t*)kv_pool;
  a.block_table = block_table;
  a.seqlens = cache_seqlens;
  a.indices = indices;
  a.sched = sched;
  a.num_splits = num_splits;
  a.num_parts = num_parts;
  const size_t slots = mla::ws_slots(num_parts, s.units);
  a.ws_lse = (float*)workspace;
  a.ws_o = (uint16_t*)((char*)workspace + mla::ws_lse_bytes(slots, s.rows));
  a.out = (uint16_t*)out;
  a.lse = lse;
  if (mla::small_decode_applies(s))
    return hip_status(mla::launch_decode_small(a, (hipStream_t)stream), "decode kernel launch");
  return hip_status(mla::launch_decode(a, (hipStream_t)stream), "decode kernel launch");
}

mla_status mla_decode_paged_fp8(const mla_problem* p, const void* q, const void* kv_pool,
                                const int32_t* block_table, const int32_t* cache_seqlens,
                                const int32_t* sched, int32_t num_parts,
                                const int32_t* num_splits, void* workspace,
                                size_t workspace_bytes, void* out, float* lse, void* stream) {
  if (!p) return fail(MLA_ERR_INVALID_ARGUMENT, "p: NULL problem");
  if (p->kv_format != MLA_KV_FP8_656)
    return fail(MLA_ERR_INVALID_ARGUMENT, "kv_format: mla_decode_paged_fp8 needs MLA_KV_FP8_656");
  if (p->topk != 0) return fail(MLA_ERR_INVALID_ARGUMENT, "topk: mla_decode_paged_fp8 is dense (topk must be 0)");
  return mla_decode_paged(p, q, kv_pool, block_table, cache_seqlens, nullptr, sched, num_parts,
                          num_splits, workspace, workspace_bytes, out, lse, stream);
}

mla_status mla_decode_sparse_fp8(const mla_problem* p, const void* q, const void* kv_pool,
                                 const int32_t* block_table, const int32_t* cache_seqlens,
                                 const int32_t* indices, const int32_t* sched,
                                 int32_t num_parts, const int32_t* num_splits, void* workspace,
                                 size_t workspace_bytes, void* out, float* lse, void* stream) {
  if (!p) return fail(MLA_ERR_INVALID_ARGUMENT, "p: NULL problem");
  if (p->kv_format != MLA_KV_FP8_656)
    return fail(MLA_ERR_INVALID_ARGUMENT, "kv_format: mla_decode_sparse_fp8 needs MLA_KV_FP8_656");
  if (p->topk <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "topk: mla_decode_sparse_fp8 needs topk > 0");
  return mla_decode_paged(p, q, kv_pool, block_table, cache_seqlens, indices, sched, num_parts,
                          num_splits, workspace, workspace_bytes, out, lse, stream);
}

mla_status mla_decode_combine(const mla_problem* p, int32_t num_parts, const int32_t* num_splits,
                              const void* workspace, size_t workspace_bytes, void* out,
                              float* lse, void* stream) {
  mla::Shape s;
  MLA_CHECK(check_problem(p, &s));
  MLA_CHECK(check_parts(num_parts));
  MLA_CHECK(check_ptr(num_splits, "num_splits", 4));
  MLA_CHECK(check_ptr(workspace, "workspace", 16));
  MLA_CHECK(check_ptr(out, "out", 16));
  MLA_CHECK(check_ptr(lse, "lse", 4));
  const size_t need = mla::ws_total_bytes(num_parts, s.units, s.rows);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes: %zu given, %zu needed", workspace_bytes, need);
  if (s.units == 0) return ok();
  const size_t slots = mla::ws_slots(num_parts, s.units);
  const float* ws_lse = (const float*)workspace;
  const uint16_t* ws_o = (const uint16_t*)((const char*)workspace + mla::ws_lse_bytes(slots, s.rows));
  return hip_status(mla::launch_combine(s, num_splits, ws_lse, ws_o, (uint16_t*)out, lse,
                                        (hipStream_t)stream),
                    "combine kernel launch");
}

mla_status mla_decode_paged_noalloc(const mla_problem* p, const void* q, const void* kv_pool,
                                    const int32_t* block_table, const int32_t* cache_seqlens,
                                    const int32_t* indices, const int32_t* sched, int32_t num_parts,
                                    const int32_t* num_splits, void* out, float* lse, void* stream) {
  mla::Shape s;
  MLA_CHECK(check_problem(p, &s));
  MLA_CHECK(check_parts(num_parts));
  MLA_CHECK(check_ptr(q, "q", 16));
  MLA_CHECK(check_ptr(kv_pool, "kv_pool", 16));
  MLA_CHECK(check_ptr(block_table, "block_table", 4));
  MLA_CHECK(check_ptr(cache_seqlens, "cache_seqlens", 4));
  if (p->topk > 0) {
    MLA_CHECK(check_ptr(indices, "indices", 4));
  } else if (indices) {
    return fail(MLA_ERR_INVALID_ARGUMENT, "indices: must be NULL when topk == 0");
  }
  MLA_CHECK(check_ptr(sched, "sched", 4));
  MLA_CHECK(check_ptr(num_splits, "num_splits", 4));
  MLA_CHECK(check_ptr(out, "out", 16));
  MLA_CHECK(check_ptr(lse, "lse", 4));
  const size_t need = mla::ws_total_bytes(num_parts, s.units, s.rows);
  if (need > MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "num_parts/batch/s_q/h_q: the split partials need %zu bytes, more than the %zu-byte static "
                "scratch of mla_decode_paged_noalloc (call mla_decode_paged with a workspace instead)",
                need, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  if (s.units == 0) return ok();
  void* ws = nullptr;
  MLA_CHECK(scratch_address((hipStream_t)stream, &ws));
  MLA_CHECK(mla_decode_paged(p, q, kv_pool, block_table, cache_seqlens, indices, sched, num_parts,
                             num_splits, ws, need, out, lse, stream));
  return mla_decode_combine(p, num_parts, num_splits, ws, need, out, lse, stream);
}

}  // extern "C"

namespace {

// Validates an indexer problem; fills the workspace size.
mla_status check_index_problem(const mla_index_problem* p, size_t* ws_bytes) {
  if (!p) return fail(MLA_ERR_INVALID_ARGUMENT, "p: NULL problem");
  if (p->batch < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "batch: must be >= 0 (got %d)", p->batch);
  if (p->s_q < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "s_q: must be >= 1 (got %d)", p->s_q);
  if (p->h < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "h: must be >= 1 (got %d)", p->h);
  if (p->h > 4096) return fail(MLA_ERR_UNSUPPORTED, "h: at most 4096 index heads (got %d)", p->h);
  if (p->d != 512) return fail(MLA_ERR_UNSUPPORTED, "d: must be 512 (got %d)", p->d);
  if (p->page_size != mla::kPage) return fail(MLA_ERR_UNSUPPORTED, "page_size: must be 64 (got %d)", p->page_size);
  if (p->num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages: must be >= 1 (got %d)", p->num_pages);
  if (p->max_pages_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq: must be >= 1 (got %d)", p->max_pages_per_seq);
  if (p->max_pages_per_seq > 1024)
    return fail(MLA_ERR_UNSUPPORTED, "max_pages_per_seq: at most 1024 (65536 rows per sequence; got %d)",
                p->max_pages_per_seq);
  const int32_t n_max = p->max_pages_per_seq * mla::kPage;
  if (p->topk < 1 || p->topk > n_max)
    return fail(MLA_ERR_INVALID_ARGUMENT, "topk: must be in [1, %d] (got %d)", n_max, p->topk);
  if (p->kpool < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "kpool: must be >= 1 (got %d)", p->kpool);
  if (p->is_causal != 0 && p->is_causal != 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "is_causal: must be 0 or 1 (got %d)", p->is_causal);
  const long long tokens = (long long)p->batch * p->s_q;
  if (tokens > (1LL << 31) - 1)
    return fail(MLA_ERR_UNSUPPORTED, "batch: batch * s_q = %lld query tokens exceed 2^31 - 1", tokens);
  if ((long long)p->batch * p->max_pages_per_seq > (1LL << 31) - 1)
    return fail(MLA_ERR_UNSUPPORTED, "block_table: more than 2^31 entries");
  int32_t per_group = 0, groups = 0;
  mla::index_groups(p->s_q, &per_group, &groups);
  const long long workgroups = (long long)p->batch * groups * ((p->max_pages_per_seq + mla::kIndexChunkPages - 1) / mla::kIndexChunkPages);
  if (workgroups > (1LL << 31) - 8)
    return fail(MLA_ERR_UNSUPPORTED, "batch: %lld score workgroups exceed the grid limit", workgroups);
  *ws_bytes = mla::index_workspace_bytes(p->batch, p->s_q, p->max_pages_per_seq);
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_fp8_index_workspace_bytes(const mla_index_problem* p, size_t* bytes) {
  size_t need = 0;
  MLA_CHECK(check_index_problem(p, &need));
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes: NULL pointer");
  *bytes = need;
  return ok();
}

}  // extern "C"

namespace {

// The indexer's shared argument checks; fills the launch description.
mla_status index_launch(const mla_index_problem* p, const void* q_fp8, const float* q_scale,
                        const void* kv_pool, const int32_t* block_table, const int32_t* cache_seqlens,
                        void* workspace, size_t workspace_bytes, int32_t* indices, float* scores,
                        bool need_scores_in, bool need_select_out, mla::IndexLaunch* l) {
  size_t need = 0;
  MLA_CHECK(check_index_problem(p, &need));
  if (need_scores_in) {
    MLA_CHECK(check_ptr(q_fp8, "q_fp8", 16));
    MLA_CHECK(check_ptr(q_scale, "q_scale", 16));
    MLA_CHECK(check_ptr(kv_pool, "kv_pool", 16));
    MLA_CHECK(check_ptr(block_table, "block_table", 4));
  }
  MLA_CHECK(check_ptr(cache_seqlens, "cache_seqlens", 4));
  MLA_CHECK(check_ptr(workspace, "workspace", 16));
  if (need_select_out) {
    MLA_CHECK(check_ptr(indices, "indices", 4));
    if (scores) MLA_CHECK(check_ptr(scores, "scores", 4));
  }
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes: %zu given, %zu needed", workspace_bytes, need);
  l->batch = p->batch;
  l->s_q = p->s_q;
  l->h = p->h;
  l->kpool = p->kpool;
  l->is_causal = p->is_causal;
  l->max_pages = p->max_pages_per_seq;
  l->topk = p->topk;
  l->q = (const uint8_t*)q_fp8;
  l->qs = q_scale;
  l->kv = (const uint8_t*)kv_pool;
  l->block_table = block_table;
  l->seqlens = cache_seqlens;
  l->ws = (float*)workspace;
  l->indices = indices;
  l->scores = scores;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_fp8_index_top_k(const mla_index_problem* p, const void* q_fp8, const float* q_scale,
                               const void* kv_pool, const int32_t* block_table,
                               const int32_t* cache_seqlens, void* workspace,
                               size_t workspace_bytes, int32_t* indices, float* scores,
                               void* stream) {
  mla::IndexLaunch l;
  MLA_CHECK(index_launch(p, q_fp8, q_scale, kv_pool, block_table, cache_seqlens, workspace,
                         workspace_bytes, indices, scores, true, true, &l));
  MLA_CHECK(hip_status(mla::launch_index_scores(l, (hipStream_t)stream), "indexer score kernel launch"));
  return hip_status(mla::launch_index_select(l, (hipStream_t)stream), "indexer selection kernel launch");
}

mla_status mla_fp8_index_scores(const mla_index_problem* p, const void* q_fp8, const float* q_scale,
                                const void* kv_pool, const int32_t* block_table,
                                const int32_t* cache_seqlens, void* workspace,
                                size_t workspace_bytes, void* stream) {
  mla::IndexLaunch l;
  MLA_CHECK(index_launch(p, q_fp8, q_scale, kv_pool, block_table, cache_seqlens, workspace,
                         workspace_bytes, nullptr, nullptr, true, false, &l));
  return hip_status(mla::launch_index_scores(l, (hipStream_t)stream), "indexer score kernel launch");
}

mla_status mla_fp8_index_select(const mla_index_problem* p, const int32_t* cache_seqlens,
                                const void* workspace, size_t workspace_bytes, int32_t* indices,
                                float* scores, void* stream) {
  mla::IndexLaunch l;
  MLA_CHECK(index_launch(p, nullptr, nullptr, nullptr, nullptr, cache_seqlens, (void*)workspace,
                         workspace_bytes, indices, scores, false, true, &l));
  return hip_status(mla::launch_index_select(l, (hipStream_t)stream), "indexer selection kernel launch");
}

mla_status mla_decode_check_inputs(const mla_problem* p, const int32_t* block_table,
                                   const int32_t* cache_seqlens, int32_t* result, void* stream) {
  mla::Shape s;
  MLA_CHECK(check_problem(p, &s));
  MLA_CHECK(check_ptr(result, "result", 4));
  if (s.batch > 0) {
    MLA_CHECK(check_ptr(block_table, "block_table", 4));
    MLA_CHECK(check_ptr(cache_seqlens, "cache_seqlens", 4));
  }
  return hip_status(mla::launch_check_inputs(s, block_table, cache_seqlens, result, (hipStream_t)stream),
                    "input check kernel launch");
}

mla_status mla_kv_quantize_fp8(int32_t batch, int32_t n_new, int32_t page_size,
                               int32_t num_pages, int32_t max_pages_per_seq, const void* kv_new,
                               const int32_t* start_pos, const int32_t* block_table,
                               void* kv_pool, void* stream) {
  if (batch < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "batch: must be >= 0 (got %d)", batch);
  if (n_new < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_new: must be >= 0 (got %d)", n_new);
  if (page_size != mla::kPage)
    return fail(MLA_ERR_UNSUPPORTED, "page_size: must be 64 (got %d)", page_size);
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages: must be >= 1 (got %d)", num_pages);
  if (max_pages_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq: must be >= 1 (got %d)", max_pages_per_seq);
  if ((int64_t)batch * n_new > INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "n_new: batch * n_new = %lld tokens exceed 2^31 - 1",
                (long long)batch * n_new);
  if ((int64_t)batch * max_pages_per_seq >= INT32_MAX)
    return fail(MLA_ERR_UNSUPPORTED, "block_table: more than 2^31 entries");
  MLA_CHECK(check_ptr(kv_new, "kv_new", 16));
  MLA_CHECK(check_ptr(start_pos, "start_pos", 4));
  MLA_CHECK(check_ptr(block_table, "block_table", 4));
  MLA_CHECK(check_ptr(kv_pool, "kv_pool", 16));
  if ((int64_t)batch * n_new == 0) return ok();
  return hip_status(mla::launch_kv_quantize_fp8(batch, n_new, num_pages, max_pages_per_seq,
                                                (const uint16_t*)kv_new, start_pos, block_table,
                                                (uint8_t*)kv_pool, (hipStream_t)stream),
                    "FP8 KV writer kernel launch");
}

}  // extern "C"

namespace {

// Workspace of a sparse prefill: identity block table, the cache length,
// metadata, then the decode workspace of one chunk (each part 256-aligned).
struct PrefillLayout {
  size_t table, seqlen, sched, num_splits, decode, total;
  size_t decode_bytes;
};

mla_status prefill_problem(int32_t n, int32_t h_q, int32_t s_kv, int32_t topk, int32_t kv_format,
                           int32_t flags, float softmax_scale, mla_problem* p) {
  if (s_kv < 1 || s_kv > INT32_MAX - 63)
    return fail(MLA_ERR_INVALID_ARGUMENT, "s_kv: must be in [1, 2^31 - 64] (got %d)", s_kv);
  if (topk < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "topk: must be >= 1 (got %d)", topk);
  const int32_t pages = (int32_t)(((int64_t)s_kv + 63) / 64);
  *p = mla_problem{1, n < 1 ? 1 : n, h_q, 1, mla::kDqk, mla::kDv, mla::kPage, pages, pages,
                   topk, kv_format, 0, flags, softmax_scale};
  mla::Shape s;
  return check_problem(p, &s);
}

mla_status prefill_layout(int32_t s_q, int32_t h_q, int32_t s_kv, int32_t topk, int32_t kv_format,
                          int32_t flags, float softmax_scale, int32_t num_parts, PrefillLayout* L) {
  if (s_q < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "s_q: must be >= 0 (got %d)", s_q);
  const int32_t chunk = s_q < mla::kPrefillChunk ? s_q : mla::kPrefillChunk;
  mla_problem p;
  MLA_CHECK(prefill_problem(chunk, h_q, s_kv, topk, kv_format, flags, softmax_scale, &p));
  MLA_CHECK(check_parts(num_parts));
  size_t sched_ints = 0, splits_ints = 0, ws = 0;
  MLA_CHECK(mla_decode_metadata_size(&p, num_parts, &sched_ints, &splits_ints));
  MLA_CHECK(mla_decode_workspace_bytes(&p, num_parts, &ws));
  L->table = 0;
  L->seqlen = mla::align256(L->table + (size_t)p.num_pages * 4);
  L->sched = L->seqlen + 256;
  L->num_splits = mla::align256(L->sched + sched_ints * 4);
  L->decode = mla::align256(L->num_splits + splits_ints * 4);
  L->decode_bytes = ws;
  L->total = L->decode + ws;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_sparse_prefill_workspace_bytes(int32_t s_q, int32_t h_q, int32_t s_kv, int32_t topk,
                                              int32_t kv_format, int32_t num_parts, size_t* bytes) {
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes: NULL pointer");
  PrefillLayout L;
  MLA_CHECK(prefill_layout(s_q, h_q, s_kv, topk, kv_format, 0, 1.0f, num_parts, &L));
  *bytes = L.total;
  return ok();
}

mla_status mla_sparse_prefill(int32_t s_q, int32_t h_q, int32_t s_kv, int32_t topk,
                              int32_t kv_format, int32_t flags, float softmax_scale,
                              const void* q, const void* kv, const int32_t* indices,
                              int32_t num_parts, void* workspace, size_t workspace_bytes,
                              void* out, float* lse, void* stream) {
  PrefillLayout L;
  MLA_CHECK(prefill_layout(s_q, h_q, s_kv, topk, kv_format, flags, softmax_scale, num_parts, &L));
  if (s_q == 0) return ok();  // nothing to read or write; empty tensors may have NULL data
  MLA_CHECK(check_ptr(q, "q", 16));
  MLA_CHECK(check_ptr(kv, "kv", 16));
  MLA_CHECK(check_ptr(indices, "indices", 4));
  MLA_CHECK(check_ptr(workspace, "workspace", 256));
  MLA_CHECK(check_ptr(out, "out", 16));
  MLA_CHECK(check_ptr(lse, "lse", 4));
  if (workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes: %zu given, %zu needed", workspace_bytes, L.total);
  char* ws = (char*)workspace;
  int32_t* table = (int32_t*)(ws + L.table);
  int32_t* seqlen = (int32_t*)(ws + L.seqlen);
  int32_t* sched = (int32_t*)(ws + L.sched);
  int32_t* num_splits = (int32_t*)(ws + L.num_splits);
  hipStream_t st = (hipStream_t)stream;
  const int32_t pages = (int32_t)(((int64_t)s_kv + 63) / 64);
  MLA_CHECK(hip_status(mla::launch_identity_table(table, pages, seqlen, s_kv, st),
                       "identity table kernel launch"));
  for (int32_t c0 = 0; c0 < s_q; c0 += mla::kPrefillChunk) {
    const int32_t n = s_q - c0 < mla::kPrefillChunk ? s_q - c0 : mla::kPrefillChunk;
    mla_problem p;
    MLA_CHECK(prefill_problem(n, h_q, s_kv, topk, kv_format, flags, softmax_scale, &p));
    const int64_t row0 = (int64_t)c0 * h_q;
    const uint16_t* qc = (const uint16_t*)q + row0 * mla::kDqk;
    const int32_t* ic = indices + (int64_t)c0 * topk;
    uint16_t* oc = (uint16_t*)out + row0 * mla::kDv;
    float* lc = lse + row0;
    MLA_CHECK(mla_decode_get_metadata(&p, seqlen, num_parts, sched, num_splits, stream));
    MLA_CHECK(mla_decode_paged(&p, qc, kv, table, seqlen, ic, sched, num_parts, num_splits,
                               ws + L.decode, L.decode_bytes, oc, lc, stream));
    MLA_CHECK(mla_decode_combine(&p, num_parts, num_splits, ws + L.decode, L.decode_bytes, oc, lc,
                                 stream));
  }
  return ok();
}

const char* mla_last_error(void) { return g_err; }

}  // extern "C"
