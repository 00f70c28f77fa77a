// paged_attention.cpp -- the C ABI declared in include/paged_attention.h:
// argument checks, planning (pa_plan.cpp) and dispatch to the decode or
// prefill schedule. Nothing is launched unless every check passes.
#include "paged_attention.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "pa_kernels.h"
#include "pa_plan.h"

namespace {

thread_local std::string g_last_error;
std::atomic<uint32_t> g_epoch{0};

uint32_t next_epoch() {
  uint32_t e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  while (e == 0) e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  return e;
}

int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

pa::Shape make_shape(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t query_len,
                     int32_t head_dim, int32_t num_pages, int32_t page_size, int32_t max_pages,
                     bool causal) {
  pa::Shape s;
  s.batch = batch;
  s.num_q_heads = num_q_heads;
  s.num_kv_heads = num_kv_heads;
  s.query_len = query_len;
  s.head_dim = head_dim;
  s.num_pages = num_pages;
  s.page_size = page_size;
  s.max_pages = max_pages;
  s.causal = causal;
  return s;
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

// An explicit mask of the uniform entry points.
struct MaskSpec {
  const float* ptr;
  int64_t sb, sh, sl;
  int32_t len;
};

// The uniform-layout operator, with or without an explicit mask.
int run_uniform(const void* query, const void* key_pages, const void* value_pages, const int32_t* block_table,
                const int32_t* context_lens, const MaskSpec* mask, void* out, int32_t batch, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t query_len, int32_t head_dim, int32_t num_pages, int32_t page_size,
                int32_t max_pages, float scale, int32_t causal, void* workspace, size_t workspace_bytes,
                int32_t schedule, int32_t decode_work_items, void* stream) {
  if (!query || !key_pages || !value_pages || !block_table || !context_lens || !out)
    return set_error(PA_ERR_INVALID, "a tensor pointer is NULL");
  if (causal != 0 && causal != 1) return set_error(PA_ERR_INVALID, "causal must be 0 or 1");
  if (!std::isfinite(scale)) return set_error(PA_ERR_INVALID, "scale must be finite");
  pa::Plan plan;
  std::string err;
  const pa::Shape s = make_shape(batch, num_q_heads, num_kv_heads, query_len, head_dim, num_pages,
                                 page_size, max_pages, causal != 0);
  const int rc = pa::make_plan(s, schedule, decode_work_items, true, &plan, &err);
  if (rc != pa::kOk) return set_error(rc, err);
  if (mask && plan.schedule == pa::kSchedulePrefill64x32)
    return set_error(PA_ERR_UNSUPPORTED, "the 64 x 32 prefill tiling takes no explicit mask");
  if (plan.schedule == pa::kSchedulePrefill && plan.kv_splits > 1 &&
      (workspace == nullptr || workspace_bytes < plan.workspace_bytes)) {
    // a prefill without the workspace its key-range split needs runs unsplit
    plan.kv_splits = 1;
    plan.workspace_bytes = 0;
  }
  if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
    return set_error(PA_ERR_WORKSPACE, "workspace smaller than paged_attention_workspace_bytes() = " +
                                           std::to_string(plan.workspace_bytes));
  const size_t q_bytes = size_t(batch) * num_q_heads * query_len * head_dim * 2;
  const size_t pool_bytes = size_t(num_pages) * num_kv_heads * page_size * head_dim * 2;
  if (overlaps(out, q_bytes, query, q_bytes) || overlaps(out, q_bytes, key_pages, pool_bytes) ||
      overlaps(out, q_bytes, value_pages, pool_bytes) ||
      overlaps(out, q_bytes, block_table, size_t(batch) * max_pages * 4) ||
      overlaps(out, q_bytes, context_lens, size_t(batch) * 4) ||
      (plan.workspace_bytes > 0 && overlaps(out, q_bytes, workspace, plan.workspace_bytes)))
    return set_error(PA_ERR_INVALID, "out overlaps an input or the workspace");
  if (mask) {
    // the mask buffer spans (B-1)*sb + (H_q-1)*sh + (L-1)*sl + len floats
    const size_t span = size_t((batch - 1) * mask->sb + (num_q_heads - 1) * mask->sh +
                               (query_len - 1) * mask->sl + mask->len) * sizeof(float);
    if (overlaps(out, q_bytes, mask->ptr, span)) return set_error(PA_ERR_INVALID, "out overlaps the mask");
  }

  pa::KernelArgs k;
  k.query = query;
  k.key_pages = key_pages;
  k.value_pages = value_pages;
  k.block_table = block_table;
  k.context_lens = context_lens;
  k.out = out;
  k.workspace = workspace;
  k.batch = batch;
  k.num_q_heads = num_q_heads;
  k.num_kv_heads = num_kv_heads;
  k.query_len = query_len;
  k.num_pages = num_pages;
  k.page_size = page_size;
  k.max_pages = max_pages;
  k.head_dim = head_dim;
  k.scale = scale;
  k.causal = causal;
  k.epoch = next_epoch();
  if (mask) {
    k.mask = mask->ptr;
    k.mask_stride_b = mask->sb;
    k.mask_stride_h = mask->sh;
    k.mask_stride_l = mask->sl;
    k.mask_len = mask->len;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = plan.schedule == pa::kScheduleDecode ? pa::launch_decode(k, plan, st)
                                                            : pa::launch_prefill(k, plan, st);
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, std::string("launch failed: ") + hipGetErrorString(e));
  g_last_error.clear();
  return PA_OK;
}

// ---- the library's own scratch for paged_attention_static ----
//
// One array per GPU, held until the process ends: the decode schedule's
// arrival counters and partial states, and the split prefill's, for callers
// that cannot allocate. 64 MiB covers every decode launch of head dim 128
// (8 query rows per kv head, 2048 work items: 17 MB) and every split prefill
// of head dim 128 (at most 512 parts of 128 rows: 34 MB).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zero-fills the scratch once per device: its head holds arrival counters.
__global__ void zero_scratch(uint4* p, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += size_t(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch (the host-side name of the
// array is only a stand-in), looked up and zero-filled on the first call on
// that device. Returns nullptr with the error set on failure.
void* device_scratch(hipStream_t stream, int* code) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *code = set_error(PA_ERR_LAUNCH, "no current HIP device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *code = set_error(PA_ERR_LAUNCH, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
      return nullptr;
    }
    hipLaunchKernelGGL(zero_scratch, dim3(1024), dim3(256), 0, stream, static_cast<uint4*>(ptr), kScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) {
      *code = set_error(PA_ERR_LAUNCH, std::string("scratch fill failed: ") + hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int paged_attention_ex(const void* query, const void* key_pages, const void* value_pages,
                       const int32_t* block_table, const int32_t* context_lens, void* out,
                       int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t query_len,
                       int32_t head_dim, int32_t num_pages, int32_t page_size, int32_t max_pages,
                       float scale, int32_t causal, void* workspace, size_t workspace_bytes,
                       int32_t schedule, int32_t decode_work_items, void* stream) {
  return run_uniform(query, key_pages, value_pages, block_table, context_lens, nullptr, out, batch, num_q_heads,
                     num_kv_heads, query_len, head_dim, num_pages, page_size, max_pages, scale, causal, workspace,
                     workspace_bytes, schedule, decode_work_items, stream);
}

int paged_attention_masked(const void* query, const void* key_pages, const void* value_pages,
                           const int32_t* block_table, const int32_t* context_lens, const float* mask,
                           int64_t mask_stride_b, int64_t mask_stride_h, int64_t mask_stride_l,
                           int32_t mask_len, void* out, int32_t batch, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t query_len, int32_t head_dim, int32_t num_pages,
                           int32_t page_size, int32_t max_pages, float scale, int32_t causal,
                           void* workspace, size_t workspace_bytes, int32_t schedule,
                           int32_t decode_work_items, void* stream) {
  if (!mask) return set_error(PA_ERR_INVALID, "mask is NULL");
  if (mask_stride_b < 0 || mask_stride_h < 0 || mask_stride_l < 0)
    return set_error(PA_ERR_INVALID, "mask strides must be >= 0");
  if (mask_len < 1) return set_error(PA_ERR_INVALID, "mask_len must be positive");
  const int64_t lim = int64_t(1) << 40;  // keeps the extent arithmetic far from overflow
  if (mask_stride_b > lim || mask_stride_h > lim || mask_stride_l > lim)
    return set_error(PA_ERR_UNSUPPORTED, "mask strides too large");
  const MaskSpec m{mask, mask_stride_b, mask_stride_h, mask_stride_l, mask_len};
  return run_uniform(query, key_pages, value_pages, block_table, context_lens, &m, out, batch, num_q_heads,
                     num_kv_heads, query_len, head_dim, num_pages, page_size, max_pages, scale, causal, workspace,
                     workspace_bytes, schedule, decode_work_items, stream);
}

int paged_attention(const void* query, const void* key_pages, const void* value_pages,
                    const int32_t* block_table, const int32_t* context_lens, void* out,
                    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t query_len,
                    int32_t head_dim, int32_t num_pages, int32_t page_size, int32_t max_pages,
                    float scale, int32_t causal, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return paged_attention_ex(query, key_pages, value_pages, block_table, context_lens, out, batch,
                            num_q_heads, num_kv_heads, query_len, head_dim, num_pages, page_size,
                            max_pages, scale, causal, workspace, workspace_bytes, PA_SCHEDULE_AUTO, 0,
                            stream);
}

int paged_attention_static(const void* query, const void* key_pages, const void* value_pages,
                           const int32_t* block_table, const int32_t* context_lens, void* out, int32_t batch,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t query_len, int32_t head_dim,
                           int32_t num_pages, int32_t page_size, int32_t max_pages, float scale, int32_t causal,
                           void* stream) {
  if (!query || !key_pages || !value_pages || !block_table || !context_lens || !out)
    return set_error(PA_ERR_INVALID, "a tensor pointer is NULL");
  // sizes next: nothing is touched for a call the scratch cannot serve
  pa::Plan plan;
  std::string err;
  const pa::Shape s = make_shape(batch, num_q_heads, num_kv_heads, query_len, head_dim, num_pages, page_size,
                                 max_pages, causal != 0);
  const int rc = pa::make_plan(s, PA_SCHEDULE_AUTO, 0, true, &plan, &err);
  if (rc != pa::kOk) return set_error(rc, err);
  if (plan.schedule == pa::kScheduleDecode && plan.workspace_bytes > kScratchBytes)
    return set_error(PA_ERR_UNSUPPORTED, "the decode schedule needs " + std::to_string(plan.workspace_bytes) +
                                             " bytes of scratch; paged_attention_static holds " +
                                             std::to_string(kScratchBytes) + " (use paged_attention)");
  int code = PA_OK;
  void* ws = device_scratch(static_cast<hipStream_t>(stream), &code);
  if (ws == nullptr) return code;
  // a split prefill that needs more than the scratch runs unsplit (as with a short workspace)
  return paged_attention(query, key_pages, value_pages, block_table, context_lens, out, batch, num_q_heads,
                         num_kv_heads, query_len, head_dim, num_pages, page_size, max_pages, scale, causal, ws,
                         kScratchBytes, stream);
}

size_t paged_attention_static_scratch_bytes(void) { return kScratchBytes; }

size_t paged_attention_workspace_bytes_ex(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t query_len, int32_t head_dim, int32_t page_size,
                                          int32_t max_pages, int32_t schedule, int32_t decode_work_items) {
  pa::Plan plan;
  std::string err;
  const pa::Shape s = make_shape(batch, num_q_heads, num_kv_heads, query_len, head_dim, 1, page_size,
                                 max_pages, false);
  const int rc = pa::make_plan(s, schedule, decode_work_items, false, &plan, &err);
  if (rc != pa::kOk) {
    set_error(rc, err);
    return static_cast<size_t>(-1);
  }
  g_last_error.clear();
  return plan.workspace_bytes;
}

size_t paged_attention_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t query_len, int32_t head_dim, int32_t page_size,
                                       int32_t max_pages) {
  return paged_attention_workspace_bytes_ex(batch, num_q_heads, num_kv_heads, query_len, head_dim,
                                            page_size, max_pages, PA_SCHEDULE_AUTO, 0);
}

int paged_attention_schedule(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t query_len, int32_t head_dim, int32_t page_size,
                             int32_t max_pages) {
  pa::Plan plan;
  std::string err;
  const pa::Shape s = make_shape(batch, num_q_heads, num_kv_heads, query_len, head_dim, 1, page_size,
                                 max_pages, false);
  const int rc = pa::make_plan(s, PA_SCHEDULE_AUTO, 0, false, &plan, &err);
  if (rc != pa::kOk) return set_error(rc, err);
  g_last_error.clear();
  return plan.schedule;
}

int paged_attention_check_metadata(const int32_t* block_table, const int32_t* context_lens,
                                   int32_t batch, int32_t max_pages, int32_t num_pages,
                                   int32_t page_size, int32_t query_len, int32_t causal,
                                   void* stream) {
  if (!block_table || !context_lens) return set_error(PA_ERR_INVALID, "a tensor pointer is NULL");
  if (batch < 1 || max_pages < 1 || num_pages < 1 || page_size < 1 || query_len < 1)
    return set_error(PA_ERR_INVALID, "all sizes must be positive");
  std::vector<int32_t> bt(size_t(batch) * max_pages), ctx(batch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(bt.data(), block_table, bt.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(ctx.data(), context_lens, ctx.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, std::string("copy failed: ") + hipGetErrorString(e));
  const int64_t max_ctx = int64_t(max_pages) * page_size;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t c = ctx[b];
    if (c < 1 || c > max_ctx)
      return set_error(PA_ERR_METADATA, "context_lens[" + std::to_string(b) + "] = " + std::to_string(c) +
                                            " outside [1, max_pages * page_size]");
    if (causal && c < query_len)
      return set_error(PA_ERR_METADATA, "context_lens[" + std::to_string(b) + "] < query_len under causal");
    const int64_t used = (int64_t(c) + page_size - 1) / page_size;
    for (int64_t j = 0; j < used; ++j) {
      const int32_t p = bt[size_t(b) * max_pages + j];
      if (p < 0 || p >= num_pages)
        return set_error(PA_ERR_METADATA, "block_table[" + std::to_string(b) + "][" + std::to_string(j) +
                                              "] = " + std::to_string(p) + " is not a page of the pool");
    }
  }
  g_last_error.clear();
  return PA_OK;
}

int paged_kv_append(const void* key_new, const void* value_new, void* key_pages, void* value_pages,
                    const int32_t* block_table, const int32_t* context_lens, int32_t batch,
                    int32_t num_kv_heads, int32_t new_len, int32_t head_dim, int32_t num_pages,
                    int32_t page_size, int32_t max_pages, void* stream) {
  if (!key_new || !value_new || !key_pages || !value_pages || !block_table || !context_lens)
    return set_error(PA_ERR_INVALID, "a tensor pointer is NULL");
  if (batch < 1 || num_kv_heads < 1 || new_len < 1 || head_dim < 1 || num_pages < 1 || page_size < 1 ||
      max_pages < 1)
    return set_error(PA_ERR_INVALID, "all sizes must be positive");
  if (!pa::head_dim_supported(head_dim))
    return set_error(PA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 from 8 to 256");
  const int64_t max_ctx = int64_t(max_pages) * page_size;
  if (max_ctx > INT32_MAX) return set_error(PA_ERR_UNSUPPORTED, "max_pages * page_size exceeds int32");
  if (max_ctx < new_len) return set_error(PA_ERR_INVALID, "max_pages * page_size < new_len");
  const int64_t rows = int64_t(batch) * num_kv_heads * new_len;
  if (rows > (int64_t(1) << 34)) return set_error(PA_ERR_UNSUPPORTED, "batch * num_kv_heads * new_len too large");
  const size_t new_bytes = size_t(rows) * head_dim * 2;
  const size_t pool_bytes = size_t(num_pages) * num_kv_heads * page_size * head_dim * 2;
  if (overlaps(key_pages, pool_bytes, value_pages, pool_bytes))
    return set_error(PA_ERR_INVALID, "key_pages and value_pages overlap");
  if (overlaps(key_new, new_bytes, key_pages, pool_bytes) || overlaps(key_new, new_bytes, value_pages, pool_bytes) ||
      overlaps(value_new, new_bytes, key_pages, pool_bytes) || overlaps(value_new, new_bytes, value_pages, pool_bytes))
    return set_error(PA_ERR_INVALID, "new K/V overlap a page pool");
  pa::AppendKernelArgs k;
  k.key_new = key_new;
  k.value_new = value_new;
  k.key_pages = key_pages;
  k.value_pages = value_pages;
  k.block_table = block_table;
  k.context_lens = context_lens;
  k.batch = batch;
  k.num_kv_heads = num_kv_heads;
  k.new_len = new_len;
  k.num_pages = num_pages;
  k.page_size = page_size;
  k.max_pages = max_pages;
  k.head_dim = head_dim;
  const hipError_t e = pa::launch_append(k, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, std::string("launch failed: ") + hipGetErrorString(e));
  g_last_error.clear();
  return PA_OK;
}

int paged_attention_varlen_ex(const void* query, const void* key_pages, const void* value_pages,
                              const int32_t* block_table, const int32_t* context_lens,
                              const int32_t* query_start, void* out, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t total_query, int32_t max_query_len,
                              int32_t head_dim, int32_t num_pages, int32_t page_size, int32_t max_pages,
                              float scale, int32_t causal, void* workspace, size_t workspace_bytes,
                              int32_t decode_max_len, int32_t decode_work_items, void* stream) {
  if (!key_pages || !value_pages || !block_table || !context_lens || !query_start)
    return set_error(PA_ERR_INVALID, "a tensor pointer is NULL");
  if (total_query < 0) return set_error(PA_ERR_INVALID, "total_query must be >= 0");
  if (total_query > 0 && (!query || !out)) return set_error(PA_ERR_INVALID, "a tensor pointer is NULL");
  if (causal != 0 && causal != 1) return set_error(PA_ERR_INVALID, "causal must be 0 or 1");
  if (!std::isfinite(scale)) return set_error(PA_ERR_INVALID, "scale must be finite");
  if (total_query > 0 && (max_query_len < 1 || max_query_len > total_query))
    return set_error(PA_ERR_INVALID, "max_query_len must be in [1, total_query]");
  pa::VarlenPlan plan;
  std::string err;
  const pa::Shape s = make_shape(batch, num_q_heads, num_kv_heads, total_query > 0 ? max_query_len : 1,
                                 head_dim, num_pages, page_size, max_pages, causal != 0);
  const int rc = pa::make_plan_varlen(s, decode_max_len, decode_work_items, true, &plan, &err);
  if (rc != pa::kOk) return set_error(rc, err);
  if (int64_t(total_query) * num_q_heads > INT32_MAX)
    return set_error(PA_ERR_UNSUPPORTED, "total_query * num_q_heads exceeds int32");
  if (total_query == 0) {  // no query rows: nothing to compute or write
    g_last_error.clear();
    return PA_OK;
  }
  if (plan.run_prefill && plan.pre.kv_splits > 1 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes)) {
    // a prefill part without the workspace its key-range split needs runs unsplit
    plan.pre.kv_splits = 1;
    plan.pre.workspace_bytes = 0;
    plan.workspace_bytes = plan.run_decode ? plan.dec.workspace_bytes : 0;
  }
  if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
    return set_error(PA_ERR_WORKSPACE, "workspace smaller than paged_attention_varlen_workspace_bytes() = " +
                                           std::to_string(plan.workspace_bytes));
  const size_t q_bytes = size_t(total_query) * num_q_heads * head_dim * 2;
  const size_t pool_bytes = size_t(num_pages) * num_kv_heads * page_size * head_dim * 2;
  if (overlaps(out, q_bytes, query, q_bytes) || overlaps(out, q_bytes, key_pages, pool_bytes) ||
      overlaps(out, q_bytes, value_pages, pool_bytes) ||
      overlaps(out, q_bytes, block_table, size_t(batch) * max_pages * 4) ||
      overlaps(out, q_bytes, context_lens, size_t(batch) * 4) ||
      overlaps(out, q_bytes, query_start, size_t(batch + 1) * 4) ||
      (plan.workspace_bytes > 0 && overlaps(out, q_bytes, workspace, plan.workspace_bytes)))
    return set_error(PA_ERR_INVALID, "out overlaps an input or the workspace");

  pa::KernelArgs k;
  k.query = query;
  k.key_pages = key_pages;
  k.value_pages = value_pages;
  k.block_table = block_table;
  k.context_lens = context_lens;
  k.out = out;
  k.workspace = workspace;
  k.batch = batch;
  k.num_q_heads = num_q_heads;
  k.num_kv_heads = num_kv_heads;
  k.query_len = max_query_len;
  k.num_pages = num_pages;
  k.page_size = page_size;
  k.max_pages = max_pages;
  k.head_dim = head_dim;
  k.scale = scale;
  k.causal = causal;
  k.epoch = next_epoch();
  k.query_start = query_start;
  k.total_query = total_query;
  k.dec_max_len = plan.dec_max_len;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (plan.run_decode) e = pa::launch_decode(k, plan.dec, st);
  if (e == hipSuccess && plan.run_prefill) {
    pa::KernelArgs kp = k;
    if (plan.pre.kv_splits > 1) kp.workspace = static_cast<char*>(workspace) + plan.pre_ws_offset;
    e = pa::launch_prefill(kp, plan.pre, st);
  }
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, std::string("launch failed: ") + hipGetErrorString(e));
  g_last_error.clear();
  return PA_OK;
}

int paged_attention_varlen(const void* query, const void* key_pages, const void* value_pages,
                           const int32_t* block_table, const int32_t* context_lens, const int32_t* query_start,
                           void* out, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t total_query, int32_t max_query_len, int32_t head_dim, int32_t num_pages,
                           int32_t page_size, int32_t max_pages, float scale, int32_t causal, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return paged_attention_varlen_ex(query, key_pages, value_pages, block_table, context_lens, query_start, out,
                                   batch, num_q_heads, num_kv_heads, total_query, max_query_len, head_dim,
                                   num_pages, page_size, max_pages, scale, causal, workspace, workspace_bytes, -1,
                                   0, stream);
}

size_t paged_attention_varlen_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t max_query_len, int32_t head_dim, int32_t page_size,
                                              int32_t max_pages, int32_t decode_max_len,
                                              int32_t decode_work_items) {
  pa::VarlenPlan plan;
  std::string err;
  const pa::Shape s = make_shape(batch, num_q_heads, num_kv_heads, max_query_len, head_dim, 1, page_size,
                                 max_pages, false);
  const int rc = pa::make_plan_varlen(s, decode_max_len, decode_work_items, false, &plan, &err);
  if (rc != pa::kOk) {
    set_error(rc, err);
    return static_cast<size_t>(-1);
  }
  g_last_error.clear();
  return plan.workspace_bytes;
}

int paged_attention_varlen_check_metadata(const int32_t* block_table, const int32_t* context_lens,
                                          const int32_t* query_start, int32_t batch, int32_t max_pages,
                                          int32_t num_pages, int32_t page_size, int32_t total_query,
                                          int32_t max_query_len, int32_t causal, void* stream) {
  if (!block_table || !context_lens || !query_start) return set_error(PA_ERR_INVALID, "a tensor pointer is NULL");
  if (batch < 1 || max_pages < 1 || num_pages < 1 || page_size < 1 || total_query < 0 || max_query_len < 0)
    return set_error(PA_ERR_INVALID, "sizes must be positive (total_query and max_query_len may be 0)");
  std::vector<int32_t> bt(size_t(batch) * max_pages), ctx(batch), qs(size_t(batch) + 1);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(bt.data(), block_table, bt.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(ctx.data(), context_lens, ctx.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(qs.data(), query_start, qs.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(PA_ERR_LAUNCH, std::string("copy failed: ") + hipGetErrorString(e));
  if (qs[0] != 0 || qs[batch] != total_query)
    return set_error(PA_ERR_METADATA, "query_start must start at 0 and end at total_query");
  const int64_t max_ctx = int64_t(max_pages) * page_size;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = int64_t(qs[b + 1]) - qs[b];
    const std::string at = "[" + std::to_string(b) + "]";
    if (L < 0) return set_error(PA_ERR_METADATA, "query_start decreases at " + at);
    if (L > max_query_len) return set_error(PA_ERR_METADATA, "query length of sequence " + at + " > max_query_len");
    if (L == 0) continue;  // a sequence without query rows is never read
    const int32_t c = ctx[b];
    if (c < 1 || c > max_ctx)
      return set_error(PA_ERR_METADATA, "context_lens" + at + " = " + std::to_string(c) +
                                            " outside [1, max_pages * page_size]");
    if (causal && c < L)
      return set_error(PA_ERR_METADATA, "context_lens" + at + " < its query length under causal");
    const int64_t used = (int64_t(c) + page_size - 1) / page_size;
    for (int64_t j = 0; j < used; ++j) {
      const int32_t p = bt[size_t(b) * max_pages + j];
      if (p < 0 || p >= num_pages)
        return set_error(PA_ERR_METADATA, "block_table" + at + "[" + std::to_string(j) + "] = " + std::to_string(p) +
                                              " is not a page of the pool");
    }
  }
  g_last_error.clear();
  return PA_OK;
}

const char* paged_attention_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
