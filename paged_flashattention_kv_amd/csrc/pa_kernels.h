// pa_kernels.h -- launch entry points of the two gfx950 schedules, called by
// the C-ABI layer after validation and planning.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_plan.h"

namespace pa {

struct KernelArgs {
  const void* query;
  const void* key_pages;
  const void* value_pages;
  const int32_t* block_table;
  const int32_t* context_lens;
  void* out;
  void* workspace;
  int batch, num_q_heads, num_kv_heads, query_len, num_pages, page_size, max_pages;
  int head_dim = 128;  // a multiple of 8 up to 256 (the row length of query, pages and out)
  float scale;
  int causal;
  uint32_t epoch;  // per-call tag of the arrival counters in the workspace (never 0)
  // Mixed batch: query and out are packed token-major [total_query, H_q, D]
  // and sequence b owns tokens [query_start[b], query_start[b + 1]);
  // query_len is then the longest query of the batch. The decode launch
  // serves sequences with 1 <= L_b <= dec_max_len, the prefill launch those
  // with L_b > dec_max_len. query_start == nullptr: the uniform layout
  // [B, H_q, query_len, D], every sequence served by the one launch.
  const int32_t* query_start = nullptr;
  int total_query = 0;
  int dec_max_len = 0;
  // Explicit additive mask (natural-log units, uniform layout only): row
  // (b, h, l), key s at mask[b*mask_stride_b + h*mask_stride_h +
  // l*mask_stride_l + s] for s < mask_len; keys at or past mask_len are
  // absent. nullptr: no mask.
  const float* mask = nullptr;
  int64_t mask_stride_b = 0, mask_stride_h = 0, mask_stride_l = 0;
  int mask_len = 0;
};

// Short-query split-context schedule (pa_decode.hip).
hipError_t launch_decode(const KernelArgs& k, const Plan& p, hipStream_t stream);

// Long-query bf16-MFMA tiled schedule (pa_prefill.hip).
hipError_t launch_prefill(const KernelArgs& k, const Plan& p, hipStream_t stream);

struct AppendKernelArgs {
  const void* key_new;
  const void* value_new;
  void* key_pages;
  void* value_pages;
  const int32_t* block_table;
  const int32_t* context_lens;
  int batch, num_kv_heads, new_len, num_pages, page_size, max_pages;
  int head_dim = 128;  // a multiple of 8 up to 256
};

// Writes new tokens' K/V into their page slots (pa_append.hip).
hipError_t launch_append(const AppendKernelArgs& k, hipStream_t stream);

}  // namespace pa
