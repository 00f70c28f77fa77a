// pa_plan.h -- host-side argument validation and launch planning for the
// paged attention operator. Pure C++ (no HIP): it decides which schedule
// runs, with which tile/split parameters, and how much workspace it needs.
// Kept free of device code so that it can be unit-tested on a CPU-only host
// under AddressSanitizer/UBSan.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <string>

namespace pa {

// Head dims the operator serves: any multiple of 8 from 8 to 256. 64, 128
// and 256 have kernel instances of their own; any other runs the next larger
// instance with the dims past it masked (zero query, no output stores).
constexpr bool head_dim_supported(int64_t d) { return d >= 8 && d <= 256 && d % 8 == 0; }
constexpr int instance_dim(int64_t d) { return d <= 64 ? 64 : d <= 128 ? 128 : 256; }
// keys per decode wave step: 8 KB of K and V at the instance's head dim (two
// keys per lane, 16 dims each)
constexpr int decode_step(int64_t head_dim) { return int(2048 / instance_dim(head_dim)); }
constexpr int kDecodeMaxRows = 8;    // q rows (GQA group x query_len) per decode work item
// The automatic dispatch sends a query to the decode schedule while its rows
// per kv head stay within kDecodeAutoRows. Measured over query lengths 1-16,
// contexts 128-32768 and GQA 1, 4 and 8 (16 sequences, Qwen3-4B head
// count): with 6 or 8 rows the tiled prefill schedule was faster at every
// context (1.2-2.8x); with up to 4 rows the decode schedule wins once a call
// streams several hundred MB of K/V, and it balances ragged batches.
constexpr int kDecodeAutoRows = 4;
constexpr int kDecodeWindow = 2048;  // keys whose block-table entries a decode work item stages at once
constexpr int kDecodeAutoCap = 2048; // most decode work items the automatic choice launches
constexpr int kDecodeMaxWork = 65536;
constexpr int kPrefillBlockM = 128;  // packed (position, query head) rows per prefill work item
constexpr int kPrefillBlockN = 64;   // keys per prefill K/V tile
// A prefill launch with fewer work items than kPrefillSplitTarget (two per CU
// on a 256-CU part) splits the work items' key ranges into parts of about
// equal length, merged through the workspace: the kernel picks the shortest
// part length at which all parts fit the resident workgroups (at most
// kPrefillSplitTarget) and gives each work item as many parts as its own
// length calls for (at most kPrefillMaxSplits, at least two tiles each).
constexpr int kPrefillSplitTarget = 512;
constexpr int kPrefillMaxSplits = 8;
constexpr int kScheduleDecode = 1;
constexpr int kSchedulePrefill = 2;
// The prefill schedule at 64 packed rows x 32 keys per tile (two waves per
// work item): the tiling of the matrix kernel in "Week 3 Day 5: Paged
// FlashAttention", Task 1, kept to measure the 128 x 64 tiling against.
// Explicit only; native head dims (64, 128, 256), no explicit mask, never
// split.
constexpr int kSchedulePrefill64x32 = 3;
constexpr int kPrefill64x32Rows = 64;
constexpr int kPrefill64x32Keys = 32;

struct Shape {
  int64_t batch = 0, num_q_heads = 0, num_kv_heads = 0, query_len = 0, head_dim = 0;
  int64_t num_pages = 1;  // only checked when the call has a page pool
  int64_t page_size = 0, max_pages = 0;
  bool causal = true;
};

struct Plan {
  int schedule = 0;
  int group = 0;           // num_q_heads / num_kv_heads
  int rows = 0;            // decode: q rows per work item (group * query_len)
  int rows_pad = 0;        // decode: rows rounded up to 1, 2, 4 or 8
  int work_items = 0;      // decode: requested work items (0 = as many as stay resident)
  int work_cap = 0;        // decode: most work items the workspace is sized for
  int bt_entries = 0;      // decode: block-table entries staged per window
  int n_qtiles = 0;        // prefill: 128-row (64-row) tiles of the group * query_len rows of a (sequence, kv head)
  int kv_splits = 1;       // prefill: parts of each work item's key range (1: no split)
  int ps_log2 = -1;        // log2(page_size) or -1 if not a power of two
  bool aligned = false;    // every tile lies inside one page
  int64_t max_ctx = 0;     // max_pages * page_size
  int64_t num_work = 0;    // work items (workgroups) of the main kernel
  size_t workspace_bytes = 0;
  // decode: arrival counters [B * H_kv] u64 (zero-filled before first use),
  // partial (max, sum) [work_cap][2][rows][2] f32, partial outputs
  // [work_cap][2][rows][D] f32. Split prefill: counters [num_work] u64,
  // (max, sum) [kPrefillSplitTarget][128][2] f32, outputs
  // [kPrefillSplitTarget][128][D] f32.
  size_t ws_ctr_offset = 0;
  size_t ws_ml_offset = 0;
  size_t ws_acc_offset = 0;
};

// Error codes (the same values as the PA_ERR_* codes of the C header).
constexpr int kOk = 0;
constexpr int kErrInvalid = -1;
constexpr int kErrUnsupported = -2;
constexpr int kErrWorkspace = -3;

// A mixed batch (per-sequence query lengths, queries packed token-major):
// sequences with 1 <= L_b <= dec_max_len run the decode schedule, longer
// ones the prefill schedule, as two launches on one stream.
struct VarlenPlan {
  int dec_max_len = 0;
  bool run_decode = false;
  bool run_prefill = false;
  Plan dec;  // decode part: rows = group * dec_max_len (the workspace slot stride)
  Plan pre;  // prefill part: query tiles cover max_query_len
  size_t pre_ws_offset = 0;  // the prefill part's workspace (key-range split) follows the decode part's
  size_t workspace_bytes = 0;
};

// How a finite `scale` reaches the kernels. Both schedules take the running
// maximum on raw q.k scores and multiply by c = scale * log2(e) afterwards,
// which is the maximum of the scaled scores only for c > 0. A negative scale
// is therefore folded into the query: q.k * scale = (-q).k * |scale|, and
// negating a bf16 value flips its sign bit exactly (qsign is XORed into every
// packed pair of query values). A zero scale -- every visible key weighted
// alike -- becomes the least normal float: for raw scores below 2^100 in
// magnitude the exponent argument stays under 2^-25, so each weight rounds to
// exactly 1 in bf16, which is the uniform softmax a zero scale defines, while
// hidden keys (-inf scores) keep weight 0.
struct ScaleFold {
  float c;         // |scale| * log2(e) (> 0)
  uint32_t qsign;  // 0x80008000 for a negative scale, else 0
};

inline ScaleFold fold_scale(float scale) {
  constexpr float kLog2eHost = 1.4426950408889634f;
  const float mag = std::fabs(scale);
  ScaleFold f;
  f.c = (mag > 0.f ? mag : 0x1p-126f) * kLog2eHost;
  f.qsign = std::signbit(scale) && mag > 0.f ? 0x80008000u : 0u;
  return f;
}

// Validates `s` and fills `plan`. `schedule` is 0 (auto), 1 (decode), 2
// (prefill) or 3 (prefill at 64 x 32 tiles); `decode_work_items` is 0 (auto)
// or an explicit number of decode work items. Returns kOk or a negative code
// with a message in `err`.
int make_plan(const Shape& s, int schedule, int decode_work_items, bool check_pool, Plan* plan,
              std::string* err);

// Plans a mixed batch. `s.query_len` is the longest query of the batch
// (max_query_len). `decode_max_len` is -1 (auto: max_query_len when
// group * max_query_len <= 8, else 1 when group <= 8, else 0), 0 (every
// sequence takes the prefill schedule) or an explicit bound with
// group * decode_max_len <= 8.
int make_plan_varlen(const Shape& s, int decode_max_len, int decode_work_items, bool check_pool,
                     VarlenPlan* plan, std::string* err);

}  // namespace pa
