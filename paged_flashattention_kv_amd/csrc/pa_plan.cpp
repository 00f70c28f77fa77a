// pa_plan.cpp -- validation and launch planning (host only, no HIP).
#include "pa_plan.h"

#include <climits>

namespace pa {

namespace {

int fail(std::string* err, int code, const std::string& msg) {
  if (err) *err = msg;
  return code;
}

int log2_exact(int64_t v) {
  if (v <= 0 || (v & (v - 1)) != 0) return -1;
  int r = 0;
  while ((int64_t(1) << r) < v) ++r;
  return r;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

int auto_decode_split(int64_t batch, int64_t num_kv_heads, int64_t max_ctx, int64_t page_size) {
  // Smallest split (512, 1024, ...) that keeps the grid at or under ~4096
  // work items: enough to fill 256 CUs several times over while each work
  // item still streams at least 512 keys (256 KiB of K+V).
  const int64_t pairs = batch * num_kv_heads;
  int64_t split = 512;
  while (split < 65536 && pairs * cdiv(max_ctx, split) > 4096) split *= 2;
  // Never stage more block-table entries than the kernel's LDS holds.
  while (split > 256 && cdiv(split, page_size) + 1 > kDecodeMaxBt) split /= 2;
  return int(split);
}

int make_plan(const Shape& s, int schedule, int decode_split, bool check_pool, Plan* plan,
              std::string* err) {
  if (s.batch < 1 || s.num_q_heads < 1 || s.num_kv_heads < 1 || s.query_len < 1 ||
      s.head_dim < 1 || s.page_size < 1 || s.max_pages < 1)
    return fail(err, kErrInvalid, "all sizes must be positive");
  if (check_pool && s.num_pages < 1) return fail(err, kErrInvalid, "num_pages must be positive");
  if (s.num_q_heads % s.num_kv_heads != 0)
    return fail(err, kErrInvalid, "num_q_heads must be a multiple of num_kv_heads");
  if (s.head_dim != kHeadDim) return fail(err, kErrUnsupported, "only head_dim == 128 is implemented");
  const int64_t max_ctx = s.max_pages * s.page_size;
  if (max_ctx > INT32_MAX) return fail(err, kErrUnsupported, "max_pages * page_size exceeds int32");
  if (s.causal && max_ctx < s.query_len)
    return fail(err, kErrInvalid, "causal attention needs max_pages * page_size >= query_len");
  if (s.batch * s.num_q_heads * s.query_len > INT32_MAX)
    return fail(err, kErrUnsupported, "batch * num_q_heads * query_len exceeds int32");
  if (schedule < 0 || schedule > 2) return fail(err, kErrInvalid, "schedule must be 0, 1 or 2");

  Plan p;
  p.group = int(s.num_q_heads / s.num_kv_heads);
  p.max_ctx = max_ctx;
  p.ps_log2 = log2_exact(s.page_size);
  const int64_t rows = int64_t(p.group) * s.query_len;
  if (schedule == 0) schedule = rows <= kDecodeMaxRows ? kScheduleDecode : kSchedulePrefill;
  p.schedule = schedule;

  if (schedule == kScheduleDecode) {
    if (rows > kDecodeMaxRows)
      return fail(err, kErrInvalid,
                  "decode schedule needs query_len * num_q_heads / num_kv_heads <= 8");
    p.rows = int(rows);
    p.rows_pad = 1;
    while (p.rows_pad < p.rows) p.rows_pad *= 2;
    int split = decode_split;
    if (split == 0) {
      split = auto_decode_split(s.batch, s.num_kv_heads, max_ctx, s.page_size);
    } else if (split < 256 || split > 65536 || split % 256 != 0) {
      return fail(err, kErrInvalid, "decode_split must be a multiple of 256 in [256, 65536]");
    }
    if (cdiv(split, s.page_size) + 1 > kDecodeMaxBt)
      return fail(err, kErrInvalid, "decode_split / page_size too large for the staged block table");
    p.split_len = split;
    p.n_split = int(cdiv(max_ctx, split));
    p.direct = p.n_split == 1;
    p.bt_entries = int(cdiv(split, s.page_size) + 1);
    p.aligned = s.page_size % kDecodeTile == 0;
    p.num_work = int64_t(p.n_split) * s.num_kv_heads * s.batch;
    if (p.num_work > INT32_MAX) return fail(err, kErrUnsupported, "decode grid too large");
    if (!p.direct) {
      const size_t nrows = size_t(s.batch) * size_t(s.num_q_heads) * size_t(s.query_len);
      p.ws_acc_offset = 0;
      p.ws_ml_offset = align_up(nrows * size_t(p.n_split) * kHeadDim * sizeof(float), 256);
      p.workspace_bytes = align_up(p.ws_ml_offset + nrows * size_t(p.n_split) * 2 * sizeof(float), 256);
    }
  } else {
    p.n_qtiles = int(cdiv(s.query_len, kPrefillBlockM));
    p.aligned = s.page_size % kPrefillBlockN == 0;
    p.num_work = int64_t(p.n_qtiles) * s.num_q_heads * s.batch;
    if (p.num_work > INT32_MAX) return fail(err, kErrUnsupported, "prefill grid too large");
  }
  *plan = p;
  if (err) err->clear();
  return kOk;
}

}  // namespace pa
