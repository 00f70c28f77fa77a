// pa_plan.cpp -- validation and launch planning (host only, no HIP).
#include "pa_plan.h"

#include <algorithm>
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

int make_plan(const Shape& s, int schedule, int decode_work_items, bool check_pool, Plan* plan,
              std::string* err) {
  if (s.batch < 1 || s.num_q_heads < 1 || s.num_kv_heads < 1 || s.query_len < 1 ||
      s.head_dim < 1 || s.page_size < 1 || s.max_pages < 1)
    return fail(err, kErrInvalid, "all sizes must be positive");
  if (check_pool && s.num_pages < 1) return fail(err, kErrInvalid, "num_pages must be positive");
  if (s.num_q_heads % s.num_kv_heads != 0)
    return fail(err, kErrInvalid, "num_q_heads must be a multiple of num_kv_heads");
  if (!head_dim_supported(s.head_dim))
    return fail(err, kErrUnsupported, "head_dim must be a multiple of 8 from 8 to 256");
  const int64_t max_ctx = s.max_pages * s.page_size;
  if (max_ctx > INT32_MAX) return fail(err, kErrUnsupported, "max_pages * page_size exceeds int32");
  if (s.causal && max_ctx < s.query_len)
    return fail(err, kErrInvalid, "causal attention needs max_pages * page_size >= query_len");
  if (s.batch * s.num_q_heads * s.query_len > INT32_MAX)
    return fail(err, kErrUnsupported, "batch * num_q_heads * query_len exceeds int32");
  if (schedule < 0 || schedule > 3) return fail(err, kErrInvalid, "schedule must be 0, 1, 2 or 3");
  if (schedule == kSchedulePrefill64x32 && instance_dim(s.head_dim) != s.head_dim)
    return fail(err, kErrUnsupported, "the 64 x 32 prefill tiling serves head dims 64, 128 and 256");

  Plan p;
  p.group = int(s.num_q_heads / s.num_kv_heads);
  p.max_ctx = max_ctx;
  p.ps_log2 = log2_exact(s.page_size);
  const int64_t rows = int64_t(p.group) * s.query_len;
  if (schedule == 0) schedule = rows <= kDecodeAutoRows ? kScheduleDecode : kSchedulePrefill;
  p.schedule = schedule;

  if (schedule == kScheduleDecode) {
    if (rows > kDecodeMaxRows)
      return fail(err, kErrInvalid,
                  "decode schedule needs query_len * num_q_heads / num_kv_heads <= 8");
    p.rows = int(rows);
    p.rows_pad = 1;
    while (p.rows_pad < p.rows) p.rows_pad *= 2;
    if (decode_work_items < 0 || decode_work_items > kDecodeMaxWork)
      return fail(err, kErrInvalid, "decode_work_items must be in [0, 65536]");
    p.work_items = decode_work_items;
    p.work_cap = decode_work_items > 0 ? decode_work_items : kDecodeAutoCap;
    // the work split's products must stay inside int64: cost units (at most
    // 3x the granules, a segment start costing 2) times the weight before a
    // work item (at most 16 per item, times work_cap items), with room to spare
    const int64_t granules = s.batch * s.num_kv_heads * cdiv(max_ctx, 64);
    if (granules > (int64_t(1) << 53) / p.work_cap)
      return fail(err, kErrUnsupported, "decode work too large for the granule arithmetic");
    p.bt_entries = int(kDecodeWindow / s.page_size + 2);
    p.aligned = s.page_size % decode_step(s.head_dim) == 0;  // a wave step lies inside one page
    p.num_work = p.work_cap;
    const size_t slots = size_t(p.work_cap) * 2 * size_t(p.rows);
    p.ws_ctr_offset = 0;
    p.ws_ml_offset = align_up(size_t(s.batch) * size_t(s.num_kv_heads) * sizeof(uint64_t), 256);
    p.ws_acc_offset = align_up(p.ws_ml_offset + slots * 2 * sizeof(float), 256);
    p.workspace_bytes = align_up(p.ws_acc_offset + slots * size_t(instance_dim(s.head_dim)) * sizeof(float), 256);
  } else if (schedule == kSchedulePrefill64x32) {
    p.n_qtiles = int(cdiv(rows, kPrefill64x32Rows));
    p.aligned = s.page_size % kPrefill64x32Keys == 0;
    p.num_work = int64_t(p.n_qtiles) * s.num_kv_heads * s.batch;
    if (p.num_work > INT32_MAX) return fail(err, kErrUnsupported, "prefill grid too large");
  } else {
    // rows of a work item: (position, query head) pairs of one kv head's group
    p.n_qtiles = int(cdiv(rows, kPrefillBlockM));
    p.aligned = s.page_size % kPrefillBlockN == 0;
    p.num_work = int64_t(p.n_qtiles) * s.num_kv_heads * s.batch;
    if (p.num_work > INT32_MAX) return fail(err, kErrUnsupported, "prefill grid too large");
    if (p.num_work < kPrefillSplitTarget) {
      // room for up to kPrefillMaxSplits parts per work item (the kernel picks each item's count)
      const int64_t splits = std::min<int64_t>(kPrefillMaxSplits, max_ctx / (2 * kPrefillBlockN));
      p.kv_splits = int(std::max<int64_t>(splits, 1));
    }
    if (p.kv_splits > 1) {
      // one entry per workgroup of the split launch: kPrefillSplitTarget parts at most
      const size_t parts = size_t(kPrefillSplitTarget) * kPrefillBlockM;
      p.ws_ctr_offset = 0;
      p.ws_ml_offset = align_up(size_t(p.num_work) * sizeof(uint64_t), 256);
      p.ws_acc_offset = align_up(p.ws_ml_offset + parts * 2 * sizeof(float), 256);
      p.workspace_bytes =
          align_up(p.ws_acc_offset + parts * size_t(instance_dim(s.head_dim)) * sizeof(float), 256);
    }
  }
  *plan = p;
  if (err) err->clear();
  return kOk;
}

int make_plan_varlen(const Shape& s, int decode_max_len, int decode_work_items, bool check_pool,
                     VarlenPlan* plan, std::string* err) {
  // the checks every part shares (sizes, GQA ratio, head_dim) come from make_plan
  Plan probe;
  int rc = make_plan(s, kSchedulePrefill, 0, check_pool, &probe, err);
  if (rc != kOk) return rc;
  const int group = probe.group;
  VarlenPlan v;
  if (decode_max_len < -1) return fail(err, kErrInvalid, "decode_max_len must be -1 (auto), 0 or positive");
  if (decode_work_items < 0 || decode_work_items > kDecodeMaxWork)
    return fail(err, kErrInvalid, "decode_work_items must be in [0, 65536]");
  if (decode_max_len == -1) {
    // Every query fits the automatic decode bound: the uniform rule.
    // Otherwise only one-token queries take the decode schedule, if their
    // rows fit the bound: its cost grows with the rows of its widest sequence
    // (2.2x from 4 to 8 rows, measured), so a 2-token query would slow every
    // decode of the batch.
    if (int64_t(group) * s.query_len <= kDecodeAutoRows)
      v.dec_max_len = int(s.query_len);
    else
      v.dec_max_len = group <= kDecodeAutoRows ? 1 : 0;
  } else {
    if (int64_t(decode_max_len) * group > kDecodeMaxRows)
      return fail(err, kErrInvalid, "decode_max_len * num_q_heads / num_kv_heads must be <= 8");
    v.dec_max_len = int(std::min<int64_t>(decode_max_len, s.query_len));
  }
  if (v.dec_max_len > 0) {
    Shape sd = s;
    sd.query_len = v.dec_max_len;
    rc = make_plan(sd, kScheduleDecode, decode_work_items, check_pool, &v.dec, err);
    if (rc != kOk) return rc;
    v.run_decode = true;
    v.workspace_bytes = v.dec.workspace_bytes;
  }
  if (s.query_len > v.dec_max_len) {
    v.pre = probe;
    v.run_prefill = true;
    if (v.pre.kv_splits > 1) {
      v.pre_ws_offset = align_up(v.workspace_bytes, 256);
      v.workspace_bytes = v.pre_ws_offset + v.pre.workspace_bytes;
    }
  }
  *plan = v;
  if (err) err->clear();
  return kOk;
}

}  // namespace pa
