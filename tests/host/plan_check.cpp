// Host-only checks of the planning/validation code (built with g++ and
// AddressSanitizer/UBSan by tests/test_abi.py; no HIP involved).
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "pa_plan.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::printf("FAIL line %d: %s\n", __LINE__, #cond);             \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static pa::Shape shape(int B, int Hq, int Hkv, int L, int D, int ps, int mp, bool causal = true) {
  pa::Shape s;
  s.batch = B; s.num_q_heads = Hq; s.num_kv_heads = Hkv; s.query_len = L; s.head_dim = D;
  s.num_pages = 10; s.page_size = ps; s.max_pages = mp; s.causal = causal;
  return s;
}

int main() {
  pa::Plan p;
  std::string err;
  // invalid sizes
  CHECK(pa::make_plan(shape(0, 32, 8, 1, 128, 16, 4), 0, 0, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 30, 8, 1, 128, 16, 4), 0, 0, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 100, 16, 4), 0, 0, true, &p, &err) == pa::kErrUnsupported);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 264, 16, 4), 0, 0, true, &p, &err) == pa::kErrUnsupported);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 0, 16, 4), 0, 0, true, &p, &err) == pa::kErrInvalid);
  // head dims without an instance of their own run the next larger one (workspace sized for it)
  for (int D : {8, 56, 72, 80, 96, 112, 136, 160, 192, 248}) {
    CHECK(pa::make_plan(shape(2, 8, 2, 1, D, 16, 40), 0, 0, true, &p, &err) == pa::kOk);
    CHECK(p.schedule == pa::kScheduleDecode && p.aligned == (16 % (2048 / pa::instance_dim(D)) == 0));
    pa::Plan q;
    CHECK(pa::make_plan(shape(2, 8, 2, 1, pa::instance_dim(D), 16, 40), 0, 0, true, &q, &err) == pa::kOk);
    CHECK(p.workspace_bytes == q.workspace_bytes);
  }
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 512, 16, 4), 0, 0, true, &p, &err) == pa::kErrUnsupported);
  // other head dims: the decode step (8 KB of K and V per wave) and the workspace follow D
  for (int D : {64, 128, 256}) {
    for (int ps : {8, 16, 32, 64, 5}) {
      CHECK(pa::make_plan(shape(2, 8, 2, 1, D, ps, 40), 0, 0, true, &p, &err) == pa::kOk);
      CHECK(p.schedule == pa::kScheduleDecode && p.aligned == (ps % (2048 / D) == 0));
    }
    CHECK(pa::make_plan(shape(2, 8, 2, 1, D, 16, 40), 0, 0, true, &p, &err) == pa::kOk);
    CHECK(p.workspace_bytes >= size_t(p.work_cap) * 2 * 4 * D * 4);
    CHECK(pa::make_plan(shape(2, 8, 2, 100, D, 64, 40), 0, 0, true, &p, &err) == pa::kOk);
    CHECK(p.schedule == pa::kSchedulePrefill && p.aligned);
  }
  CHECK(pa::make_plan(shape(1, 32, 8, 100, 128, 16, 4), 0, 0, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 100, 128, 16, 4, false), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 128, 16, 4), 4, 0, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 128, 16, 4), -1, 0, true, &p, &err) == pa::kErrInvalid);
  // the 64 x 32 prefill tiling: explicit, native head dims, 64-row tiles, never split
  for (int D : {64, 128, 256}) {
    CHECK(pa::make_plan(shape(4, 32, 8, 2048, D, 128, 16), 3, 0, true, &p, &err) == pa::kOk);
    CHECK(p.schedule == pa::kSchedulePrefill64x32 && p.aligned && p.n_qtiles == 128 && p.num_work == 4096);
    CHECK(p.kv_splits == 1 && p.workspace_bytes == 0);
  }
  CHECK(pa::make_plan(shape(8, 32, 8, 65, 128, 128, 30), 3, 0, true, &p, &err) == pa::kOk);
  CHECK(p.n_qtiles == 5 && p.num_work == 320 && p.kv_splits == 1 && p.workspace_bytes == 0);
  CHECK(pa::make_plan(shape(1, 4, 2, 13, 128, 32, 4), 3, 0, true, &p, &err) == pa::kOk);
  CHECK(p.aligned && p.n_qtiles == 1);
  CHECK(pa::make_plan(shape(1, 4, 2, 13, 128, 16, 4), 3, 0, true, &p, &err) == pa::kOk);
  CHECK(!p.aligned);
  CHECK(pa::make_plan(shape(1, 4, 2, 1, 128, 16, 4), 3, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kSchedulePrefill64x32);  // explicit: even a one-row query
  for (int D : {8, 80, 96, 192})
    CHECK(pa::make_plan(shape(4, 32, 8, 64, D, 128, 16), 3, 0, true, &p, &err) == pa::kErrUnsupported);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 128, 16, 4), 1, -1, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 128, 16, 4), 1, 65537, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 3, 128, 16, 4), 1, 0, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 128, 1 << 20, 1 << 12), 0, 0, true, &p, &err) == pa::kErrUnsupported);
  CHECK(!err.empty());
  // the decode work split's products: granules * work items at most 2^53 (2^43 granules here)
  CHECK(pa::make_plan(shape(1 << 16, 8, 8, 1, 128, 1 << 14, 1 << 16), 1, 0, true, &p, &err) == pa::kErrUnsupported);
  CHECK(pa::make_plan(shape(1 << 14, 8, 8, 1, 128, 1 << 14, 1 << 16), 1, 0, true, &p, &err) == pa::kOk);
  // dispatch on the query length
  for (int L = 1; L <= 64; ++L) {
    for (int G : {1, 2, 4, 8}) {
      CHECK(pa::make_plan(shape(3, 8 * G, 8, L, 128, 16, 300), 0, 0, true, &p, &err) == pa::kOk);
      CHECK(p.schedule == (G * L <= 4 ? pa::kScheduleDecode : pa::kSchedulePrefill));
      if (p.schedule == pa::kScheduleDecode) {
        CHECK(p.rows == G * L && p.rows_pad >= p.rows && p.rows_pad <= 8);
        CHECK(p.work_cap == pa::kDecodeAutoCap && p.work_items == 0);
        CHECK(p.workspace_bytes >= size_t(3) * 8 * 8 + size_t(p.work_cap) * 2 * G * L * 130 * 4);
        CHECK(p.ws_acc_offset % 256 == 0 && p.ws_ml_offset % 256 == 0 && p.ws_ml_offset >= 3 * 8 * 8);
        CHECK(p.ws_ctr_offset == 0);
        CHECK(p.bt_entries == pa::kDecodeWindow / 16 + 2);
      } else {
        CHECK(p.n_qtiles == (G * L + 127) / 128);
        // 3 * 8 * n_qtiles work items, fewer than 512: room for up to 8
        // parts of each key range (4800 keys, 75 tiles); the kernel picks
        // each item's count
        const int64_t nw = int64_t(3) * 8 * p.n_qtiles;
        CHECK(p.num_work == nw);
        const int want = pa::kPrefillMaxSplits;
        CHECK(want == 8 && p.kv_splits == want);
        if (want > 1) {
          CHECK(p.ws_ctr_offset == 0 && p.ws_ml_offset >= size_t(nw) * 8 && p.ws_ml_offset % 256 == 0);
          // one entry per workgroup of the split launch
          CHECK(p.ws_acc_offset >= p.ws_ml_offset + size_t(512) * 128 * 2 * 4 && p.ws_acc_offset % 256 == 0);
          CHECK(p.workspace_bytes >= p.ws_acc_offset + size_t(512) * 128 * 128 * 4);
        } else {
          CHECK(p.workspace_bytes == 0);
        }
      }
    }
  }
  // key-range splits: at least two 64-key tiles per part, none from 512 work items up
  CHECK(pa::make_plan(shape(1, 4, 2, 13, 128, 4, 4), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kSchedulePrefill && p.kv_splits == 1 && p.workspace_bytes == 0);
  CHECK(pa::make_plan(shape(1, 4, 2, 150, 128, 64, 3), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.n_qtiles == 3 && p.num_work == 6 && p.kv_splits == 1);  // 192 keys: one part of two tiles at most
  CHECK(pa::make_plan(shape(1, 4, 2, 150, 128, 64, 4), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.kv_splits == 2 && p.workspace_bytes > 0);
  CHECK(pa::make_plan(shape(1, 4, 2, 150, 128, 64, 7), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.kv_splits == 3);  // 448 keys: 7 tiles, three parts of two at most
  CHECK(pa::make_plan(shape(8, 32, 8, 65, 128, 128, 29), 0, 0, true, &p, &err) == pa::kOk);
  // the chunked continuation: 4 x 65 rows per kv head
  CHECK(p.n_qtiles == 3 && p.num_work == 192 && p.kv_splits == 8);
  CHECK(pa::make_plan(shape(2, 128, 8, 256, 128, 128, 16), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.num_work == 512 && p.kv_splits == 1 && p.workspace_bytes == 0);
  // the five measured shapes
  CHECK(pa::make_plan(shape(64, 32, 8, 1, 128, 128, 33), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kScheduleDecode && p.aligned && p.rows == 4);
  CHECK(pa::make_plan(shape(16, 32, 8, 1, 128, 16, 2048), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kScheduleDecode && p.aligned);
  CHECK(pa::make_plan(shape(4, 32, 8, 2048, 128, 128, 16), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kSchedulePrefill && p.aligned && p.n_qtiles == 64 && p.num_work == 2048);
  CHECK(pa::make_plan(shape(8, 32, 8, 65, 128, 128, 30), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kSchedulePrefill && p.n_qtiles == 3);
  CHECK(pa::make_plan(shape(1, 4, 2, 13, 128, 4, 4), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kSchedulePrefill && !p.aligned);
  // a staging window of any page size fits the block-table entries it needs
  for (int ps : {1, 2, 3, 7, 16, 100, 128, 2047, 2048, 4096}) {
    CHECK(pa::make_plan(shape(2, 8, 8, 1, 128, ps, 10), 1, 0, true, &p, &err) == pa::kOk);
    const int worst = (pa::kDecodeWindow - 1 + ps - 1) / ps + 1;  // window starting one key into a page
    CHECK(p.bt_entries >= worst);
    CHECK(p.aligned == (ps % pa::decode_step(128) == 0));
  }
  // explicit work item counts size the workspace
  CHECK(pa::make_plan(shape(2, 8, 8, 1, 128, 16, 10), 1, 7, true, &p, &err) == pa::kOk);
  CHECK(p.work_items == 7 && p.work_cap == 7);
  // mixed batches: which lengths take the decode schedule, and the parts' plans
  pa::VarlenPlan v;
  for (int maxL : {1, 2, 3, 8, 65, 128, 2048}) {
    for (int G : {1, 2, 4, 8, 16}) {
      CHECK(pa::make_plan_varlen(shape(5, 8 * G, 8, maxL, 128, 16, 300), -1, 0, true, &v, &err) == pa::kOk);
      const int want = G * maxL <= 4 ? maxL : (G <= 4 ? 1 : 0);
      CHECK(v.dec_max_len == want);
      CHECK(v.run_decode == (want > 0) && v.run_prefill == (maxL > want));
      const size_t dec_ws = v.run_decode ? v.dec.workspace_bytes : 0;
      if (v.run_decode) {
        CHECK(v.dec.schedule == pa::kScheduleDecode && v.dec.rows == G * want && v.dec.rows_pad <= 8);
        CHECK(dec_ws > 0);
      }
      if (v.run_prefill) {
        CHECK(v.pre.schedule == pa::kSchedulePrefill && v.pre.n_qtiles == (G * maxL + 127) / 128);
        if (v.pre.kv_splits > 1) {
          CHECK(v.pre_ws_offset >= dec_ws && v.pre_ws_offset % 256 == 0);
          CHECK(v.workspace_bytes == v.pre_ws_offset + v.pre.workspace_bytes);
        } else {
          CHECK(v.workspace_bytes == dec_ws);
        }
      } else {
        CHECK(v.workspace_bytes == dec_ws);
      }
    }
  }
  CHECK(pa::make_plan_varlen(shape(64, 32, 8, 128, 128, 128, 9), 0, 0, true, &v, &err) == pa::kOk);
  CHECK(!v.run_decode && v.run_prefill && v.dec_max_len == 0 && v.pre.num_work == 2048 && v.workspace_bytes == 0);
  CHECK(pa::make_plan_varlen(shape(64, 32, 8, 128, 128, 128, 9), 1, 0, true, &v, &err) == pa::kOk);
  CHECK(v.run_decode && v.run_prefill && v.dec_max_len == 1 && v.dec.rows == 4);
  CHECK(pa::make_plan_varlen(shape(64, 32, 8, 128, 128, 128, 9), 3, 0, true, &v, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan_varlen(shape(64, 32, 8, 128, 128, 128, 9), -2, 0, true, &v, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan_varlen(shape(64, 32, 8, 128, 128, 128, 9), -1, -1, true, &v, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan_varlen(shape(64, 32, 8, 128, 128, 128, 9), -1, 70000, true, &v, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan_varlen(shape(64, 30, 8, 128, 128, 128, 9), -1, 0, true, &v, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan_varlen(shape(64, 32, 8, 128, 100, 128, 9), -1, 0, true, &v, &err) == pa::kErrUnsupported);
  // explicit decode work items reach the decode part
  CHECK(pa::make_plan_varlen(shape(4, 32, 8, 1, 128, 16, 9), -1, 5, true, &v, &err) == pa::kOk);
  CHECK(v.run_decode && !v.run_prefill && v.dec.work_items == 5 && v.dec.work_cap == 5);
  // scale folding: c > 0 always; a negative scale flips the query's sign bits
  {
    const pa::ScaleFold pos = pa::fold_scale(0.0883883f);
    CHECK(pos.qsign == 0u && pos.c > 0.127f && pos.c < 0.128f);
    const pa::ScaleFold neg = pa::fold_scale(-0.0883883f);
    CHECK(neg.qsign == 0x80008000u && neg.c == pos.c);
    const pa::ScaleFold zero = pa::fold_scale(0.0f);
    CHECK(zero.qsign == 0u && zero.c > 0.f && zero.c < 1e-37f);
    const pa::ScaleFold nzero = pa::fold_scale(-0.0f);
    CHECK(nzero.qsign == 0u && nzero.c == zero.c);
  }
  if (failures == 0) std::printf("plan_check: all passed\n");
  return failures == 0 ? 0 : 1;
}
