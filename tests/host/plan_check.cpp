// Host-only checks of the planning/validation code (built with g++ and
// AddressSanitizer/UBSan by tests/test_abi.py; no HIP involved).
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
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 64, 16, 4), 0, 0, true, &p, &err) == pa::kErrUnsupported);
  CHECK(pa::make_plan(shape(1, 32, 8, 100, 128, 16, 4), 0, 0, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 100, 128, 16, 4, false), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 128, 16, 4), 3, 0, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 128, 16, 4), 1, 100, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 3, 128, 16, 4), 1, 0, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 128, 1, 100000), 1, 4096, true, &p, &err) == pa::kErrInvalid);
  CHECK(pa::make_plan(shape(1, 32, 8, 1, 128, 1 << 20, 1 << 12), 0, 0, true, &p, &err) == pa::kErrUnsupported);
  CHECK(!err.empty());
  // dispatch on the query length
  for (int L = 1; L <= 64; ++L) {
    for (int G : {1, 2, 4, 8}) {
      CHECK(pa::make_plan(shape(3, 8 * G, 8, L, 128, 16, 300), 0, 0, true, &p, &err) == pa::kOk);
      CHECK(p.schedule == (G * L <= 8 ? pa::kScheduleDecode : pa::kSchedulePrefill));
      if (p.schedule == pa::kScheduleDecode) {
        CHECK(p.rows == G * L && p.rows_pad >= p.rows && p.rows_pad <= 8);
        CHECK(p.split_len % 256 == 0 && p.n_split * (long)p.split_len >= p.max_ctx);
        CHECK((p.n_split == 1) == p.direct);
        CHECK(p.direct ? p.workspace_bytes == 0 : p.workspace_bytes >= size_t(3) * 8 * G * L * p.n_split * 130 * 4);
        CHECK(p.bt_entries <= pa::kDecodeMaxBt);
      } else {
        CHECK(p.n_qtiles == (L + 127) / 128 && p.workspace_bytes == 0);
      }
    }
  }
  // the five measured shapes
  CHECK(pa::make_plan(shape(64, 32, 8, 1, 128, 128, 33), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kScheduleDecode && p.aligned && p.rows == 4);
  CHECK(pa::make_plan(shape(16, 32, 8, 1, 128, 16, 2048), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kScheduleDecode && !p.aligned && p.num_work >= 1024);
  CHECK(pa::make_plan(shape(4, 32, 8, 2048, 128, 128, 16), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kSchedulePrefill && p.aligned && p.n_qtiles == 16);
  CHECK(pa::make_plan(shape(8, 32, 8, 65, 128, 128, 30), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kSchedulePrefill && p.n_qtiles == 1);
  CHECK(pa::make_plan(shape(1, 4, 2, 13, 128, 4, 4), 0, 0, true, &p, &err) == pa::kOk);
  CHECK(p.schedule == pa::kSchedulePrefill && !p.aligned);
  // automatic split lengths stay within the staged block table
  for (int ps : {1, 2, 3, 16, 100, 128, 4096})
    for (int ctx : {1, 100, 5000, 70000, 1 << 20}) {
      const int s = pa::auto_decode_split(16, 8, ctx, ps);
      CHECK(s >= 256 && s % 256 == 0 && (s + ps - 1) / ps + 1 <= pa::kDecodeMaxBt);
    }
  if (failures == 0) std::printf("plan_check: all passed\n");
  return failures == 0 ? 0 : 1;
}
