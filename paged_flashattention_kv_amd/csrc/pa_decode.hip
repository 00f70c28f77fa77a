// pa_decode.hip -- short-query (decode) schedule of the paged attention
// operator for gfx950.
//
// What it computes: the online-softmax attention of "Week 2 Day 5: Fused
// Decode Attention" (Task 2: cached scaled query in registers, lane-partial
// dot products reduced across lanes, running maximum / denominator /
// weighted-V accumulator, each rescale factor computed once; partial states
// merged through a common maximum) over paged K/V ("Week 3 Day 5: Paged
// FlashAttention", Task 1: logical position -> block_table -> page slot).
//
// Schedule (HBM-bound; no matrix cores):
//   work item = (split of the context, kv head, sequence), 256 threads.
//   All query rows that read this kv head -- the GQA group times the query
//   length, at most 8 rows -- are served by ONE pass over the split's keys,
//   so every K/V byte is read from HBM once per kv head.
//   Each wave walks 32-key tiles of the split (waves interleave tiles).
//   Lane layout inside a tile: lane = 8 * kg + dc. Lane (kg, dc) holds keys
//   kg, kg+8, kg+16, kg+24 of the tile and, for each, head dims
//   [8dc, 8dc+8) and [64+8dc, 64+8dc+8): two 16-byte loads per key row, and
//   one load instruction covers eight 128-byte row halves.
//   q.k: packed bf16 dot products (v_dot2_f32_bf16), then a sum over the 8
//   lanes of the key (DPP). The running maximum is shared by the whole wave
//   (reduced per tile), so partial sums over the wave's lanes need no
//   rescaling when they are combined at the end.
//   Split end: wave partials are summed across lanes, then the 4 waves merge
//   in LDS through a common maximum. With one split per sequence the result
//   is normalised and stored directly; otherwise the split's (max, sum, acc)
//   goes to the workspace and pa_decode_merge combines the splits.
//
// Page translation ("Week 3 Day 5", Task 1): the split's block-table entries
// are staged in LDS once. Aligned path (page_size % 32 == 0): a 32-key tile
// lies inside one page, so its rows are one contiguous 8 KiB span found
// with one table entry. Generic path: every key row is translated
// separately (tiles that cross page boundaries, e.g. 16-token pages).
// Keys at or past the split end are never loaded (their page may not
// exist); their scores are forced to -inf by a separate mask ("Day 22: the
// fused paged-attention kernel", "What I learned", item 2).

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 32;

struct DecodeArgs {
  const uint16_t* query;
  const uint16_t* kpages;
  const uint16_t* vpages;
  const int32_t* block_table;
  const int32_t* context_lens;
  uint16_t* out;
  float* ws_acc;
  float* ws_ml;
  int num_q_heads, num_kv_heads, query_len, group, rows;
  int page_size, ps_log2, max_pages;
  int split_len, n_split;
  float c;  // scale * log2(e)
  int causal;
};

__device__ __forceinline__ int div_ps(int s, int ps, int ps_log2) { return ps_log2 >= 0 ? (s >> ps_log2) : s / ps; }

template <int ROWS, bool ALIGNED, bool DIRECT>
__global__ void __launch_bounds__(kThreads) pa_decode_split(DecodeArgs a) {
  extern __shared__ int32_t lds_bt[];
  __shared__ float lds_m[kWaves][ROWS];
  __shared__ float lds_l[kWaves][ROWS];
  __shared__ float lds_acc[kWaves][ROWS][128];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 3;
  const int dc = lane & 7;

  int wid = blockIdx.x;
  const int split = wid % a.n_split;
  wid /= a.n_split;
  const int kvh = wid % a.num_kv_heads;
  const int b = wid / a.num_kv_heads;

  const int ctx = a.context_lens[b];
  const int s0 = split * a.split_len;
  if (s0 >= ctx) return;  // this split holds no key of the sequence
  const int s1 = min(s0 + a.split_len, ctx);

  // Stage the split's block-table entries.
  const int lp0 = div_ps(s0, a.page_size, a.ps_log2);
  const int nbt = div_ps(s1 - 1, a.page_size, a.ps_log2) - lp0 + 1;
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages + lp0;
  for (int i = tid; i < nbt; i += kThreads) lds_bt[i] = bt_row[i];

  // Query rows of this kv head: row r -> q head kvh*group + r / L, position r % L.
  uint32_t q[ROWS][8];
  int last[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    if (r < a.rows) {
      const int h = kvh * a.group + r / a.query_len;
      const int l = r % a.query_len;
      const uint16_t* qp = a.query + (((size_t)b * a.num_q_heads + h) * a.query_len + l) * 128;
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(qp + dc * 8);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(qp + 64 + dc * 8);
      q[r][0] = lo.x; q[r][1] = lo.y; q[r][2] = lo.z; q[r][3] = lo.w;
      q[r][4] = hi.x; q[r][5] = hi.y; q[r][6] = hi.z; q[r][7] = hi.w;
      last[r] = a.causal ? l + ctx - a.query_len : ctx - 1;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) q[r][j] = 0u;
      last[r] = ctx - 1;
    }
  }
  int min_last = ctx - 1;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) min_last = min(min_last, last[r]);
  __syncthreads();

  float m[ROWS], lsum[ROWS], acc[ROWS][16];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    m[r] = -INFINITY;
    lsum[r] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[r][j] = 0.f;
  }

  const size_t head_stride = (size_t)a.page_size * 128;  // elements between kv heads of a page
  const size_t page_stride = head_stride * a.num_kv_heads;
  const size_t head_off = (size_t)kvh * head_stride;

  for (int t0 = s0 + wave * kTile; t0 < s1; t0 += kWaves * kTile) {
    // ---- page-translating load of the tile's K and V rows (registers) ----
    u32x4_t kr[4][2], vr[4][2];
    size_t row_off[4];
    bool ok[4];
    if (ALIGNED) {
      const int lp = div_ps(t0, a.page_size, a.ps_log2);
      const int slot0 = t0 - lp * a.page_size;
      const size_t base = (size_t)lds_bt[lp - lp0] * page_stride + head_off + (size_t)slot0 * 128;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        row_off[i] = base + (size_t)(kg + 8 * i) * 128;
        ok[i] = t0 + kg + 8 * i < s1;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = t0 + kg + 8 * i;
        ok[i] = s < s1;
        const int sc = ok[i] ? s : s0;
        const int lp = div_ps(sc, a.page_size, a.ps_log2);
        const int slot = sc - lp * a.page_size;
        row_off[i] = (size_t)lds_bt[lp - lp0] * page_stride + head_off + (size_t)slot * 128;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ok[i]) {
        kr[i][0] = *reinterpret_cast<const u32x4_t*>(a.kpages + row_off[i] + dc * 8);
        kr[i][1] = *reinterpret_cast<const u32x4_t*>(a.kpages + row_off[i] + 64 + dc * 8);
      } else {
        kr[i][0] = u32x4_t{0u, 0u, 0u, 0u};
        kr[i][1] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ok[i]) {
        vr[i][0] = *reinterpret_cast<const u32x4_t*>(a.vpages + row_off[i] + dc * 8);
        vr[i][1] = *reinterpret_cast<const u32x4_t*>(a.vpages + row_off[i] + 64 + dc * 8);
      } else {
        vr[i][0] = u32x4_t{0u, 0u, 0u, 0u};
        vr[i][1] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }

    // ---- scores: lane-partial bf16 dot products, summed over the key's 8 lanes ----
    float s[ROWS][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float d = 0.f;
        d = dot2_bf16(q[r][0], kr[i][0].x, d);
        d = dot2_bf16(q[r][1], kr[i][0].y, d);
        d = dot2_bf16(q[r][2], kr[i][0].z, d);
        d = dot2_bf16(q[r][3], kr[i][0].w, d);
        d = dot2_bf16(q[r][4], kr[i][1].x, d);
        d = dot2_bf16(q[r][5], kr[i][1].y, d);
        d = dot2_bf16(q[r][6], kr[i][1].z, d);
        d = dot2_bf16(q[r][7], kr[i][1].w, d);
        s[r][i] = sum_lanes8(d) * a.c;
      }
    }
    // ---- visibility: past the split end, or hidden by the causal rule ----
    if (t0 + kTile > s1 || t0 + kTile - 1 > min_last) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = t0 + kg + 8 * i;
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
          if (!(key < s1 && key <= last[r])) s[r][i] = -INFINITY;
      }
    }
    // ---- online softmax with a wave-wide running maximum ----
    float p[ROWS][4];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float tmax = fmaxf(fmaxf(s[r][0], s[r][1]), fmaxf(s[r][2], s[r][3]));
      tmax = max_stride8(tmax);
      const float m_new = fmaxf(m[r], tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m[r] - m_use);
      m[r] = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[r][i] = fast_exp2(s[r][i] - m_use);
      lsum[r] = lsum[r] * alpha + ((p[r][0] + p[r][1]) + (p[r][2] + p[r][3]));
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[r][j] *= alpha;
    }
    // ---- weighted values ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[16];
      const uint32_t w[8] = {vr[i][0].x, vr[i][0].y, vr[i][0].z, vr[i][0].w,
                             vr[i][1].x, vr[i][1].y, vr[i][1].z, vr[i][1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[2 * j] = bf16_lo(w[j]);
        v[2 * j + 1] = bf16_hi(w[j]);
      }
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[r][j] = fmaf(p[r][i], v[j], acc[r][j]);
    }
  }

  // ---- merge: lanes of the wave (same maximum), then the 4 waves in LDS ----
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    lsum[r] = sum_stride8(lsum[r]);  // over the 8 key groups of the wave
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[r][j] = sum_stride8(acc[r][j]);
  }
  if (kg == 0) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lds_acc[wave][r][dc * 8 + j] = acc[r][j];
        lds_acc[wave][r][64 + dc * 8 + j] = acc[r][8 + j];
      }
    }
    if (dc == 0) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        lds_m[wave][r] = m[r];
        lds_l[wave][r] = lsum[r];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < a.rows * 128; idx += kThreads) {
    const int r = idx >> 7;
    const int d = idx & 127;
    float mw[kWaves];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = lds_m[w][r];
      M = fmaxf(M, mw[w]);
    }
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - M);
      den = fmaf(f, lds_l[w][r], den);
      num = fmaf(f, lds_acc[w][r][d], num);
    }
    const int h = kvh * a.group + r / a.query_len;
    const int l = r % a.query_len;
    const size_t orow = ((size_t)b * a.num_q_heads + h) * a.query_len + l;
    if (DIRECT) {
      a.out[orow * 128 + d] = to_bf16(num / den);
    } else {
      a.ws_acc[(orow * a.n_split + split) * 128 + d] = num;
      if (d == 0) {
        a.ws_ml[(orow * a.n_split + split) * 2 + 0] = M;
        a.ws_ml[(orow * a.n_split + split) * 2 + 1] = den;
      }
    }
  }
}

// Combines the per-split partial states of one output row ("Week 2 Day 5",
// Task 2: common maximum, one rescale factor per partial, one denominator,
// one thread per head dimension). Splits whose state is empty (maximum
// -inf) contribute nothing.
__global__ void __launch_bounds__(128) pa_decode_merge(DecodeArgs a) {
  const int orow = blockIdx.x;
  const int d = threadIdx.x;
  const int b = orow / (a.num_q_heads * a.query_len);
  const int ctx = a.context_lens[b];
  const int n = (ctx + a.split_len - 1) / a.split_len;
  const float* ml = a.ws_ml + (size_t)orow * a.n_split * 2;
  const float* acc = a.ws_acc + (size_t)orow * a.n_split * 128 + d;
  float M = -INFINITY;
  for (int j = 0; j < n; ++j) M = fmaxf(M, ml[2 * j]);
  float den = 0.f, num = 0.f;
  for (int j = 0; j < n; ++j) {
    const float mj = ml[2 * j];
    if (mj == -INFINITY) continue;
    const float f = fast_exp2(mj - M);
    den = fmaf(f, ml[2 * j + 1], den);
    num = fmaf(f, acc[(size_t)j * 128], num);
  }
  a.out[(size_t)orow * 128 + d] = to_bf16(num / den);
}

template <int ROWS, bool ALIGNED, bool DIRECT>
hipError_t launch_split(const DecodeArgs& a, int64_t grid, size_t lds_bytes, hipStream_t stream) {
  hipLaunchKernelGGL((pa_decode_split<ROWS, ALIGNED, DIRECT>), dim3((unsigned)grid), dim3(kThreads), lds_bytes,
                     stream, a);
  return hipGetLastError();
}

template <int ROWS>
hipError_t launch_rows(const DecodeArgs& a, bool aligned, bool direct, int64_t grid, size_t lds, hipStream_t st) {
  if (aligned) return direct ? launch_split<ROWS, true, true>(a, grid, lds, st) : launch_split<ROWS, true, false>(a, grid, lds, st);
  return direct ? launch_split<ROWS, false, true>(a, grid, lds, st) : launch_split<ROWS, false, false>(a, grid, lds, st);
}

}  // namespace

hipError_t launch_decode(const KernelArgs& k, const Plan& p, hipStream_t stream) {
  DecodeArgs a;
  a.query = static_cast<const uint16_t*>(k.query);
  a.kpages = static_cast<const uint16_t*>(k.key_pages);
  a.vpages = static_cast<const uint16_t*>(k.value_pages);
  a.block_table = k.block_table;
  a.context_lens = k.context_lens;
  a.out = static_cast<uint16_t*>(k.out);
  char* ws = static_cast<char*>(k.workspace);
  a.ws_acc = p.direct ? nullptr : reinterpret_cast<float*>(ws + p.ws_acc_offset);
  a.ws_ml = p.direct ? nullptr : reinterpret_cast<float*>(ws + p.ws_ml_offset);
  a.num_q_heads = k.num_q_heads;
  a.num_kv_heads = k.num_kv_heads;
  a.query_len = k.query_len;
  a.group = p.group;
  a.rows = p.rows;
  a.page_size = k.page_size;
  a.ps_log2 = p.ps_log2;
  a.max_pages = k.max_pages;
  a.split_len = p.split_len;
  a.n_split = p.n_split;
  a.c = k.scale * kLog2e;
  a.causal = k.causal;
  const size_t lds = (size_t)p.bt_entries * sizeof(int32_t);
  hipError_t e;
  switch (p.rows_pad) {
    case 1: e = launch_rows<1>(a, p.aligned, p.direct, p.num_work, lds, stream); break;
    case 2: e = launch_rows<2>(a, p.aligned, p.direct, p.num_work, lds, stream); break;
    case 4: e = launch_rows<4>(a, p.aligned, p.direct, p.num_work, lds, stream); break;
    default: e = launch_rows<8>(a, p.aligned, p.direct, p.num_work, lds, stream); break;
  }
  if (e != hipSuccess || p.direct) return e;
  const int64_t nrows = (int64_t)k.batch * k.num_q_heads * k.query_len;
  hipLaunchKernelGGL(pa_decode_merge, dim3((unsigned)nrows), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
