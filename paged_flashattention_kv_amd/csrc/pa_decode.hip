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
// Work division (HBM-bound; no matrix cores): the decode work is the sum of
// the context lengths times the kv heads. It is cut into 64-key granules,
// laid out segment by segment (segment = one (sequence, kv head) pair, in
// sequence-major order), and the granule range is split over a fixed number
// of work items -- as many 256-thread work items as the GPU keeps resident
// at once -- by a cost model: every granule costs the same, a segment start
// (a new piece, with its fixed latency) costs a few granules more, and the
// second workgroup on each CU (served after the first) gets a smaller share,
// so every work item streams for about the same time whatever the mix of
// context lengths. The split is a deterministic function of the context
// lengths, so results are bit-reproducible. A work item walks its contiguous
// range piece by piece (a piece = the part of one segment inside the range).
// A piece that is a whole segment is normalised and stored directly; a
// piece of a segment shared with other work items (at most the first and
// the last piece of a range) leaves its (max, sum, acc) state in the
// workspace and counts itself in at the segment's counter; the work item
// that arrives last combines the segment's partials and stores the output.
// One kernel launch per call.
//
// Inside a piece: all query rows that read this kv head -- the GQA group
// times the query length, at most 8 rows -- are served by ONE pass over the
// piece's keys, so every K/V byte is read from HBM once per kv head. Waves
// interleave steps of 8 KB of K and V. Lane layout for head dim D (64, 128
// or 256): LPK = D/16 lanes per key row, lane = LPK * kg + dc; lane (kg, dc)
// holds key kg (and kg + 64/LPK) and head dims [8dc, 8dc+8) and
// [D/2+8dc, D/2+8dc+8): two 16-byte loads per key row. q.k: packed bf16 dot
// products (v_dot2_f32_bf16) summed over the key's LPK lanes with DPP. The exponent
// reference is shared by the whole wave, so wave partials combine without
// rescaling; the 4 waves merge in LDS through a common maximum. Register
// stages rotate so the next steps' K/V loads are in flight while a step is
// computed. Head dims other than 64, 128 and 256 (any multiple of 8 up to
// 256) run the next larger instance D: rows are dv elements long in memory,
// the query's dims past dv are zero, a lane's chunk past dv re-reads the
// row's first chunk (finite data, weighted by a zero query) and no output
// dim past dv is stored.
//
// Page translation ("Week 3 Day 5", Task 1): the block-table entries of a
// 2048-key window are staged in LDS. Aligned path (page_size a multiple of
// the wave step, 2048 / D keys): a step lies inside one page, found with one
// table entry. Generic path: every
// key row is translated on its own (steps that cross page boundaries, e.g.
// 16-token pages). Keys past the piece end are never loaded from their own
// (possibly missing) page; their scores are forced to -inf by a separate
// mask ("Day 22: the fused paged-attention kernel", "What I learned", 2).

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Keys each lane holds per step (a wave step covers 8 * kTK keys), and the
// number of register stages per wave: the K/V loads of the next
// kStages - 1 steps are issued before the current step is computed (one
// stage fewer in the 4-row instances, see decode_piece).
#ifndef PA_DECODE_TK
#define PA_DECODE_TK 2
#endif
constexpr int kTK = PA_DECODE_TK;
#ifndef PA_DECODE_STAGES
#define PA_DECODE_STAGES 3
#endif
constexpr int kStages = PA_DECODE_STAGES;
// Lane geometry for head dim D: D/16 lanes hold one key row (16 dims each,
// two 16-byte chunks), so one load instruction covers 64/(D/16) key rows and
// a wave step 8 KB of K and V whatever D is.
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128 || D == 256, "head dims 64, 128 and 256");
  static constexpr int LPK = D / 16;         // lanes per key row
  static constexpr int KPI = 64 / LPK;       // key rows per load instruction
  static constexpr int kStep = KPI * kTK;    // keys per wave step
};
// The exponent reference of a row moves only when a tile's maximum exceeds it
// by more than kTau (log2 units), so weights stay <= 2^kTau and the common
// case needs no rescale of the accumulators.
constexpr float kTau = 8.0f;
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // (1.0, 1.0) in bf16

constexpr int kGran = 64;    // keys per granule: work ranges start and end on granules
// The work split's cost model (see WorkSplit): a segment start costs 2
// granules, and the grid's second half gets 12/16 of the first half's share.
// Measured on the decode batch (per-workgroup timestamps): a piece costs 6-8
// us of fixed latency (about 3 granules of streaming) and the second
// workgroup on a CU streams ~18% slower; with the even split the last work
// items (five pieces, second half) ended 25-30 us after the median. A/B on one
// MI355X: decode batch 115.6 -> 107.8 us; long-context decode 333.5 -> 341.2
// us (its segments are long and uniform, so it gains nothing and pays the
// skew). With two register stages in the 4-row instances a start cost of 2
// granules replaced 4 where two work items share a CU (decode batch
// 105.8-106.2 -> 104.1-104.6 us, masked decode and mixed batch ~1% faster,
// long decode 0.6% slower, 1 and 2 rows unchanged; 1 granule: 111.9 us, 3:
// 105.4 us); the 8-row instance, one work item per CU, keeps 4 (2 measured
// 6% slower there).
template <int ROWS>
constexpr int split_piece_cost() { return ROWS <= 4 ? 2 : 4; }  // granules a segment start costs
constexpr int kSplitWa = 16;        // weight of the grid's first half
constexpr int kSplitWb = 12;        // weight of the grid's second half
constexpr int kWindow = 2048;  // keys per block-table staging window

struct DecodeArgs {
  const uint16_t* query;
  const uint16_t* kpages;
  const uint16_t* vpages;
  const int32_t* block_table;
  const int32_t* context_lens;
  uint16_t* out;
  uint64_t* ws_ctr;  // [batch * num_kv_heads] arrival counters of shared segments (epoch << 32 | count)
  float* ws_ml;      // [work_items][2][rows][2]   partial (reference max, sum)
  float* ws_acc;     // [work_items][2][rows][128] partial unnormalised outputs
  uint32_t epoch;    // differs from the previous call's and from 0
  // Packed mixed batch: query/out [total_query, H_q, 128], sequence b owns
  // tokens [qstart[b], qstart[b + 1]) and is served here when its length is
  // 1 .. query_len. nullptr: the uniform [B, H_q, query_len, 128] layout.
  const int32_t* qstart;
  int total_query;
  int dv;  // head dim of query, pages and out (<= D: dims past it are masked)
  int batch, num_q_heads, num_kv_heads, query_len, group, rows;
  int page_size, ps_log2, max_pages;
  int work_items;
  float c;         // |scale| * log2(e), > 0 (fold_scale)
  uint32_t qsign;  // XORed into every packed query pair: a negative scale negates q
  int causal;
  // Explicit additive mask (natural-log units) of row (b, h, l), key s at
  // mask[b*msb + h*msh + l*msl + s] for s < mask_len; keys at or past
  // mask_len are absent. Used by the MASKED instances only.
  const float* mask;
  int64_t msb, msh, msl;
  int mask_len;
};

__device__ __forceinline__ int div_ps(int s, int ps, int ps_log2) { return ps_log2 >= 0 ? (s >> ps_log2) : s / ps; }

struct Stage {
  u32x4_t k[kTK][2];
  u32x4_t v[kTK][2];
};

struct Pager {
  const uint16_t* kpages;
  const uint16_t* vpages;
  const int32_t* lds_bt;  // block-table entries of the split, from logical page lp0
  size_t page_stride, head_off;
  int lp0, s0, s1, page_size, ps_log2;
  int kg, dc;
  int dv;      // row length in elements
  int c0, c1;  // element offsets of the lane's two chunks in a row (a masked chunk re-reads chunk 0)
};

// Every K/V row is read once per launch. At head dims 128 and 256 the loads
// carry the streaming hint, so the rows pass through the caches without
// evicting lines still to be hit (block-table entries, query rows,
// partials): 8-11% faster than plain loads on pools larger than the
// last-level cache. At head dim 64 the hint measured 4% slower; plain loads.
template <int D>
__device__ __forceinline__ u32x4_t load_kv(const uint16_t* p) {
  if constexpr (D >= 128) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Page-translating load of one step: keys t0 + kg + KPI*i (i < kTK), dims
// [8dc, 8dc+8) and [D/2+8dc, D/2+8dc+8). Keys at or past the split end are
// redirected to the split's first key (always a valid row) so every load is
// unconditional; their scores are masked to -inf and their weight is 0.
template <bool ALIGNED, int D, bool GEN>
__device__ __forceinline__ void load_stage(const Pager& g, int t0, Stage& st) {
  constexpr int KPI = Geo<D>::KPI;
  const int dvr = GEN ? g.dv : D;  // row length in memory
  const int c0 = GEN ? g.c0 : g.dc * 8, c1 = GEN ? g.c1 : D / 2 + g.dc * 8;
  size_t row[kTK];
  if (ALIGNED) {
    // page_size % kStep == 0 and t0 % kStep == 0: the step lies inside one
    // page. A step wholly past the split end reads the split's first page.
    const int tb = t0 < g.s1 ? t0 : g.s0;
    const int lp = div_ps(tb, g.page_size, g.ps_log2);
    const size_t base = (size_t)g.lds_bt[lp - g.lp0] * g.page_stride + g.head_off +
                        (size_t)(tb - lp * g.page_size) * dvr;
#pragma unroll
    for (int i = 0; i < kTK; ++i) {
      const int key = t0 + g.kg + KPI * i;
      row[i] = key < g.s1 ? base + (size_t)(g.kg + KPI * i) * dvr : base;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kTK; ++i) {
      int key = t0 + g.kg + KPI * i;
      key = key < g.s1 ? key : g.s0;
      const int lp = div_ps(key, g.page_size, g.ps_log2);
      row[i] = (size_t)g.lds_bt[lp - g.lp0] * g.page_stride + g.head_off + (size_t)(key - lp * g.page_size) * dvr;
    }
  }
#pragma unroll
  for (int i = 0; i < kTK; ++i) {
    st.k[i][0] = load_kv<D>(g.kpages + row[i] + c0);
    st.k[i][1] = load_kv<D>(g.kpages + row[i] + c1);
  }
#pragma unroll
  for (int i = 0; i < kTK; ++i) {
    st.v[i][0] = load_kv<D>(g.vpages + row[i] + c0);
    st.v[i][1] = load_kv<D>(g.vpages + row[i] + c1);
  }
}

template <int ROWS>
struct RowState {
  float m[ROWS];     // exponent reference (wave-uniform), log2 units
  float lsum[ROWS];  // this lane's share of the row sum
  float acc[ROWS][16];
};

// The mask entries of one step for this lane's keys (t0 + kg + KPI*i) and
// every row, loaded with the step's K/V. The index is clamped into the mask
// row; entries of keys at or past mask_len are discarded in compute_stage.
template <int ROWS, int D>
__device__ __forceinline__ void load_mask(const float* const (&mrow)[ROWS], int mask_len, int t0, int kg,
                                          float (&mv)[ROWS][kTK]) {
  constexpr int KPI = Geo<D>::KPI;
#pragma unroll
  for (int i = 0; i < kTK; ++i) {
    const int key = min(t0 + kg + KPI * i, mask_len - 1);
#pragma unroll
    for (int r = 0; r < ROWS; ++r) mv[r][i] = mrow[r][key];
  }
}

template <int ROWS, int D, bool MASKED>
__device__ __forceinline__ void compute_stage(const Stage& st, const float (&mv)[MASKED ? ROWS : 1][kTK], int t0,
                                              int s1, int mask_len, const uint32_t (&q)[ROWS][8],
                                              const int (&last)[ROWS], int min_last, float c_in, int kg,
                                              RowState<ROWS>& rs) {
  constexpr int LPK = Geo<D>::LPK, KPI = Geo<D>::KPI, kStep = Geo<D>::kStep;
  // scores (raw q.k): lane-partial bf16 dot products, summed over the key's LPK lanes
  float s[ROWS][kTK];
#pragma unroll
  for (int i = 0; i < kTK; ++i) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float d = 0.f;
      d = dot2_bf16(q[r][0], st.k[i][0].x, d);
      d = dot2_bf16(q[r][1], st.k[i][0].y, d);
      d = dot2_bf16(q[r][2], st.k[i][0].z, d);
      d = dot2_bf16(q[r][3], st.k[i][0].w, d);
      d = dot2_bf16(q[r][4], st.k[i][1].x, d);
      d = dot2_bf16(q[r][5], st.k[i][1].y, d);
      d = dot2_bf16(q[r][6], st.k[i][1].z, d);
      d = dot2_bf16(q[r][7], st.k[i][1].w, d);
      s[r][i] = sum_lanes<LPK>(d);
    }
  }
  // With a mask the score becomes scale * q.k + mask in log2 units here, and
  // the softmax below takes it as is (c = 1); without one, the raw q.k and
  // c = scale * log2(e) folded into the exponent argument.
  float c = c_in;
  if constexpr (MASKED) {
#pragma unroll
    for (int i = 0; i < kTK; ++i) {
      const int key = t0 + kg + KPI * i;
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
        s[r][i] = key < mask_len ? fmaf(s[r][i], c_in, mv[r][i] * kLog2e) : -INFINITY;
    }
    c = 1.f;
  }
  // visibility: past the split end, or hidden by the causal rule (separate from the load)
  if (t0 + kStep > s1 || t0 + kStep - 1 > min_last) {
#pragma unroll
    for (int i = 0; i < kTK; ++i) {
      const int key = t0 + kg + KPI * i;
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
        if (!(key < s1 && key <= last[r])) s[r][i] = -INFINITY;
    }
  }
  // online softmax: the step maximum moves the reference only past the
  // threshold. The weights of keys (2i, 2i + 1) are packed as a bf16 pair:
  // P V below runs on packed bf16 dot products, and the row sum adds the same
  // rounded weights.
  static_assert(kTK % 2 == 0, "keys are paired for the packed weights");
  uint32_t pp[ROWS][kTK / 2];
  // the rows' step maxima first: independent reductions that overlap
  float tmaxes[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    float tmax = s[r][0];
#pragma unroll
    for (int i = 1; i < kTK; ++i) tmax = fmaxf(tmax, s[r][i]);
    tmaxes[r] = max_stride<LPK>(tmax) * c;
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const float tmax = tmaxes[r];
    if (tmax > rs.m[r] + kTau) {  // uniform across the wave
      const float alpha = fast_exp2(rs.m[r] - tmax);  // 0 when the old reference is -inf
      rs.m[r] = tmax;
      rs.lsum[r] *= alpha;
#pragma unroll
      for (int j = 0; j < 16; ++j) rs.acc[r][j] *= alpha;
    }
    const float mref = rs.m[r] == -INFINITY ? 0.f : rs.m[r];
#pragma unroll
    for (int i = 0; i < kTK / 2; ++i) {
      pp[r][i] = pack_bf16x2(fast_exp2(fmaf(s[r][2 * i], c, -mref)), fast_exp2(fmaf(s[r][2 * i + 1], c, -mref)));
      rs.lsum[r] = dot2_bf16(pp[r][i], kOnesBf16x2, rs.lsum[r]);
    }
  }
  // weighted values: for each pair of keys and each pair of dims, the two
  // keys' values of one dim are gathered into a bf16 pair (v_perm_b32) and
  // dotted with the pair of weights, accumulating in fp32
#pragma unroll
  for (int i = 0; i < kTK / 2; ++i) {
    const uint32_t w0[8] = {st.v[2 * i][0].x, st.v[2 * i][0].y, st.v[2 * i][0].z, st.v[2 * i][0].w,
                            st.v[2 * i][1].x, st.v[2 * i][1].y, st.v[2 * i][1].z, st.v[2 * i][1].w};
    const uint32_t w1[8] = {st.v[2 * i + 1][0].x, st.v[2 * i + 1][0].y, st.v[2 * i + 1][0].z, st.v[2 * i + 1][0].w,
                            st.v[2 * i + 1][1].x, st.v[2 * i + 1][1].y, st.v[2 * i + 1][1].z, st.v[2 * i + 1][1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = __builtin_amdgcn_perm(w1[j], w0[j], 0x05040100u);  // dim 2j of both keys
      const uint32_t hi = __builtin_amdgcn_perm(w1[j], w0[j], 0x07060302u);  // dim 2j + 1 of both keys
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        rs.acc[r][2 * j] = dot2_bf16(pp[r][i], lo, rs.acc[r][2 * j]);
        rs.acc[r][2 * j + 1] = dot2_bf16(pp[r][i], hi, rs.acc[r][2 * j + 1]);
      }
    }
  }
}

__device__ __forceinline__ int64_t n_gran(int ctx) { return ctx > 0 ? (ctx + kGran - 1) / kGran : 0; }

// Query rows of sequence b that this launch serves (0: none), and for a
// packed batch the token of its first row. A packed sequence whose offsets
// fall outside [0, total_query] or whose length is not 1 .. query_len is
// not served (no row of it is read or written).
__device__ __forceinline__ int seq_rows(const DecodeArgs& a, int b, int& start) {
  start = 0;
  if (a.qstart == nullptr) return a.query_len;
  const int s0 = a.qstart[b], s1 = a.qstart[b + 1];
  if (s0 < 0 || s1 > a.total_query || s1 <= s0 || s1 - s0 > a.query_len) return 0;
  start = s0;
  return s1 - s0;
}

// Granules of sequence b's K/V per kv head that this launch streams.
__device__ __forceinline__ int64_t seq_gran(const DecodeArgs& a, int b) {
  int start;
  return seq_rows(a, b, start) > 0 ? n_gran(a.context_lens[b]) : 0;
}

// Row index of query (and output) row l of head h of sequence b, which has
// L rows starting at token `start` (rows are head_dim elements long).
__device__ __forceinline__ size_t row_idx(const DecodeArgs& a, int b, int start, int L, int h, int l) {
  return a.qstart ? (size_t)(start + l) * a.num_q_heads + h : ((size_t)b * a.num_q_heads + h) * L + l;
}

// A value every lane of the wave holds, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---- the split of the work over the grid ----
//
// The work is laid out in granules, segment by segment (segment = one
// (sequence, kv head), sequence-major), and split over the work items by
// cost: a granule costs 1, and the start of a segment costs `c` more -- the
// fixed latency of a piece (query rows, block-table window, pipeline fill,
// partial store and arrival), so a work item whose range crosses many segment
// boundaries gets fewer granules. The second half of the grid -- with two
// resident workgroups per CU, the second one on each CU, whose waves the SIMD
// serves after the first's -- gets weight wb against wa for the first half.
// Granule g belongs to the work item whose cost range holds g's last cost
// unit; every work item computes the same split from the same prefix, so the
// pieces, partial slots and merges are the same on every run.
struct WorkSplit {
  int64_t T;     // granules
  int64_t C;     // cost units: T + c * segments
  int32_t P, H;  // work items; size of the first half (H = P: one weight for all)
  int32_t Wt;    // kSplitWa * H + kSplitWb * (P - H)
  int32_t c;     // cost of a segment start (0: an even split of granules)
};

// floor(num / den) for 0 <= num, 0 < den: a double-precision estimate
// corrected with integer products (a 64-bit integer division is a long
// emulated sequence; the estimate is exact or one off for num < 2^53).
__device__ __forceinline__ int64_t div_floor(int64_t num, int64_t den) {
  int64_t q = (int64_t)((double)num / (double)den);
  while (q > 0 && q * den > num) --q;
  while ((q + 1) * den <= num) ++q;
  return q;
}

// Weight of the work items before w.
__device__ __forceinline__ int64_t weight_before(const WorkSplit& s, int64_t w) {
  return (int64_t)kSplitWa * min(w, (int64_t)s.H) + (int64_t)kSplitWb * max(w - s.H, (int64_t)0);
}

// First cost unit of work item w: floor(C * weight_before(w) / Wt).
__device__ __forceinline__ int64_t cost_begin(const WorkSplit& s, int64_t w) {
  return w >= s.P ? s.C : div_floor(s.C * weight_before(s, w), s.Wt);
}

// The work item whose cost range holds cost unit x (0 <= x < C): the largest
// w with cost_begin(w) <= x, i.e. with weight_before(w) <= K =
// floor(((x + 1) * Wt - 1) / C).
__device__ __forceinline__ int64_t item_of_cost(const WorkSplit& s, int64_t x) {
  const int64_t K = div_floor((x + 1) * s.Wt - 1, s.C);
  const int64_t ha = (int64_t)kSplitWa * s.H;
  const int64_t w = K < ha ? K / kSplitWa : s.H + (K - ha) / kSplitWb;
  return min(w, (int64_t)s.P - 1);
}

// Granule that cost unit x of sequence b maps to (0 <= x - cp < the
// sequence's cost): the first granule whose last cost unit is at or past x.
// gp = granules per kv head before b, cp = cost units before b, ng = b's
// granules per kv head. Work item w holds the granules from the one that
// cost_begin(w) maps to up to the one that cost_begin(w + 1) maps to.
__device__ __forceinline__ int64_t granule_of(const WorkSplit& s, int64_t x, int64_t gp, int64_t cp, int64_t ng,
                                              int64_t hk) {
  const int64_t seg = ng + s.c, rel = x - cp;  // rel < hk * seg
  int64_t kvh;
  if (rel < ((int64_t)1 << 32) && seg < ((int64_t)1 << 32))
    kvh = (int64_t)((uint32_t)rel / (uint32_t)seg);
  else
    kvh = rel / seg;
  const int64_t off = rel - kvh * seg;
  return gp * hk + kvh * ng + max(off - s.c, (int64_t)0);
}

// The split for this launch: the cost terms only when every work item still
// gets at least one granule (each range longer than a segment start's cost),
// else the even split of granules.
template <int ROWS>
__device__ __forceinline__ WorkSplit make_split(const DecodeArgs& a, int64_t gran_per_head, int64_t nonempty) {
  WorkSplit s;
  s.T = gran_per_head * a.num_kv_heads;
  s.P = a.work_items;
  s.H = s.P / 2;
  s.c = split_piece_cost<ROWS>();
  s.C = s.T + (int64_t)s.c * nonempty * a.num_kv_heads;
  s.Wt = kSplitWa * s.H + kSplitWb * (s.P - s.H);
  const bool ok = s.T >= s.P && s.P >= 2 && s.C * min(kSplitWa, kSplitWb) >= (int64_t)(s.c + 2) * s.Wt;
  if (!ok) {  // the even split: one weight, no cost terms
    s.c = 0;
    s.C = s.T;
    s.H = s.P;
    s.Wt = kSplitWa * s.P;
  }
  return s;
}

// The work items holding pieces of segment [S, E) (granules; its first cost
// unit is CS) and the number of non-empty ones. With at least as many
// granules as work items every work item holds one or more granules; with
// fewer (even split), every non-empty work item holds exactly one, so the
// segment's E - S granules sit in E - S work items.
struct SegmentItems {
  int64_t wf, wl;
  uint32_t count;
};

__device__ __forceinline__ SegmentItems segment_items(const WorkSplit& s, int64_t S, int64_t E, int64_t CS) {
  SegmentItems it;
  it.wf = item_of_cost(s, CS + s.c);              // work item holding granule S
  it.wl = item_of_cost(s, CS + s.c + (E - S) - 1);  // work item holding granule E - 1
  it.count = (uint32_t)(s.T >= s.P ? it.wl - it.wf + 1 : E - S);
  return it;
}

// One piece: keys [k0, k1) of segment (b, kvh), for the group * L query
// rows of that kv head (sequence b has L rows from token `start`). Merges
// the 4 waves' states and either stores the output (the piece is the whole
// segment) or leaves the partial state in the workspace slot.
template <int ROWS, bool ALIGNED, int D, bool MASKED, bool GEN>
__device__ __forceinline__ void decode_piece(const DecodeArgs& a, int32_t* lds_bt, float (*lds_m)[ROWS],
                                             float (*lds_l)[ROWS], float (*lds_acc)[ROWS][D], int b, int kvh,
                                             int ctx, int L, int start, int k0, int k1, bool direct, int slot) {
  constexpr int LPK = Geo<D>::LPK, kStep = Geo<D>::kStep;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane / LPK;
  const int dc = lane % LPK;

  // Query rows of this kv head: row r -> q head kvh*group + r / L, position r % L.
  const int rows = a.group * L;
  uint32_t q[ROWS][8];
  int last[ROWS];
  const float* mrow[ROWS];  // mask row of each query row (MASKED only)
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    mrow[r] = a.mask;
    if (r < rows) {
      const int h = kvh * a.group + r / L;
      const int l = r % L;
      if (MASKED) mrow[r] = a.mask + (size_t)b * a.msb + (size_t)h * a.msh + (size_t)l * a.msl;
      // dims past dv are zero in the query, so their (re-read) keys add nothing
      const uint16_t* qp = a.query + row_idx(a, b, start, L, h, l) * (GEN ? a.dv : D);
      u32x4_t lo = u32x4_t{0u, 0u, 0u, 0u}, hi = lo;
      const bool use_lo = !GEN || dc * 8 < a.dv, use_hi = !GEN || D / 2 + dc * 8 < a.dv;
      const uint32_t sl = use_lo ? a.qsign : 0u, sh = use_hi ? a.qsign : 0u;
      if (use_lo) lo = *reinterpret_cast<const u32x4_t*>(qp + dc * 8);
      if (use_hi) hi = *reinterpret_cast<const u32x4_t*>(qp + D / 2 + dc * 8);
      q[r][0] = lo.x ^ sl; q[r][1] = lo.y ^ sl; q[r][2] = lo.z ^ sl; q[r][3] = lo.w ^ sl;
      q[r][4] = hi.x ^ sh; q[r][5] = hi.y ^ sh; q[r][6] = hi.z ^ sh; q[r][7] = hi.w ^ sh;
      last[r] = a.causal ? l + ctx - L : ctx - 1;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) q[r][j] = 0u;
      last[r] = ctx - 1;
    }
  }
  int min_last = ctx - 1;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) min_last = min(min_last, last[r]);

  RowState<ROWS> rs;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    rs.m[r] = -INFINITY;
    rs.lsum[r] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) rs.acc[r][j] = 0.f;
  }

  Pager g;
  g.kpages = a.kpages;
  g.vpages = a.vpages;
  g.lds_bt = lds_bt;
  g.page_stride = (size_t)a.page_size * (GEN ? a.dv : D) * a.num_kv_heads;
  g.head_off = (size_t)kvh * a.page_size * (GEN ? a.dv : D);
  g.dv = a.dv;
  g.c0 = dc * 8 < a.dv ? dc * 8 : 0;
  g.c1 = D / 2 + dc * 8 < a.dv ? D / 2 + dc * 8 : 0;
  g.page_size = a.page_size;
  g.ps_log2 = a.ps_log2;
  g.kg = kg;
  g.dc = dc;
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;

  for (int ka = k0; ka < k1; ka += kWindow) {
    const int kb = min(ka + kWindow, k1);
    // stage the window's block-table entries
    const int lp0 = div_ps(ka, a.page_size, a.ps_log2);
    const int nbt = div_ps(kb - 1, a.page_size, a.ps_log2) - lp0 + 1;
    __syncthreads();  // the previous window (or piece) is done with lds_bt
    for (int i = tid; i < nbt; i += kThreads) lds_bt[i] = bt_row[lp0 + i];
    __syncthreads();
    g.lp0 = lp0;
    g.s0 = ka;
    g.s1 = kb;

    // Each wave walks steps ka + wave*kStep, + kWaves*kStep, ...; kStages
    // register stages rotate so kStages - 1 steps of loads are in flight
    // while the oldest landed step is computed. Every stage load is issued
    // unconditionally (steps past the window re-read its first row), which
    // keeps the number of outstanding loads the same on every path, so the
    // waits before each step cover only that step's own loads.
    constexpr int kStride = kWaves * kStep;
    // register stages: the 4-row instances hold one fewer, which keeps the
    // masked one within the two-wave register budget (two work items per CU)
    // and measured faster for both (decode batch 107.6 -> 106.0 us, long
    // decode 342 -> 336 us, masked decode batch 127 -> 109 us); with 1 and 2
    // rows three stages measured 1-3% faster
    constexpr int kSt = ROWS == 4 ? kStages - 1 : kStages;
    int t = ka + wave * kStep;
    if (t < kb) {
      Stage st[kSt];
      float mv[kSt][MASKED ? ROWS : 1][kTK];  // mask entries riding with each stage
#pragma unroll
      for (int i = 0; i < kSt - 1; ++i) {
        load_stage<ALIGNED, D, GEN>(g, t + i * kStride, st[i]);
        if constexpr (MASKED) load_mask<ROWS, D>(mrow, a.mask_len, t + i * kStride, kg, mv[i]);
      }
      bool done = false;
      while (!done) {
#pragma unroll
        for (int j = 0; j < kSt; ++j) {
          load_stage<ALIGNED, D, GEN>(g, t + (kSt - 1) * kStride, st[(j + kSt - 1) % kSt]);
          if constexpr (MASKED)
            load_mask<ROWS, D>(mrow, a.mask_len, t + (kSt - 1) * kStride, kg, mv[(j + kSt - 1) % kSt]);
          compute_stage<ROWS, D, MASKED>(st[j], mv[j], t, kb, a.mask_len, q, last, min_last, a.c, kg, rs);
          t += kStride;
          if (t >= kb) {
            done = true;
            break;
          }
        }
      }
    }
  }

  // ---- merge: lanes of the wave (same reference), then the 4 waves in LDS ----
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    rs.lsum[r] = sum_stride<LPK>(rs.lsum[r]);  // over the key groups of the wave
#pragma unroll
    for (int j = 0; j < 16; ++j) rs.acc[r][j] = sum_stride<LPK>(rs.acc[r][j]);
  }
  if (kg == 0) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lds_acc[wave][r][dc * 8 + j] = rs.acc[r][j];
        lds_acc[wave][r][D / 2 + dc * 8 + j] = rs.acc[r][8 + j];
      }
    }
    if (dc == 0) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        lds_m[wave][r] = rs.m[r];
        lds_l[wave][r] = rs.lsum[r];
      }
    }
  }
  __syncthreads();
  const size_t part = ((size_t)blockIdx.x * 2 + slot) * a.rows;
  for (int idx = tid; idx < rows * D; idx += kThreads) {
    const int r = idx / D;
    const int d = idx % D;
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
    if (direct) {
      const int h = kvh * a.group + r / L;
      const int l = r % L;
      if (!GEN || d < a.dv) a.out[row_idx(a, b, start, L, h, l) * (GEN ? a.dv : D) + d] = to_bf16(num / den);
    } else {
      // device-coherent stores (no cache-wide fence needed; see arrive_last)
      store_coherent(a.ws_acc + (part + r) * D + d, num);
      if (d == 0) {
        store_coherent(a.ws_ml + (part + r) * 2 + 0, M);
        store_coherent(a.ws_ml + (part + r) * 2 + 1, den);
      }
    }
  }
}

// Combines the partial states of one shared segment ("Week 2 Day 5", Task 2:
// common maximum, one rescale factor per partial, one denominator, the head
// dimensions in parallel). Work item w's piece sits in slot 0 when the
// segment is the first piece of w's range, else in slot 1. The slot index of
// every work item of the segment (-1 for an empty one) is listed in LDS, up
// to kThreads at a time; each thread then folds kMergeBatch partials per
// round, with all of their loads issued before the first is used. Partials
// with maximum -inf (no visible key) contribute 0.
constexpr int kMergeBatch = 8;

template <int D, bool GEN>
__device__ void merge_segment(const DecodeArgs& a, int32_t* lds_parts, int b, int kvh, int L, int start, int64_t CS,
                              const SegmentItems& it, const WorkSplit& sp) {
  const int n_rd = a.group * L * D;
  const int64_t n_w = it.wl - it.wf + 1;
  const int tid = threadIdx.x;
  for (int base = 0; base < n_rd; base += kThreads) {  // uniform trip count (barriers inside)
    const int idx = base + tid;
    const int r = idx < n_rd ? idx / D : 0;
    const int d = idx % D;
    float M = -INFINITY, den = 0.f, num = 0.f;
    for (int64_t c0 = 0; c0 < n_w; c0 += kThreads) {
      const int nc = (int)min((int64_t)kThreads, n_w - c0);
      __syncthreads();  // the previous list is no longer read
      if (tid < nc) {
        // The segment is w's first piece (slot 0) when w's cost range starts at
        // or after the segment's first cost unit CS, else w's last piece (slot 1).
        // With c = 0 a cost unit is a granule and a range may be empty; with
        // c > 0 every range holds a granule.
        const int64_t w = it.wf + c0 + tid;
        const int64_t xw = cost_begin(sp, w);
        const bool empty = sp.c == 0 && xw == cost_begin(sp, w + 1);
        lds_parts[tid] = empty ? -1 : (int)(w * 2 + (xw >= CS ? 0 : 1));
      }
      __syncthreads();
      for (int j0 = 0; j0 < nc; j0 += kMergeBatch) {
        float mj[kMergeBatch], lj[kMergeBatch], aj[kMergeBatch];
        bool ok[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const int pi = lds_parts[min(j0 + u, nc - 1)];
          ok[u] = j0 + u < nc && pi >= 0;
          const size_t part = (size_t)(pi > 0 ? pi : 0) * a.rows + r;  // slot 0 of item 0: a valid address
          mj[u] = load_coherent(a.ws_ml + part * 2);
          lj[u] = load_coherent(a.ws_ml + part * 2 + 1);
          aj[u] = load_coherent(a.ws_acc + part * D + d);
        }
        float Mb = M;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          mj[u] = ok[u] ? mj[u] : -INFINITY;
          Mb = fmaxf(Mb, mj[u]);
        }
        if (Mb > -INFINITY) {
          const float fo = M == -INFINITY ? 0.f : fast_exp2(M - Mb);
          den *= fo;
          num *= fo;
#pragma unroll
          for (int u = 0; u < kMergeBatch; ++u) {
            const float f = mj[u] == -INFINITY ? 0.f : fast_exp2(mj[u] - Mb);
            den = fmaf(f, ok[u] ? lj[u] : 0.f, den);
            num = fmaf(f, ok[u] ? aj[u] : 0.f, num);
          }
          M = Mb;
        }
      }
    }
    if (idx < n_rd && (!GEN || d < a.dv)) {
      const int h = kvh * a.group + r / L;
      const int l = r % L;
      a.out[row_idx(a, b, start, L, h, l) * (GEN ? a.dv : D) + d] = to_bf16(num / den);
    }
  }
}

// Two resident workgroups per CU (a register budget of 256 per lane) for the
// instances that fit it; the 8-row ones take one.
template <int ROWS, bool ALIGNED, int D, bool MASKED, bool GEN>
__global__ void __launch_bounds__(kThreads, ROWS <= 4 ? 2 : 1) pa_decode_work(DecodeArgs a) {
  extern __shared__ int32_t lds_bt[];
  __shared__ float lds_m[kWaves][ROWS];
  __shared__ float lds_l[kWaves][ROWS];
  __shared__ float lds_acc[kWaves][ROWS][D];
  // granules per kv head (low 40 bits) and non-empty sequences (high 24 bits),
  // inclusive over thread chunks
  __shared__ int64_t lds_scan[kThreads];
  __shared__ int64_t lds_start[5];  // sequence holding this item's first cost unit, its prefixes, G0, G1
  __shared__ int32_t lds_parts[kThreads];  // partial slots of the segment being merged
  __shared__ bool lds_last;
  constexpr int kZShift = 40;
  const int64_t kGMask = ((int64_t)1 << kZShift) - 1;

  const int tid = threadIdx.x;
  // ---- granule prefix over sequences: thread t sums a contiguous chunk ----
  const int chunk = (a.batch + kThreads - 1) / kThreads;
  const int c0 = min(a.batch, tid * chunk), c1 = min(a.batch, c0 + chunk);
  int64_t mine = 0;
  for (int b = c0; b < c1; ++b) {
    const int64_t ng = seq_gran(a, b);
    mine += ng + (ng > 0 ? (int64_t)1 << kZShift : 0);
  }
  lds_scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {  // inclusive scan
    const int64_t v = tid >= off ? lds_scan[tid - off] : 0;
    __syncthreads();
    lds_scan[tid] += v;
    __syncthreads();
  }
  // every lane computes the same split: scalar registers
  const int64_t all = uniform64(lds_scan[kThreads - 1]);
  const WorkSplit sp = make_split<ROWS>(a, all & kGMask, all >> kZShift);
  const int64_t hk = a.num_kv_heads;
  const int64_t w = blockIdx.x;
  const int64_t x0 = cost_begin(sp, w), x1 = cost_begin(sp, w + 1);
  {
    // which sequences hold cost units x0 (this item's first) and x1 (the next
    // item's first): each thread checks its own chunk of sequences
    const int64_t ex = lds_scan[tid] - mine;
    int64_t gp = ex & kGMask, cp = hk * (gp + sp.c * (ex >> kZShift));
    for (int b = c0; b < c1; ++b) {
      const int64_t ng = seq_gran(a, b);
      const int64_t cb = ng > 0 ? hk * (ng + sp.c) : 0;
      if (x0 >= cp && x0 < cp + cb) {
        lds_start[0] = b;
        lds_start[1] = gp;
        lds_start[2] = cp;
        lds_start[3] = granule_of(sp, x0, gp, cp, ng, hk);
      }
      if (x1 >= cp && x1 < cp + cb) lds_start[4] = granule_of(sp, x1, gp, cp, ng, hk);
      gp += ng;
      cp += cb;
    }
  }
  __syncthreads();
  // a cost unit past the end (no work in this launch, or the last item's end) maps to T
  const int64_t G0 = x0 >= sp.C ? sp.T : uniform64(lds_start[3]);
  const int64_t G1 = x1 >= sp.C ? sp.T : uniform64(lds_start[4]);
  if (G0 >= G1) return;  // no work for this item (uniform)

  int b = (int)uniform64(lds_start[0]);
  int64_t pref = uniform64(lds_start[1]);   // granules per kv head before sequence b
  int64_t cpref = uniform64(lds_start[2]);  // cost units before sequence b
  int64_t G = G0;
  int nth = 0;
  while (G < G1) {
    const int ctx = a.context_lens[b];
    int start;
    const int L = seq_rows(a, b, start);
    const int64_t ng = L > 0 ? n_gran(ctx) : 0;
    if (ng == 0) {  // nothing of sequence b in the granule order
      ++b;
      continue;
    }
    const int64_t base = pref * a.num_kv_heads;  // first granule of sequence b
    const int kvh = (int)((G - base) / ng);
    const int64_t S = base + kvh * ng, E = S + ng;
    const int64_t gend = G1 < E ? G1 : E;
    const int k0 = (int)((G - S) * kGran);
    const int k1 = (int)min((gend - S) * kGran, (int64_t)ctx);
    const bool direct = G == S && gend == E;
    decode_piece<ROWS, ALIGNED, D, MASKED, GEN>(a, lds_bt, lds_m, lds_l, lds_acc, b, kvh, ctx, L, start, k0, k1, direct,
                                   nth == 0 ? 0 : 1);
    if (!direct) {
      // publish this piece, then the last of the segment's work items merges it
      // (CS: the segment's first cost unit)
      const int64_t CS = cpref + kvh * (ng + (int64_t)sp.c);
      const SegmentItems it = segment_items(sp, S, E, CS);
      wait_stores();
      __syncthreads();
      if (tid == 0) lds_last = arrive_last(a.ws_ctr + (size_t)b * a.num_kv_heads + kvh, a.epoch, it.count);
      __syncthreads();
      if (lds_last) merge_segment<D, GEN>(a, lds_parts, b, kvh, L, start, CS, it, sp);
    }
    G = gend;
    ++nth;
    if (G == base + (int64_t)a.num_kv_heads * ng) {  // past the last kv head of sequence b
      ++b;
      pref += ng;
      cpref += (int64_t)a.num_kv_heads * (ng + (int64_t)sp.c);
    }
  }
}

template <int ROWS, bool ALIGNED, int D, bool MASKED, bool GEN>
hipError_t launch_work(const DecodeArgs& a, size_t lds_bytes, hipStream_t stream) {
  hipLaunchKernelGGL((pa_decode_work<ROWS, ALIGNED, D, MASKED, GEN>), dim3((unsigned)a.work_items), dim3(kThreads), lds_bytes,
                     stream, a);
  return hipGetLastError();
}

// Work items the GPU keeps resident for one kernel instance (cached per
// device; registers, not shared memory, bound it for every page size).
template <int ROWS, bool ALIGNED, int D, bool MASKED, bool GEN>
int resident_items(size_t lds_bytes) {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] > 0) return cache[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)pa_decode_work<ROWS, ALIGNED, D, MASKED, GEN>, kThreads,
                                                   lds_bytes) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  const int n = cus * per_cu;
  cache[dev] = n;
  return n;
}

template <int ROWS, int D, bool MASKED>
hipError_t launch_rows(DecodeArgs& a, bool aligned, int requested, int cap, size_t lds, hipStream_t st) {
  if (a.dv != D) {
    // a head dim without an instance of its own: the next larger one, masked
    // dims, the per-row loader
    a.work_items = requested > 0 ? requested : min(cap, resident_items<ROWS, false, D, MASKED, true>(lds));
    return launch_work<ROWS, false, D, MASKED, true>(a, lds, st);
  }
  if (aligned) {
    a.work_items = requested > 0 ? requested : min(cap, resident_items<ROWS, true, D, MASKED, false>(lds));
    return launch_work<ROWS, true, D, MASKED, false>(a, lds, st);
  }
  a.work_items = requested > 0 ? requested : min(cap, resident_items<ROWS, false, D, MASKED, false>(lds));
  return launch_work<ROWS, false, D, MASKED, false>(a, lds, st);
}

template <int D, bool MASKED>
hipError_t launch_mask(DecodeArgs& a, const Plan& p, size_t lds, hipStream_t stream) {
  switch (p.rows_pad) {
    case 1: return launch_rows<1, D, MASKED>(a, p.aligned, p.work_items, p.work_cap, lds, stream);
    case 2: return launch_rows<2, D, MASKED>(a, p.aligned, p.work_items, p.work_cap, lds, stream);
    case 4: return launch_rows<4, D, MASKED>(a, p.aligned, p.work_items, p.work_cap, lds, stream);
    default: return launch_rows<8, D, MASKED>(a, p.aligned, p.work_items, p.work_cap, lds, stream);
  }
}

template <int D>
hipError_t launch_dim(DecodeArgs& a, const Plan& p, size_t lds, hipStream_t stream) {
  return a.mask ? launch_mask<D, true>(a, p, lds, stream) : launch_mask<D, false>(a, p, lds, stream);
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
  a.ws_ctr = reinterpret_cast<uint64_t*>(ws + p.ws_ctr_offset);
  a.ws_ml = reinterpret_cast<float*>(ws + p.ws_ml_offset);
  a.ws_acc = reinterpret_cast<float*>(ws + p.ws_acc_offset);
  a.batch = k.batch;
  a.num_q_heads = k.num_q_heads;
  a.num_kv_heads = k.num_kv_heads;
  a.query_len = k.query_len;
  a.group = p.group;
  a.rows = p.rows;
  a.page_size = k.page_size;
  a.ps_log2 = p.ps_log2;
  a.max_pages = k.max_pages;
  const ScaleFold sf = fold_scale(k.scale);
  a.c = sf.c;
  a.qsign = sf.qsign;
  a.causal = k.causal;
  a.epoch = k.epoch;
  a.qstart = k.query_start;
  a.total_query = k.total_query;
  a.dv = k.head_dim;
  a.mask = k.mask;
  a.msb = k.mask_stride_b;
  a.msh = k.mask_stride_h;
  a.msl = k.mask_stride_l;
  a.mask_len = k.mask_len;
  if (k.query_start) a.query_len = k.dec_max_len;  // the longest query this launch serves
  const size_t lds = (size_t)p.bt_entries * sizeof(int32_t);
  switch (instance_dim(k.head_dim)) {
    case 64: return launch_dim<64>(a, p, lds, stream);
    case 256: return launch_dim<256>(a, p, lds, stream);
    default: return launch_dim<128>(a, p, lds, stream);
  }
}

}  // namespace pa
