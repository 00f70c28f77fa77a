// pa_prefill.hip -- long-query (prefill) schedule of the paged attention
// operator for gfx950: tiled online softmax on bf16 matrix cores.
//
// What it computes ("Week 3 Day 5: Paged FlashAttention", Task 2): for each
// query tile keep one running maximum, running sum and unnormalised output
// row per query row; for each K/V tile: scores Q K^T, scale and causal
// bounds, merge the tile maximum, rescale the sum and output, exponentials
// and sum update, P V into the output; after the last visible tile divide by
// the sum and store bf16. scale * log2(e) is applied once and the
// exponentials are base 2. A K/V tile whose first key is past the last key
// visible to the query tile is never loaded (whole-tile causal skip).
//
// Schedule:
//   work item = (128-row query tile, query head, sequence), 4 waves; wave w
//   owns query rows [32w, 32w+32) of the tile. K/V tiles are 64 keys.
//   Matrix core: v_mfma_f32_32x32x16_bf16 (fp32 accumulate). Scores are
//   computed transposed, S^T = K Q^T (A = K rows from LDS, B = the wave's
//   Q^T held in registers for the whole loop), so lane l holds 16 scores of
//   ONE query row (l % 32): the row maximum needs a single cross-lane
//   exchange (lane l ^ 32), and the rescale factor of a row lives in the
//   lane that owns that row of the output.
//   Output O^T = V^T P^T (A = V^T from LDS, B = P^T straight from the score
//   registers converted to bf16): the 8 keys a lane feeds to one MFMA are
//   exactly the 8 scores it already holds, so P never goes through LDS.
//   V is stored transposed in LDS with the keys of every 16-key step
//   permuted (bits 2 and 3 of the key index swapped) so each lane's 8 keys
//   are one 16-byte LDS read.
//
// Page-translating loader ("Week 3 Day 5", Task 1): each K/V tile is
// resolved through block_table while it is staged: thread t loads head dims
// [8(t%16), 8(t%16)+8) of keys 4(t/16) .. 4(t/16)+3 (16 lanes cover a
// 256-byte row, so a wave reads 4 full rows per instruction). Aligned path
// (page_size % 64 == 0): the tile is one contiguous span of one page, found
// with a single table entry. Generic path: each key row is translated on
// its own (tiles that cross pages). Keys at or past the context end are not
// loaded (zero) and their scores are masked to -inf separately. The next
// tile is fetched into registers while the current one is computed.
//
// Work items are ordered so that the heaviest causal query tiles start
// first and the query heads that share one K/V head run back to back on
// the same XCD (shared L2).

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kBM = kPrefillBlockM;  // 128 query rows
constexpr int kBN = kPrefillBlockN;  // 64 keys
constexpr int kKStride = 128 + 8;    // bf16 per K row in LDS (16 B pad)
constexpr int kVStride = kBN + 8;    // bf16 per V^T row in LDS (16 B pad)
// The exponent reference of a row moves only when a tile maximum exceeds it
// by more than kTau (log2 units), so weights stay <= 2^kTau.
constexpr float kTau = 8.0f;

struct PrefillArgs {
  const uint16_t* query;
  const uint16_t* kpages;
  const uint16_t* vpages;
  const int32_t* block_table;
  const int32_t* context_lens;
  uint16_t* out;
  int batch, num_q_heads, num_kv_heads, query_len, group, n_qtiles;
  int page_size, ps_log2, max_pages;
  float c;  // scale * log2(e)
  int causal;
};

__device__ __forceinline__ int div_ps(int s, int ps, int ps_log2) { return ps_log2 >= 0 ? (s >> ps_log2) : s / ps; }

// Position of key k (0..63) inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <bool ALIGNED>
__device__ __forceinline__ void load_kv_tile(const PrefillArgs& a, int b, int kvh, int ctx, int t0, int tid,
                                             u32x4_t kreg[4], u32x4_t vreg[4]) {
  const int dchunk = tid & 15;
  const int g4 = tid >> 4;
  const size_t head_stride = (size_t)a.page_size * 128;
  const size_t page_stride = head_stride * a.num_kv_heads;
  const size_t head_off = (size_t)kvh * head_stride;
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  size_t base = 0;
  if (ALIGNED) {
    const int lp = div_ps(t0, a.page_size, a.ps_log2);
    const int slot0 = t0 - lp * a.page_size;
    base = (size_t)bt_row[lp] * page_stride + head_off + (size_t)slot0 * 128;
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int key = t0 + 4 * g4 + jj;
    if (key < ctx) {
      size_t off;
      if (ALIGNED) {
        off = base + (size_t)(4 * g4 + jj) * 128;
      } else {
        const int lp = div_ps(key, a.page_size, a.ps_log2);
        const int slot = key - lp * a.page_size;
        off = (size_t)bt_row[lp] * page_stride + head_off + (size_t)slot * 128;
      }
      kreg[jj] = *reinterpret_cast<const u32x4_t*>(a.kpages + off + dchunk * 8);
      vreg[jj] = *reinterpret_cast<const u32x4_t*>(a.vpages + off + dchunk * 8);
    } else {
      kreg[jj] = u32x4_t{0u, 0u, 0u, 0u};
      vreg[jj] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void store_kv_tile(uint16_t* lds_k, uint16_t* lds_vt, int tid, const u32x4_t kreg[4],
                                              const u32x4_t vreg[4]) {
  const int dchunk = tid & 15;
  const int g4 = tid >> 4;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
    *reinterpret_cast<u32x4_t*>(lds_k + (4 * g4 + jj) * kKStride + dchunk * 8) = kreg[jj];
  // V^T: dim 8*dchunk + e of keys 4*g4 .. 4*g4+3 -> 4 adjacent positions.
  const int pos = vt_pos(4 * g4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t w0 = vreg[0][e], w1 = vreg[1][e], w2 = vreg[2][e], w3 = vreg[3][e];
    // even dim 2e: low halves; odd dim 2e+1: high halves
    const u32x2_t even = {__builtin_amdgcn_perm(w1, w0, 0x05040100u), __builtin_amdgcn_perm(w3, w2, 0x05040100u)};
    const u32x2_t odd = {__builtin_amdgcn_perm(w1, w0, 0x07060302u), __builtin_amdgcn_perm(w3, w2, 0x07060302u)};
    *reinterpret_cast<u32x2_t*>(lds_vt + (dchunk * 8 + 2 * e) * kVStride + pos) = even;
    *reinterpret_cast<u32x2_t*>(lds_vt + (dchunk * 8 + 2 * e + 1) * kVStride + pos) = odd;
  }
}

template <bool ALIGNED>
__global__ void __launch_bounds__(kThreads, 2) pa_prefill_mfma(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[kBN * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t lds_vt[128 * kVStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;  // which 8-wide k slice of an MFMA operand this lane feeds
  const int col = lane & 31;   // query row (within the wave) owned by this lane

  // ---- work item: heavy query tiles first, GQA siblings together on one XCD ----
  const int n = gridDim.x;
  int logical = blockIdx.x;
  const int G = a.group;
  if (n % (8 * G) == 0) {
    const int xcd = blockIdx.x & 7;
    const int k = blockIdx.x >> 3;
    logical = ((k / G) * 8 + xcd) * G + (k % G);
  }
  const int g = logical % G;
  int task = logical / G;
  const int kvh = task % a.num_kv_heads;
  task /= a.num_kv_heads;
  const int b = task % a.batch;
  const int qtile = a.n_qtiles - 1 - task / a.batch;
  const int head = kvh * G + g;

  const int L = a.query_len;
  const int ctx = a.context_lens[b];
  const int offset = ctx - L;  // query row l sits at logical position l + offset
  const int q0 = qtile * kBM;
  const int tile_last_row = min(q0 + kBM, L) - 1;
  const int kv_end = a.causal ? min(ctx, tile_last_row + offset + 1) : ctx;
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  const int r0 = q0 + 32 * wave;  // first query row of this wave
  const bool wave_has_rows = r0 < L;
  const int wave_last_row = min(r0 + 31, L - 1);
  const int wave_kv_end = a.causal ? min(ctx, wave_last_row + offset + 1) : ctx;

  // ---- Q^T operand: lane holds row r0 + col, dims 16ks + 8half .. +8 ----
  bf16x8_t qv[8];
  {
    const int row = r0 + col;
    const uint16_t* qp = a.query + (((size_t)b * a.num_q_heads + head) * L + row) * 128 + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4_t w = u32x4_t{0u, 0u, 0u, 0u};
      if (row < L) w = *reinterpret_cast<const u32x4_t*>(qp + 16 * ks);
      qv[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  f32x16_t acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_o[db][i] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's half of the row sum

  u32x4_t kreg[4], vreg[4];
  if (n_tiles > 0) load_kv_tile<ALIGNED>(a, b, kvh, ctx, 0, tid, kreg, vreg);

  const int row_abs = r0 + col;
  for (int t = 0; t < n_tiles; ++t) {
    const int t0 = t * kBN;
    __syncthreads();  // every wave is done reading the previous tile
    store_kv_tile(lds_k, lds_vt, tid, kreg, vreg);
    __syncthreads();
    if (t + 1 < n_tiles) load_kv_tile<ALIGNED>(a, b, kvh, ctx, t0 + kBN, tid, kreg, vreg);
    if (!wave_has_rows || t0 >= wave_kv_end) continue;

    // ---- S^T = K Q^T : two 32-key blocks ----
    f32x16_t acc_s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_s[kb][i] = 0.f;
      const uint16_t* kp = lds_k + (32 * kb + col) * kKStride + 8 * half;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t kfrag = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(kp + 16 * ks));
        acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qv[ks], acc_s[kb], 0, 0, 0);
      }
    }

    // ---- mask, online softmax (row = this lane's query row) ----
    // element i of block kb is key 32kb + 8(i/4) + 4half + i%4 of the tile.
    // The maximum is taken on raw scores (c > 0); the scale is folded into
    // the exponent argument.
    const bool need_mask = (t0 + kBN > ctx) || (a.causal && t0 + kBN - 1 > r0 + offset);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          const bool vis = key < ctx && (!a.causal || key <= row_abs + offset);
          acc_s[kb][i] = vis ? acc_s[kb][i] : -INFINITY;
        }
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, acc_s[kb][i]);
    tmax = max_xor32(tmax) * a.c;  // log2 units
    // The exponent reference moves only when the tile maximum exceeds it by
    // more than kTau; otherwise the weights stay <= 2^kTau and the output
    // needs no rescale. The branch is taken when any row of the wave moves.
    const bool grow = tmax > m_run + kTau;
    if (__ballot(grow)) {
      const float alpha = grow ? fast_exp2(m_run - tmax) : 1.f;  // 0 while the old reference is -inf
      m_run = grow ? tmax : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
    }
    const float neg_ref = m_run == -INFINITY ? 0.f : -m_run;
    float psum = 0.f;
    uint32_t pk[2][8];  // P^T operand, packed bf16 pairs
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = fast_exp2(fmaf(acc_s[kb][i], a.c, neg_ref));
        const float p1 = fast_exp2(fmaf(acc_s[kb][i + 1], a.c, neg_ref));
        psum += p0 + p1;
        pk[kb][i >> 1] = pack_bf16x2(p0, p1);
      }
    }
    l_run += psum;

    // ---- O^T += V^T P^T : 4 blocks of 32 dims, 4 steps of 16 keys ----
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t* src = &pk[ks >> 1][(ks & 1) * 4];
      const u32x4_t pw = {src[0], src[1], src[2], src[3]};
      const bf16x8_t pfrag = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* vp = lds_vt + (32 * db + col) * kVStride + 16 * ks + 8 * half;
        const bf16x8_t vfrag = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(vp));
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag, pfrag, acc_o[db], 0, 0, 0);
      }
    }
  }

  // ---- finalize: divide by the row sum, store bf16 ----
  if (!wave_has_rows) return;
  const float l_tot = sum_xor32(l_run);
  if (row_abs >= L) return;
  const float inv = 1.f / l_tot;
  uint16_t* op = a.out + (((size_t)b * a.num_q_heads + head) * L + row_abs) * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int d0 = 32 * db + 8 * grp + 4 * half;
      const u32x2_t w = {pack_bf16x2(acc_o[db][4 * grp] * inv, acc_o[db][4 * grp + 1] * inv),
                         pack_bf16x2(acc_o[db][4 * grp + 2] * inv, acc_o[db][4 * grp + 3] * inv)};
      *reinterpret_cast<u32x2_t*>(op + d0) = w;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const KernelArgs& k, const Plan& p, hipStream_t stream) {
  PrefillArgs a;
  a.query = static_cast<const uint16_t*>(k.query);
  a.kpages = static_cast<const uint16_t*>(k.key_pages);
  a.vpages = static_cast<const uint16_t*>(k.value_pages);
  a.block_table = k.block_table;
  a.context_lens = k.context_lens;
  a.out = static_cast<uint16_t*>(k.out);
  a.batch = k.batch;
  a.num_q_heads = k.num_q_heads;
  a.num_kv_heads = k.num_kv_heads;
  a.query_len = k.query_len;
  a.group = p.group;
  a.n_qtiles = p.n_qtiles;
  a.page_size = k.page_size;
  a.ps_log2 = p.ps_log2;
  a.max_pages = k.max_pages;
  a.c = k.scale * kLog2e;
  a.causal = k.causal;
  if (p.aligned)
    hipLaunchKernelGGL(pa_prefill_mfma<true>, dim3((unsigned)p.num_work), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(pa_prefill_mfma<false>, dim3((unsigned)p.num_work), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
