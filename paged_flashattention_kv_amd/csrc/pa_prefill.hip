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
//   work item = (128-row tile, kv head, sequence), 4 waves; wave w owns rows
//   [32w, 32w+32) of the tile. The rows are (position, query head) pairs of
//   the G query heads that read the kv head, position-major (row r:
//   position r / G of head kvh * G + r % G), so each K/V tile serves the
//   whole group and a short query still fills the waves. K/V tiles are 64
//   keys. A launch with few work items splits the key ranges into parts
//   sized from its own context lengths (up to eight per work item, all of
//   them resident at once), merged by the part that arrives last.
//   Matrix core: v_mfma_f32_32x32x16_bf16 (fp32 accumulate). Scores are
//   computed transposed, S^T = K Q^T (A = K rows from LDS, B = the wave's
//   Q^T held in registers for the whole loop), so lane l holds 16 scores of
//   ONE query row (l % 32): the row maximum needs a single cross-lane
//   exchange (lane l ^ 32), and the rescale factor of a row lives in the
//   lane that owns that row of the output.
//   Output O^T = V^T P^T (A = V^T, B = P^T straight from the score
//   registers converted to bf16): the 8 keys a lane feeds to one MFMA are
//   exactly the 8 scores it already holds, so P never goes through LDS.
//   V stays in its natural [key][dim] layout in LDS; the transposed operand
//   comes from ds_read_b64_tr_b16, which hands lane i of each 16-lane group
//   element (i mod 4) of the 8 bytes addressed by lane 4j + i/4 as its
//   element j.
//
// Page-translating loader ("Week 3 Day 5", Task 1): each K/V tile is
// resolved through block_table while it is staged, straight from HBM into
// LDS by LDS DMA (global_load_lds_dwordx4, or buffer_load_dwordx4 ... lds for
// a whole aligned tile: lane l's 16 bytes land at base + 16 l). A
// wave instruction moves 1 KiB: 4 key rows of 256 bytes at head dim 128 (8
// rows at 64, 2 at 256). Rows are stored with their 16-byte chunks
// XOR-swizzled by the key index so that both the K fragment reads and the V
// transposed reads spread over the LDS banks. Head dims 64, 128 and 256 share
// the code: D/16 contraction steps for Q K^T, D/32 output blocks for P V; at
// 256 the four tile buffers take 128 KiB of LDS and one work item runs per CU.
// Any other multiple of 8 up to 256 (dv) runs the next larger instance: rows
// are dv elements long in memory, query dims past dv are zero, LDS chunks
// past dv are filled from the row's first chunk, and no output dim past dv
// is stored. Aligned path
// (page_size % 64 == 0): the tile is one contiguous span of one page, found
// with a single table entry. Generic path: each key row is translated on
// its own (tiles that cross pages). Keys at or past the context end read a
// valid row instead of their (possibly missing) page; their scores are
// masked to -inf separately. Two LDS buffers: tile t+1 streams in while tile
// t is computed, one barrier per tile.
//
// Work items are ordered so that the heaviest causal row tiles start first;
// unsplit, the row tiles of one (sequence, kv head) are batch * num_kv_heads
// apart, on one XCD (shared L2) when that is a multiple of 8; split, all
// parts of one kv head run on one XCD when there are 8 kv heads.

#include <utility>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kBN = kPrefillBlockN;  // 64 keys per K/V tile (the automatic geometry)

// Geometry for head dim D (64, 128 or 256): a key row is 2D bytes = D/8
// chunks of 16 bytes; one global_load_lds instruction (64 lanes x 16 bytes)
// moves 1024 / (2D) rows, and a wave stages its 16 rows of a tile in D/32
// instructions.
template <int D, int BN = kBN>
struct Tile {
  static_assert(D == 64 || D == 128 || D == 256, "head dims 64, 128 and 256");
  static constexpr int kBytes = BN * 2 * D;  // one K (or V) tile of BN keys in LDS
  static constexpr int kChunks = D / 8;       // 16-byte chunks per key row
  static constexpr int kRowsPerInst = 512 / D;
  static constexpr int kInsts = D / 32;       // load instructions per wave per tile
  static constexpr int kKs = D / 16;          // 16-dim contraction steps of S = Q K^T
  static constexpr int kDb = D / 32;          // 32-dim output blocks of O = P V
  static constexpr int kBlocksPerCU = D <= 128 ? 2 : 1;  // LDS: 4 tiles per work item
};
// A wave's share of the tile loads in a work item of NW waves and BN-key
// tiles: keys [kKeys w, kKeys (w + 1)) of every tile (16 in both instances),
// kInsts instructions for K (and as many for V).
template <int D, int NW, int BN>
struct Stage {
  static constexpr int kKeys = BN / NW;
  static constexpr int kInsts = kKeys / Tile<D>::kRowsPerInst;
  static_assert(kInsts >= 1, "a wave loads whole instructions");
};
// The exponent reference of a row moves only when a tile maximum exceeds it
// by more than kTau (log2 units), so weights stay <= 2^kTau.
constexpr float kTau = 8.0f;

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4_t __attribute__((ext_vector_type(4)));

struct PrefillArgs {
  const uint16_t* query;
  const uint16_t* kpages;
  const uint16_t* vpages;
  const int32_t* block_table;
  const int32_t* context_lens;
  uint16_t* out;
  // Packed mixed batch: query/out [total_query, H_q, 128], sequence b owns
  // tokens [qstart[b], qstart[b + 1]); only sequences with skip_len < L_b <=
  // query_len are served here. nullptr: uniform [B, H_q, query_len, 128].
  const int32_t* qstart;
  int total_query, skip_len;
  int dv;  // head dim of query, pages and out (<= D: dims past it are masked)
  int batch, num_q_heads, num_kv_heads, query_len, group, n_qtiles;
  int page_size, ps_log2, max_pages;
  float c;         // |scale| * log2(e), > 0 (fold_scale)
  uint32_t qsign;  // XORed into every packed query pair: a negative scale negates q
  int causal;
  // Explicit additive mask (natural-log units, uniform layout): row (b, h, l),
  // key s at mask[b*msb + h*msh + l*msl + s] for s < mask_len; keys at or past
  // mask_len are absent. Used by the MASKED instances only.
  const float* mask;
  int64_t msb, msh, msl;
  int mask_len;
  int mask_vec;  // every mask row starts 16-byte aligned: four keys per load
  // Split key range (kv_splits > 1): work item i runs in p_i parts (1 <=
  // p_i <= kv_splits, from its length and the launch's total, see
  // split_assign); part s < p_i covers tiles [s * n / p_i, (s + 1) * n /
  // p_i) of its n tiles and leaves its rows' (reference max, row sum,
  // unnormalised output) in a workspace entry of its own; the part that
  // arrives last at counter i merges them.
  int num_work, kv_splits;
  int split_slots;   // resident workgroups of this kernel instance, at most kPrefillSplitTarget
  uint64_t* ws_ctr;  // [num_work] arrival counters (epoch << 32 | count)
  float* ws_ml;      // [kPrefillSplitTarget][128][2]
  float* ws_acc;     // [kPrefillSplitTarget][128][D]
  uint32_t epoch;
};

__device__ __forceinline__ int div_ps(int s, int ps, int ps_log2) { return ps_log2 >= 0 ? (s >> ps_log2) : s / ps; }

// 16-byte chunk c of key row `key` sits at chunk position c ^ swz(key). The
// swizzle spreads both kinds of fragment read over the 64 LDS banks (a
// 256-byte bank line):
//  - K (ds_read_b128): 16 lanes served together read one chunk of 16
//    consecutive keys, so key -> swz(key) must be one-to-one on every
//    aligned group of 16 keys;
//  - V^T (ds_read_b64_tr_b16): 32 lanes served together read chunks
//    4db .. 4db+3 of an aligned group of 4 keys, so the 4 keys must differ in
//    the top two bits of the 4-bit swizzle (the low two are the chunk's).
// 256-byte rows (D = 128) and longer ones take the low two key bits as the
// top two swizzle bits and key bits 2-3 as the low two. 128-byte rows
// (D = 64), two to a bank line, take a bit-reversed 3-bit index of the key
// pair (even and odd keys sit in different halves of the line).
template <int D>
__device__ __forceinline__ int swz(int key) {
  if (D == 64) {
    const int j = (key >> 1) & 7;
    return ((j & 1) << 2) | (j & 2) | ((j >> 2) & 1);
  }
  return ((key & 3) << 2) | ((key >> 2) & 3);
}

// The 16-byte chunk of a key row in memory that fills LDS chunk `chunk`: the
// chunk itself, or the row's first chunk for a chunk past the head dim dv
// (finite data that a zero query weights by 0 and no output dim stores).
template <bool GEN>
__device__ __forceinline__ int src_chunk(const PrefillArgs& a, int chunk) {
  return !GEN || chunk * 8 < a.dv ? chunk : 0;
}

// Byte offset of (key, chunk) inside a tile buffer.
template <int D>
__device__ __forceinline__ int tile_off(int key, int chunk) { return key * (2 * D) + ((chunk ^ swz<D>(key)) << 4); }

// Page lookup for the next tile to stage: the element offset of the key row
// each of the lane's 4 load instructions reads (generic path), or the
// tile's base row (aligned path, one entry).
template <bool ALIGNED, int D, int NW, int BN>
struct TilePages {
  size_t row[ALIGNED ? 1 : Stage<D, NW, BN>::kInsts];
};

typedef __attribute__((address_space(4))) const int32_t constant_i32;

template <bool ALIGNED, int D, bool GEN, int NW, int BN>
__device__ __forceinline__ void lookup_tile(const PrefillArgs& a, const int32_t* bt_row, size_t page_stride,
                                            size_t head_off, int ctx, int t0, int wave, int lane,
                                            TilePages<ALIGNED, D, NW, BN>& tp) {
  using T = Tile<D>;
  using S = Stage<D, NW, BN>;
  if (ALIGNED) {
    // one uniform entry per tile: a scalar load (the table is read-only here)
    const int lp = div_ps(t0, a.page_size, a.ps_log2);
    const int32_t page = ((constant_i32*)bt_row)[lp];
    tp.row[0] = (size_t)page * page_stride + head_off + (size_t)(t0 - lp * a.page_size) * (GEN ? a.dv : D);
  } else {
#pragma unroll
    for (int i = 0; i < S::kInsts; ++i) {
      int key = t0 + S::kKeys * wave + T::kRowsPerInst * i + lane / T::kChunks;
      key = key < ctx ? key : ctx - 1;  // past the context: re-read a valid row
      const int lp = div_ps(key, a.page_size, a.ps_log2);
      tp.row[i] = (size_t)bt_row[lp] * page_stride + head_off + (size_t)(key - lp * a.page_size) * (GEN ? a.dv : D);
    }
  }
}

// Issues the direct HBM -> LDS loads of one K/V tile. Wave w moves keys
// [16w, 16w + 16) of the tile (kKeys = 16 in both instances): instruction i
// covers the kRowsPerInst keys from 16w + kRowsPerInst*i; lane l takes key
// 16w + kRowsPerInst*i + l/kChunks and LDS chunk position l % kChunks, which
// holds global chunk
// (l % kChunks) ^ swz(key). A whole aligned tile is one contiguous span of
// one page: a wave-uniform base (scalar registers) plus a per-lane byte
// offset that is the same for every tile, so its loads cost no vector
// arithmetic.
// Word 3 of a raw (untyped, stride 0) buffer resource on gfx950: 32-bit data
// format, every other field zero.
constexpr int kRawBufferWord3 = 0x00020000;

// 16 bytes per lane from base + off + IMM into LDS at dst + IMM + 16 * lane,
// through a raw buffer over [base, base + bytes): base and size sit in scalar
// registers (the resource is built there), the lane's 32-bit offset is the
// only vector operand, so the load costs no vector instruction, and an offset
// past the buffer reads zeros instead of leaving it. The instruction's
// immediate offset IMM moves the source and the LDS destination alike (the
// LDS address is M0 + IMM + 16 * lane), so loads whose destinations differ by
// IMM share one M0 value. The host compilation pass has no buffer-resource
// type and never runs this code.
template <int IMM = 0>
__device__ __forceinline__ void buffer_load_lds16(const void* base, int bytes, uint32_t off, char* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRawBufferWord3), (lds_void*)dst,
      16, off, 0, IMM, 0);
#endif
}

// The per-lane byte offsets of a whole aligned tile's loads from its first
// row, computed once per work item (the empty asm statement keeps the
// compiler from re-deriving them inside the tile loop). Load i fills LDS
// bytes [1024 i, 1024 i + 1024) of the wave's part of the tile; when key rows
// have the LDS row length (no head-dim padding), its source also starts
// 1024 i bytes further into the page. The immediate offset field holds 12
// bits, so loads go in groups of four: group i / 4 has its own M0 (4096
// bytes apart) and load i carries 1024 * (i % 4) as its immediate, which the
// stored offset leaves out (every lane's key of load i is at least
// kRowsPerInst * i, so the difference stays non-negative).
template <int D, int NW, int BN>
struct TileOffsets {
  uint32_t off[Stage<D, NW, BN>::kInsts];
};

constexpr int kInstBytes = 1024;  // LDS bytes one load instruction fills (64 lanes x 16)
constexpr int kImmGroup = 4;      // loads per M0 value: immediates 0 .. 3072 stay below 4096
static_assert(kInstBytes * (kImmGroup - 1) < 4096, "buffer immediate offsets hold 12 bits");

template <int D, bool GEN, int NW, int BN>
__device__ __forceinline__ void tile_offsets(const PrefillArgs& a, int wave, int lane, TileOffsets<D, NW, BN>& to) {
  using T = Tile<D>;
  using S = Stage<D, NW, BN>;
#pragma unroll
  for (int i = 0; i < S::kInsts; ++i) {
    const int key = S::kKeys * wave + T::kRowsPerInst * i + lane / T::kChunks;  // key inside the tile
    const int chunk = src_chunk<GEN>(a, (lane % T::kChunks) ^ swz<D>(key));
    uint32_t off = (uint32_t)(key * (GEN ? a.dv : D) + chunk * 8) * 2u;  // bytes from the tile's first row
    if (!GEN) off -= (uint32_t)(kInstBytes * (i % kImmGroup));
    asm volatile("" : "+v"(off));
    to.off[i] = off;
  }
}

// The loads of a whole aligned tile without head-dim padding: one M0 value
// per group of four loads, load i placed by its immediate offset.
template <int D, int NW, int BN, size_t... I>
__device__ __forceinline__ void issue_tile_imm(const void* kbase, const void* vbase, int span,
                                               const TileOffsets<D, NW, BN>& to, char* kdst, char* vdst,
                                               std::index_sequence<I...>) {
  (buffer_load_lds16<kInstBytes * ((int)I % kImmGroup)>(kbase, span, to.off[I],
                                                         kdst + kInstBytes * kImmGroup * ((int)I / kImmGroup)), ...);
  (buffer_load_lds16<kInstBytes * ((int)I % kImmGroup)>(vbase, span, to.off[I],
                                                         vdst + kInstBytes * kImmGroup * ((int)I / kImmGroup)), ...);
}

template <bool ALIGNED, int D, bool GEN, int NW, int BN>
__device__ __forceinline__ void issue_tile(const PrefillArgs& a, const TilePages<ALIGNED, D, NW, BN>& tp,
                                           const TileOffsets<D, NW, BN>& to, int ctx, int t0, int wave, int lane,
                                           char* kbuf, char* vbuf) {
  using T = Tile<D>;
  using S = Stage<D, NW, BN>;
  if (ALIGNED && t0 + BN <= ctx) {
    const int span = BN * (GEN ? a.dv : D) * 2;  // bytes of the tile's rows
    const int wave_off = wave * S::kKeys * 2 * D;  // the wave's part of the LDS tile
    if constexpr (!GEN) {
      issue_tile_imm<D, NW, BN>(a.kpages + tp.row[0], a.vpages + tp.row[0], span, to, kbuf + wave_off,
                                vbuf + wave_off, std::make_index_sequence<S::kInsts>{});
    } else {
#pragma unroll
      for (int i = 0; i < S::kInsts; ++i) {
        const int lds_off = wave_off + i * kInstBytes;
        buffer_load_lds16(a.kpages + tp.row[0], span, to.off[i], kbuf + lds_off);
        buffer_load_lds16(a.vpages + tp.row[0], span, to.off[i], vbuf + lds_off);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < S::kInsts; ++i) {
    const int key = S::kKeys * wave + T::kRowsPerInst * i + lane / T::kChunks;  // key inside the tile
    const int chunk = src_chunk<GEN>(a, (lane % T::kChunks) ^ swz<D>(key));
    size_t row;
    if (ALIGNED) {
      // the tile lies in one page; keys past the context re-read the tile's first row
      row = tp.row[0] + (size_t)(t0 + key < ctx ? key : 0) * (GEN ? a.dv : D);
    } else {
      row = tp.row[i];
    }
    const size_t off = row + (size_t)chunk * 8;
    const int lds_off = wave * S::kKeys * 2 * D + i * 1024;
    __builtin_amdgcn_global_load_lds((global_void*)(a.kpages + off), (lds_void*)(kbuf + lds_off), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((global_void*)(a.vpages + off), (lds_void*)(vbuf + lds_off), 16, 0, 0);
  }
}

// 32-bit LDS address of a pointer into a __shared__ buffer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// ds_read_b128 issued as written (the compiler neither moves nor waits for
// it): the caller waits with lds_wait before using the result. Other LDS
// reads in flight only make such a counted wait longer, never too short.
template <int kOff>
__device__ __forceinline__ void lds_read_b128(u32x4_t& dst, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(kOff));
}

// Waits until at most n LDS reads are in flight; the fragments pass through
// the statement so that their users come after the wait.
__device__ __forceinline__ void lds_wait(int n, u32x4_t (&f)[2]) {
  switch (n) {
    case 0: asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f[0]), "+v"(f[1])); break;
    case 2: asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(f[0]), "+v"(f[1])); break;
    default: asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(f[0]), "+v"(f[1])); break;
  }
}

// Waits until at most n LDS reads are in flight (n a compile-time constant
// after unrolling); the fragment passes through the statement so that its
// users come after the wait.
__device__ __forceinline__ void lds_wait_n(int n, u32x4_t& f) {
  switch (n) {
    case 0: asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f)); break;
    case 1: asm volatile("s_waitcnt lgkmcnt(1)" : "+v"(f)); break;
    case 2: asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(f)); break;
    case 3: asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(f)); break;
    case 4: asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(f)); break;
    case 5: asm volatile("s_waitcnt lgkmcnt(5)" : "+v"(f)); break;
    default: asm volatile("s_waitcnt lgkmcnt(6)" : "+v"(f)); break;
  }
}

// The two transposed 8-byte reads of one V^T fragment (ds_read_b64_tr_b16:
// lane i of each 16-lane group receives element i % 4 of the 8 bytes that
// lane 4j + i / 4 addresses, as its element j) for 16-key step ks of the
// tile, issued as written.
template <int kStepBytes>
__device__ __forceinline__ void lds_read_tr_pair(u32x4_t& f, uint32_t lo_addr, uint32_t hi_addr, int ks) {
  u32x2_t lo, hi;
  switch (ks) {
    case 0:
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(lo_addr));
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(hi) : "v"(hi_addr));
      break;
    case 1:
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(lo_addr), "i"(kStepBytes));
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(hi_addr), "i"(kStepBytes));
      break;
    case 2:
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(lo_addr), "i"(2 * kStepBytes));
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(hi_addr), "i"(2 * kStepBytes));
      break;
    default:
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(lo_addr), "i"(3 * kStepBytes));
      asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(hi_addr), "i"(3 * kStepBytes));
      break;
  }
  f = u32x4_t{lo.x, lo.y, hi.x, hi.y};
}

__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Key tiles a work item of row tile `rtile` of a sequence with L query rows
// and context ctx streams (the whole-tile causal skip included).
template <int BM, int BN>
__device__ __forceinline__ int item_tiles(const PrefillArgs& a, int rtile, int L, int ctx) {
  const int R = a.group * L;
  const int tile_last_pos = (min(rtile * BM + BM, R) - 1) / a.group;
  const int kv_end = a.causal ? min(ctx, tile_last_pos + ctx - L + 1) : ctx;
  return (kv_end + BN - 1) / BN;
}

// What a workgroup of a split launch runs: part `part` of the n_parts of
// work item `item` (item < 0: nothing), its partial state in workspace
// entry (u0 + part) * num_kv_heads + kv head.
struct SplitItem {
  int item, part, n_parts, u0;
};

// Parts of a pair with nt key tiles (nt < 0: no rows, no part) at part
// length T: clamp(ceil(nt / T), 1, min(cap, nt / 2)), without branches.
// capT = cap * T, rT ~ 1 / T. ceil is taken of min(nt, capT) / T, which is
// at most cap and equal to cap when nt > capT; for it a single-precision
// estimate is off by one at most and one integer step corrects it.
__device__ __forceinline__ int pair_parts(int nt, int T, int cap, int capT, float rT) {
  const int y = min(nt, capT) + T - 1;
  int q = (int)((float)y * rT);
  q -= q * T > y ? 1 : 0;
  q += (q + 1) * T <= y ? 1 : 0;
  const int p = max(1, min(q, min(cap, nt >> 1)));
  return nt < 0 ? 0 : p;
}

// Assignment of a split launch's workgroups, the same in every workgroup.
// The (sequence, row tile) pairs are taken in work-item order, heavy row
// tiles first: pair o is row tile n_qtiles - 1 - o / batch of sequence
// o % batch, and streams n_o key tiles. The part length T (in tiles) is the
// smallest for which
//   H_kv * sum_o parts(n_o, T) <= a.split_slots,
//   parts(n, T) = clamp(ceil(n / T), 1, min(kv_splits, n / 2)),
// searched over NT candidates in parallel (one per thread) from
// ceil(total / slots) to the longest pair (where every pair has one part),
// so that every part is resident at once and the longest sequences do not
// set the time. The parts are listed pair by pair, each once per kv head:
// workgroup w runs the u-th listed part, u = w / H_kv, for kv head w % H_kv
// (with 8 kv heads every part of a kv head lands on one XCD and shares its
// L2); workgroups past the list run nothing. Called by every thread
// (barriers inside); there are fewer pairs than kPrefillSplitTarget.
template <int NT, int BM, int BN>
__device__ SplitItem split_assign(const PrefillArgs& a, int* lds_n, int64_t* lds_sum, int* lds_red) {
  const int nq = a.n_qtiles;
  const int pairs = a.batch * nq;
  const int pairs4 = (pairs + 3) & ~3;  // padded with empty pairs for 4-wide reads
  int64_t sum = 0;
  int longest = 0;
  for (int o = threadIdx.x; o < pairs4; o += NT) {
    int t = -1;  // no rows: no part
    if (o < pairs) {
      const int b = o % a.batch, r = nq - 1 - o / a.batch;
      int L = a.query_len;
      bool live = true;
      if (a.qstart) {
        const int s0 = a.qstart[b], s1 = a.qstart[b + 1];
        const int64_t len = (int64_t)s1 - s0;
        live = !(s0 < 0 || s1 > a.total_query || len <= a.skip_len || len > a.query_len);
        L = live ? (int)len : 0;
      }
      if (live && r * BM < a.group * L) t = max(0, item_tiles<BM, BN>(a, r, L, a.context_lens[b]));
    }
    lds_n[o] = t;
    sum += max(t, 0);
    longest = max(longest, t);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    sum += __shfl_xor(sum, m);
    longest = max(longest, __shfl_xor(longest, m));
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    lds_sum[w] = sum;
    lds_red[w] = longest;
  }
  __syncthreads();
  const int H = a.num_kv_heads;
  int64_t total = 0;
  int hi = 1;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    total += lds_sum[i];
    hi = max(hi, lds_red[i]);
  }
  total *= H;
  // ceil(total / slots) in double precision (exact below 2^53, no 64-bit integer division)
  const int lo = (int)fmin((double)hi, fmax(2.0, ceil((double)total / (double)a.split_slots)));
  const int step = max(1, (hi - lo + NT - 2) / (NT - 1));
  const int cap = a.kv_splits;
  {
    const int cand = threadIdx.x == NT - 1 ? hi : min(hi, lo + (int)threadIdx.x * step);
    const float rc = 1.0f / (float)cand;
    const int capc = cap * cand;
    int count = 0;  // at most cap * pairs
#pragma unroll 2
    for (int o = 0; o < pairs4; o += 4) {
      const int4 v = *reinterpret_cast<const int4*>(lds_n + o);  // the same address in every lane
      count += pair_parts(v.x, cand, cap, capc, rc) + pair_parts(v.y, cand, cap, capc, rc) +
               pair_parts(v.z, cand, cap, capc, rc) + pair_parts(v.w, cand, cap, capc, rc);
    }
    int best = (int64_t)count * H <= a.split_slots ? cand : hi;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) best = min(best, __shfl_xor(best, m));
    __syncthreads();  // every wave has read lds_red
    if (lane == 0) lds_red[w] = best;
  }
  __syncthreads();
  int T = lds_red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) T = min(T, lds_red[i]);
  const float rT = 1.0f / (float)T;
  const int capT = cap * T;
  // wave 0: lane l takes a run of C pairs, a wave prefix sum gives each run's first part
  const int u = (int)(blockIdx.x / (unsigned)H);
  __shared__ SplitItem found;
  if (w == 0) {
    const int C = (pairs + 63) / 64;
    const int o0 = min(pairs, lane * C), o1 = min(pairs, o0 + C);
    int mine = 0;
    for (int o = o0; o < o1; ++o) mine += pair_parts(lds_n[o], T, cap, capT, rT);
    int incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    if (lane == 63) found = SplitItem{-1, 0, 0, 0};
    int pre = incl - mine;
    if (u >= pre && u < incl) {  // one lane: the run that holds part u
      for (int o = o0; o < o1; ++o) {
        const int np = pair_parts(lds_n[o], T, cap, capT, rT);
        if (u < pre + np) {
          found = SplitItem{o * H + (int)(blockIdx.x % (unsigned)H), u - pre, np, pre};
          break;
        }
        pre += np;
      }
    }
  }
  __syncthreads();
  return found;
}

// A work item is NW waves of 32 packed rows each, and K/V tiles hold BN keys:
// NW = 4, BN = 64 (128 rows x 64 keys, the automatic prefill schedule), or
// NW = 2, BN = 32 (64 rows x 32 keys: the tiling of the matrix kernel in
// "Week 3 Day 5: Paged FlashAttention", Task 1, kept to measure against;
// unmasked and never split).
// (The second launch bound is read by the compiler as waves per SIMD for
// these sizes: 2 keeps the register budget of two waves per SIMD in both.
// The MASKED instances at head dim 128 keep it too, with four 64-bit values
// spilled to scratch and reloaded in each tile step: two work items per CU
// measured 1.7x faster on the masked long prefill than one without spills.)
template <bool ALIGNED, int D, bool MASKED, bool GEN, int NW, int BN>
__global__ void __launch_bounds__(64 * NW, NW == 4 ? Tile<D>::kBlocksPerCU : (D <= 128 ? 2 : 1))
    pa_prefill_mfma(PrefillArgs a) {
  using T = Tile<D, BN>;
  constexpr int kNT = 64 * NW;    // threads
  constexpr int kRows = 32 * NW;  // packed rows of a work item
  constexpr int kNB = BN / 32;    // 32-key score blocks per tile
  constexpr int kSteps = BN / 16;  // 16-key P V steps per tile
  static_assert((NW == 4 && BN == 64) || (NW == 2 && BN == 32 && !MASKED && !GEN), "work item geometries");
  __shared__ __attribute__((aligned(1024))) char lds_k0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v1[T::kBytes];
  __shared__ __attribute__((aligned(16))) int lds_n[kPrefillSplitTarget];  // split launches: tiles per pair
  __shared__ int64_t lds_sum[kNT / 64];
  __shared__ int lds_red[kNT / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar address math
  const int half = lane >> 5;  // which 8-wide k slice of an MFMA operand this lane feeds
  const int col = lane & 31;   // query row (within the wave) owned by this lane

  // ---- work item: (row tile, kv head, sequence), heavy row tiles first ----
  // The rows of a work item are (position, query head) pairs of the G query
  // heads that read its kv head, position-major: packed row r is position
  // r / G of head kvh * G + r % G, so every K/V tile serves the whole group
  // and short queries still fill the waves. Unsplit, workgroup w runs work
  // item w; consecutive work items of one (sequence, kv head) are batch *
  // num_kv_heads apart, on one XCD when that is a multiple of 8. Split, see
  // split_assign.
  int item = (int)blockIdx.x, part = 0, n_parts = 1, u0 = 0;
  if (a.kv_splits > 1) {
    const SplitItem si = split_assign<kNT, kRows, BN>(a, lds_n, lds_sum, lds_red);
    if (si.item < 0) return;  // past the list of parts (uniform across the workgroup)
    item = si.item;
    part = si.part;
    n_parts = si.n_parts;
    u0 = si.u0;
  }
  const int G = a.group;
  int task = item;
  const int kvh = task % a.num_kv_heads;
  task /= a.num_kv_heads;
  const int b = task % a.batch;
  const int rtile = a.n_qtiles - 1 - task / a.batch;

  int L = a.query_len, start = 0;
  if (a.qstart) {
    const int s0 = a.qstart[b], s1 = a.qstart[b + 1];
    const int64_t len = (int64_t)s1 - s0;
    if (s0 < 0 || s1 > a.total_query || len <= a.skip_len || len > a.query_len) return;
    L = (int)len;
    start = s0;
  }
  const int R = G * L;  // packed rows of this sequence and kv head
  const int q0 = rtile * kRows;
  if (q0 >= R) return;  // a row tile past this sequence's rows (uniform across the work item)
  const int ctx = a.context_lens[b];
  const int offset = ctx - L;  // query position l sits at logical position l + offset
  const int tile_last_pos = (min(q0 + kRows, R) - 1) / G;
  const int kv_end = a.causal ? min(ctx, tile_last_pos + offset + 1) : ctx;
  const int n_tiles_all = (kv_end + BN - 1) / BN;
  // this workgroup's tiles [t_lo, n_tiles): part `part` of n_parts
  const int t_lo = (int)((int64_t)part * n_tiles_all / n_parts);
  const int n_tiles = (int)((int64_t)(part + 1) * n_tiles_all / n_parts);

  const int r0 = q0 + 32 * wave;  // first packed row of this wave
  const bool wave_has_rows = r0 < R;
  const int wave_first_pos = r0 / G;
  const int wave_last_pos = (min(r0 + 31, R - 1)) / G;
  const int wave_kv_end = a.causal ? min(ctx, wave_last_pos + offset + 1) : ctx;
  // this lane's packed row: position pos of query head head (rows past R re-read row R - 1, never stored)
  const int row_abs = r0 + col;
  const int row_c = row_abs < R ? row_abs : R - 1;
  const int pos = row_c / G;
  const int head = kvh * G + row_c % G;

  const size_t head_stride = (size_t)a.page_size * (GEN ? a.dv : D);
  const size_t page_stride = head_stride * a.num_kv_heads;
  const size_t head_off = (size_t)kvh * head_stride;
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;

  // ---- first tile in flight before anything else ----
  TileOffsets<D, NW, BN> to;
  if (ALIGNED) tile_offsets<D, GEN, NW, BN>(a, wave, lane, to);
  TilePages<ALIGNED, D, NW, BN> tp;
  if (n_tiles > t_lo) {
    lookup_tile<ALIGNED, D, GEN, NW, BN>(a, bt_row, page_stride, head_off, ctx, t_lo * BN, wave, lane, tp);
    issue_tile<ALIGNED, D, GEN, NW, BN>(a, tp, to, ctx, t_lo * BN, wave, lane, lds_k0, lds_v0);
    lookup_tile<ALIGNED, D, GEN, NW, BN>(a, bt_row, page_stride, head_off, ctx, min(t_lo + 1, n_tiles - 1) * BN, wave,
                                         lane, tp);
  }

  // ---- Q^T operand: lane holds row r0 + col, dims 16ks + 8half .. +8 ----
  bf16x8_t qv[T::kKs];
  {
    const size_t qrow = a.qstart ? (size_t)(start + pos) * a.num_q_heads + head : ((size_t)b * a.num_q_heads + head) * L + pos;
    const uint16_t* qp = a.query + qrow * (GEN ? a.dv : D) + 8 * half;
#pragma unroll
    for (int ks = 0; ks < T::kKs; ++ks) {
      // dims past dv stay zero, so their (re-read) key chunks add nothing
      u32x4_t w = u32x4_t{0u, 0u, 0u, 0u};
      if (row_abs < R && (!GEN || 16 * ks + 8 * half < a.dv)) w = *reinterpret_cast<const u32x4_t*>(qp + 16 * ks) ^ a.qsign;
      qv[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  f32x16_t acc_o[T::kDb];
#pragma unroll
  for (int db = 0; db < T::kDb; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_o[db][i] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's half of the row sum

  // LDS reads of this lane (tile-relative):
  // K fragment (kb, ks): key 32kb + col, chunk 2ks + half.
  // V^T fragment (db, ks): keys 16ks + 4half + (lane%16)/4 and that + 8,
  //   dims 32db + 16((lane/16)&1) + 4(lane%4) .. +4, i.e. chunk
  //   4db + 2((lane/16)&1) + (lane%4)/2 at byte 8(lane&1) inside it.
  const int vk_lane = 4 * half + ((lane & 15) >> 2);
  const int vc_lane = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vb_lane = 8 * (lane & 1);
  const uint32_t ones_bf16x2 = 0x3F803F80u;  // (1.0, 1.0) in bf16
  // V^T fragment of 16-key step 0, dims [0, 32): rows vk_lane and vk_lane + 8,
  // chunk vc_lane, byte vb_lane. Chunk positions are XOR-swizzled and the
  // chunk bits of a row offset are zero, so dims block db is an XOR by 4db
  // chunks and step ks adds 16 rows.
  const uint32_t v_lane0 = (uint32_t)tile_off<D>(vk_lane, vc_lane) + vb_lane;
  const uint32_t v_lane1 = (uint32_t)tile_off<D>(vk_lane + 8, vc_lane) + vb_lane;

  // this lane's mask row (MASKED only)
  const float* mrow = a.mask;
  if (MASKED) mrow = a.mask + (size_t)b * a.msb + (size_t)head * a.msh + (size_t)pos * a.msl;
  // One tile: wait for its loads, barrier, start the next tile's loads into
  // the other buffer, compute. The buffers are distinct LDS objects chosen
  // statically (the loop is unrolled by two), so no wait is needed between
  // the next tile's loads and this tile's reads.
  auto tile_step = [&](int t, const char* kb_base, const char* vb_base, char* knext, char* vnext) {
    const int t0 = t * BN;
    wait_all_loads();  // this wave's part of tile t (and the next lookup) has landed
    __syncthreads();   // every wave's part is in LDS; every wave is done with tile t - 1
    const bool active = wave_has_rows && t0 < wave_kv_end;
    // mask entries of this lane's row for the tile's keys; issued before the
    // next tile's loads so that waiting for them does not wait for those
    float mvals[MASKED ? kNB : 1][16];
    if constexpr (MASKED) {
      if (active) {
        // elements 4j .. 4j+3 of a block are four consecutive keys (a multiple of 4 first)
  #pragma unroll
        for (int kb = 0; kb < kNB; ++kb)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int k0 = t0 + 32 * kb + 8 * j + 4 * half;
            if (a.mask_vec && k0 + 3 < a.mask_len) {
              const f32x4_t v = *reinterpret_cast<const f32x4_t*>(mrow + k0);
              mvals[kb][4 * j] = v.x;
              mvals[kb][4 * j + 1] = v.y;
              mvals[kb][4 * j + 2] = v.z;
              mvals[kb][4 * j + 3] = v.w;
            } else {
  #pragma unroll
              for (int e = 0; e < 4; ++e) mvals[kb][4 * j + e] = mrow[min(k0 + e, a.mask_len - 1)];
            }
          }
      }
    }
    if (t + 1 < n_tiles) issue_tile<ALIGNED, D, GEN, NW, BN>(a, tp, to, ctx, t0 + BN, wave, lane, knext, vnext);
    // Lookup for tile t + 2 (clamped so that it is unconditional), done
    // after this tile's matrix work, not between the barrier and it.
    const int t_look = min(t + 2, n_tiles - 1) * BN;
    if (!active) {
      lookup_tile<ALIGNED, D, GEN, NW, BN>(a, bt_row, page_stride, head_off, ctx, t_look, wave, lane, tp);
      return;
    }

      // ---- S^T = K Q^T : kNB 32-key blocks (two at 64-key tiles) ----
      // Contraction step ks runs the MFMAs of both blocks; the K fragments of
      // step ks + 2 are read from LDS meanwhile. The reads and their waits
      // are explicit: LDS reads complete in order, so before step ks only
      // the reads of the two later steps may still be in flight.
      f32x16_t acc_s[kNB];
  #pragma unroll
      for (int kb = 0; kb < kNB; ++kb)
  #pragma unroll
        for (int i = 0; i < 16; ++i) acc_s[kb][i] = 0.f;
      {
        // Chunk 2ks + half of key col (block 0) and key 32 + col (block 1).
        // Chunk positions are XOR-swizzled and the chunk bits of a row's
        // byte offset are zero, so step ks is an XOR by 2ks chunks.
        const uint32_t kaddr0 = lds_addr(kb_base) + tile_off<D>(col, half);
        u32x4_t kf[3][2];  // [buffer][block]
        auto read_k = [&](int ks, u32x4_t (&dst)[2]) {
          const uint32_t a0 = kaddr0 ^ (uint32_t)(ks << 5);
          lds_read_b128<0>(dst[0], a0);
          if constexpr (kNB > 1) lds_read_b128<32 * 2 * D>(dst[1], a0);
        };
        read_k(0, kf[0]);
        read_k(1, kf[1]);
  #pragma unroll
        for (int ks = 0; ks < T::kKs; ++ks) {
          if (ks + 2 < T::kKs) read_k(ks + 2, kf[(ks + 2) % 3]);
          const int younger = kNB * min(2, T::kKs - 1 - ks);  // reads issued after step ks's
          if constexpr (kNB > 1) lds_wait(younger, kf[ks % 3]);
          else lds_wait_n(younger, kf[ks % 3][0]);
  #pragma unroll
          for (int kb = 0; kb < kNB; ++kb)
            acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[ks % 3][kb]), qv[ks],
                                                                acc_s[kb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // V^T fragments of the first kVA P V groups: read during the softmax
      constexpr int kVG = kSteps * T::kDb;  // P V groups: (16-key step, 32-dim block)
      constexpr int kVA = 3;           // groups read ahead
      const uint32_t vaddr0 = lds_addr(vb_base) + v_lane0, vaddr1 = lds_addr(vb_base) + v_lane1;
      u32x4_t vf[kVA + 1];
      auto issue_v = [&](int g) {
        if (g >= kVG) return;
        const int ks = g / T::kDb, db = g % T::kDb;
        lds_read_tr_pair<16 * 2 * D>(vf[g % (kVA + 1)], vaddr0 ^ (uint32_t)(db << 6), vaddr1 ^ (uint32_t)(db << 6), ks);
      };
  #pragma unroll
      for (int g = 0; g < kVA; ++g) issue_v(g);

      // ---- mask, online softmax (row = this lane's query row) ----
      // element i of block kb is key 32kb + 8(i/4) + 4half + i%4 of the tile.
      // Without an explicit mask the maximum is taken on raw scores (c > 0)
      // and the scale is folded into the exponent argument; with one, each
      // score becomes scale * q.k + mask in log2 units first (cs = 1).
      float cs = a.c;
      if constexpr (MASKED) {
  #pragma unroll
        for (int kb = 0; kb < kNB; ++kb)
  #pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = t0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
            acc_s[kb][i] = key < a.mask_len ? fmaf(acc_s[kb][i], a.c, mvals[kb][i] * kLog2e) : -INFINITY;
          }
        cs = 1.f;
      }
      const bool need_mask = (t0 + BN > ctx) || (a.causal && t0 + BN - 1 > wave_first_pos + offset);
      if (need_mask) {
  #pragma unroll
        for (int kb = 0; kb < kNB; ++kb) {
  #pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = t0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
            const bool vis = key < ctx && (!a.causal || key <= pos + offset);
            acc_s[kb][i] = vis ? acc_s[kb][i] : -INFINITY;
          }
        }
      }
      float mx[kNB];
  #pragma unroll
      for (int kb = 0; kb < kNB; ++kb) {
        const float m0 = fmaxf(fmaxf(acc_s[kb][0], acc_s[kb][1]), acc_s[kb][2]);
        const float m1 = fmaxf(fmaxf(acc_s[kb][3], acc_s[kb][4]), acc_s[kb][5]);
        const float m2 = fmaxf(fmaxf(acc_s[kb][6], acc_s[kb][7]), acc_s[kb][8]);
        const float m3 = fmaxf(fmaxf(acc_s[kb][9], acc_s[kb][10]), acc_s[kb][11]);
        const float m4 = fmaxf(fmaxf(acc_s[kb][12], acc_s[kb][13]), acc_s[kb][14]);
        mx[kb] = fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), acc_s[kb][15]));
      }
      const float tmax = max_xor32(fmaxf(mx[0], mx[kNB - 1])) * cs;  // log2 units
      // The exponent reference moves only when the tile maximum exceeds it by
      // more than kTau; otherwise the weights stay <= 2^kTau and the output
      // needs no rescale. The branch is taken when any row of the wave moves.
      const bool grow = tmax > m_run + kTau;
      if (__ballot(grow)) {
        const float alpha = grow ? fast_exp2(m_run - tmax) : 1.f;  // 0 while the old reference is -inf
        m_run = grow ? tmax : m_run;
        l_run *= alpha;
  #pragma unroll
        for (int db = 0; db < T::kDb; ++db)
  #pragma unroll
          for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
      }
      const float neg_ref = m_run == -INFINITY ? 0.f : -m_run;
      uint32_t pk[kNB][8];  // P^T operand, packed bf16 pairs
      float psum = 0.f;
  #pragma unroll
      for (int kb = 0; kb < kNB; ++kb) {
  #pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = fast_exp2(fmaf(acc_s[kb][i], cs, neg_ref));
          const float p1 = fast_exp2(fmaf(acc_s[kb][i + 1], cs, neg_ref));
          pk[kb][i >> 1] = pack_bf16x2(p0, p1);
          psum = dot2_bf16(pk[kb][i >> 1], ones_bf16x2, psum);  // the weights the MFMA uses
        }
      }
      l_run += psum;

      // ---- O^T += V^T P^T : 4 steps of 16 keys, 32-dim blocks ----
      // LDS reads complete in order: before group g only the reads of the
      // next kVA groups may still be in flight.
  #pragma unroll
      for (int g = 0; g < kVG; ++g) {
        const int ks = g / T::kDb, db = g % T::kDb;
        issue_v(g + kVA);
        lds_wait_n(2 * min(kVA, kVG - 1 - g), vf[g % (kVA + 1)]);
        const uint32_t* src = &pk[ks >> 1][(ks & 1) * 4];
        const u32x4_t pw = {src[0], src[1], src[2], src[3]};
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[g % (kVA + 1)]),
                                                            __builtin_bit_cast(bf16x8_t, pw), acc_o[db], 0, 0, 0);
      }
      lookup_tile<ALIGNED, D, GEN, NW, BN>(a, bt_row, page_stride, head_off, ctx, t_look, wave, lane, tp);
  };
  for (int t = t_lo; t < n_tiles; t += 2) {
    tile_step(t, lds_k0, lds_v0, lds_k1, lds_v1);
    if (t + 1 < n_tiles) tile_step(t + 1, lds_k1, lds_v1, lds_k0, lds_v0);
  }
  wait_all_loads();  // no load may still be writing this work item's LDS at exit

  // ---- split key range: leave this part's state, the last part merges ----
  // State of a part in its workspace entry e: (reference max, row sum) of
  // row r at ws_ml[(e * 128 + r) * 2], the unnormalised output in the
  // register layout: chunk c = 4db + g (dims 32db + 8g + 4half .. +4) of
  // wave w's lane l at ws_acc[((e * 4 + w) * kChunks + c) * 256 + 4l], so
  // that every 16-byte store and load of a wave covers 1 KiB in one piece.
  // A row that saw no key keeps -inf, sum 0 and a zero output. The last
  // part to arrive merges the parts in order ("Week 2 Day 5", Task 2:
  // rescale each partial to the common maximum, one denominator): the
  // others from the workspace, its own from its registers (the values it
  // stored), so the sum runs in the same order, over the same values,
  // whichever part arrives last.
  constexpr int kChunks = T::kDb * 4;
  float l_fin;
  if (n_parts > 1) {
    const int H = a.num_kv_heads;
    const size_t entry = (size_t)(u0 + part) * H + kvh;
    if (wave_has_rows) {
      const float l_tot = sum_xor32(l_run);
      if (half == 0 && row_abs < R) store_coherent_x2(a.ws_ml + (entry * kRows + 32 * wave + col) * 2, f32x2_t{m_run, l_tot});
      float* wp = a.ws_acc + (entry * NW + wave) * kChunks * 256 + 4 * lane;
#pragma unroll
      for (int db = 0; db < T::kDb; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          store_coherent_x4(wp + (4 * db + g4) * 256, f32x4_t{acc_o[db][4 * g4], acc_o[db][4 * g4 + 1],
                                                             acc_o[db][4 * g4 + 2], acc_o[db][4 * g4 + 3]});
    }
    wait_stores();
    __shared__ bool lds_last;
    __syncthreads();
    if (tid == 0) lds_last = arrive_last(a.ws_ctr + item, a.epoch, (uint32_t)n_parts);
    __syncthreads();
    if (!lds_last || !wave_has_rows) return;
    // every part's (max, sum) of this lane's row (rows past R: unused values)
    f32x2_t ml[kPrefillMaxSplits];
#pragma unroll
    for (int s = 0; s < kPrefillMaxSplits; ++s) {
      const size_t e = (size_t)(u0 + min(s, n_parts - 1)) * H + kvh;
      ml[s] = load_coherent_x2(a.ws_ml + (e * kRows + 32 * wave + col) * 2);
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kPrefillMaxSplits; ++s)
      if (s < n_parts) M = fmaxf(M, ml[s].x);
    float den = 0.f;
    f32x16_t mo[T::kDb];  // the merged output (acc_o still holds this part's)
#pragma unroll
    for (int db = 0; db < T::kDb; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) mo[db][i] = 0.f;
    for (int s = 0; s < n_parts; ++s) {
      f32x4_t av[kChunks];
      if (s != part) {
        const size_t e = (size_t)(u0 + s) * H + kvh;
        const float* rp = a.ws_acc + (e * NW + wave) * kChunks * 256 + 4 * lane;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) av[c] = load_coherent_x4(rp + c * 256);
      } else {
#pragma unroll
        for (int db = 0; db < T::kDb; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            av[4 * db + g4] = f32x4_t{acc_o[db][4 * g4], acc_o[db][4 * g4 + 1], acc_o[db][4 * g4 + 2], acc_o[db][4 * g4 + 3]};
      }
      float ms = ml[0].x, ls = ml[0].y;
#pragma unroll
      for (int k = 1; k < kPrefillMaxSplits; ++k)
        if (s == k) {
          ms = ml[k].x;
          ls = ml[k].y;
        }
      const float f = ms == -INFINITY ? 0.f : fast_exp2(ms - M);  // a part without a visible key adds nothing
      den = fmaf(f, ls, den);
#pragma unroll
      for (int db = 0; db < T::kDb; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          mo[db][4 * g4] = fmaf(f, av[4 * db + g4].x, mo[db][4 * g4]);
          mo[db][4 * g4 + 1] = fmaf(f, av[4 * db + g4].y, mo[db][4 * g4 + 1]);
          mo[db][4 * g4 + 2] = fmaf(f, av[4 * db + g4].z, mo[db][4 * g4 + 2]);
          mo[db][4 * g4 + 3] = fmaf(f, av[4 * db + g4].w, mo[db][4 * g4 + 3]);
        }
    }
#pragma unroll
    for (int db = 0; db < T::kDb; ++db) acc_o[db] = mo[db];
    l_fin = den;
  } else {
    if (!wave_has_rows) return;
    l_fin = sum_xor32(l_run);
  }

  // ---- finalize: divide by the row sum, store bf16 ----
  if (row_abs >= R) return;
  const float inv = 1.f / l_fin;  // a row without any visible key: 0 / 0
  const size_t orow = a.qstart ? (size_t)(start + pos) * a.num_q_heads + head
                               : ((size_t)b * a.num_q_heads + head) * L + pos;
  uint16_t* op = a.out + orow * (GEN ? a.dv : D);
#pragma unroll
  for (int db = 0; db < T::kDb; ++db) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int d0 = 32 * db + 8 * grp + 4 * half;
      if (GEN && d0 >= a.dv) continue;  // a masked dim (dv is a multiple of 8)
      const u32x2_t w = {pack_bf16x2(acc_o[db][4 * grp] * inv, acc_o[db][4 * grp + 1] * inv),
                         pack_bf16x2(acc_o[db][4 * grp + 2] * inv, acc_o[db][4 * grp + 3] * inv)};
      *reinterpret_cast<u32x2_t*>(op + d0) = w;
    }
  }
}

// CUs and workgroups of one kernel instance the GPU keeps resident (cached
// per device).
struct Residency {
  int cus, slots;
};

template <bool ALIGNED, int D, bool MASKED, bool GEN, int NW, int BN>
Residency resident_slots() {
  static Residency cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev].slots > 0) return cache[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)pa_prefill_mfma<ALIGNED, D, MASKED, GEN, NW, BN>, 64 * NW,
                                                   0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  cache[dev] = Residency{cus, cus * per_cu};
  return cache[dev];
}

template <bool ALIGNED, int D, bool MASKED, bool GEN, int NW = 4, int BN = kBN>
hipError_t launch_instance(PrefillArgs a, const Plan& p, hipStream_t stream) {
  // split: one workgroup per workspace entry, the resident ones used
  const unsigned grid = (unsigned)(a.kv_splits > 1 ? kPrefillSplitTarget : p.num_work);
  if (a.kv_splits > 1) a.split_slots = min(kPrefillSplitTarget, resident_slots<ALIGNED, D, MASKED, GEN, NW, BN>().slots);
  hipLaunchKernelGGL((pa_prefill_mfma<ALIGNED, D, MASKED, GEN, NW, BN>), dim3(grid), dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool MASKED>
hipError_t launch_mask(const PrefillArgs& a, const Plan& p, hipStream_t stream) {
  if constexpr (!MASKED) {
    if (p.schedule == kSchedulePrefill64x32)  // native head dims only, never split (the plan's checks)
      return p.aligned ? launch_instance<true, D, false, false, 2, 32>(a, p, stream)
                       : launch_instance<false, D, false, false, 2, 32>(a, p, stream);
  }
  if (a.dv != D)  // a head dim without an instance of its own: the next larger one, masked dims, per-row loader
    return launch_instance<false, D, MASKED, true>(a, p, stream);
  if (p.aligned) return launch_instance<true, D, MASKED, false>(a, p, stream);
  return launch_instance<false, D, MASKED, false>(a, p, stream);
}

template <int D>
hipError_t launch_dim(const PrefillArgs& a, const Plan& p, hipStream_t stream) {
  return a.mask ? launch_mask<D, true>(a, p, stream) : launch_mask<D, false>(a, p, stream);
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
  const ScaleFold sf = fold_scale(k.scale);
  a.c = sf.c;
  a.qsign = sf.qsign;
  a.causal = k.causal;
  a.qstart = k.query_start;
  a.total_query = k.total_query;
  a.skip_len = k.query_start ? k.dec_max_len : 0;
  a.dv = k.head_dim;
  a.mask = k.mask;
  a.msb = k.mask_stride_b;
  a.msh = k.mask_stride_h;
  a.msl = k.mask_stride_l;
  a.mask_len = k.mask_len;
  a.mask_vec = k.mask && (reinterpret_cast<uintptr_t>(k.mask) % 16 == 0) && k.mask_stride_b % 4 == 0 &&
               k.mask_stride_h % 4 == 0 && k.mask_stride_l % 4 == 0;
  a.num_work = (int)p.num_work;
  a.kv_splits = p.kv_splits;
  a.epoch = k.epoch;
  a.ws_ctr = nullptr;
  a.ws_ml = a.ws_acc = nullptr;
  if (p.kv_splits > 1) {
    char* ws = static_cast<char*>(k.workspace);
    a.ws_ctr = reinterpret_cast<uint64_t*>(ws + p.ws_ctr_offset);
    a.ws_ml = reinterpret_cast<float*>(ws + p.ws_ml_offset);
    a.ws_acc = reinterpret_cast<float*>(ws + p.ws_acc_offset);
  }
  switch (instance_dim(k.head_dim)) {
    case 64: return launch_dim<64>(a, p, stream);
    case 256: return launch_dim<256>(a, p, stream);
    default: return launch_dim<128>(a, p, stream);
  }
}

}  // namespace pa
