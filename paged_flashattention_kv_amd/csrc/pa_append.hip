// pa_append.hip -- the write half of the paged K/V cache for gfx950: the
// keys and values of L new tokens per sequence go to their page slots
// through the same translation the attention kernels read with
// ("Week 3 Day 5: Paged FlashAttention": logical position -> block_table ->
// page, slot; the causal decode that follows a paged prefill needs the new
// token's K/V in its page first).
//
// Token l of sequence b sits at logical position s = context_lens[b] - L + l
// (context_lens counts the tokens after the append, the same convention the
// attention kernels use for query rows). Its K row for kv head h is copied
// to key_pages[block_table[b][s / page_size], h, s % page_size, :], and the
// same for V. HBM-bound: every new byte is read once and written once.
//
// Layout: one row of D bf16 values (2D bytes) per D/8 lanes, 16 bytes each;
// a 256-thread work item moves 2048/D rows of K and as many of V (16 at head
// dim 128). Rows are ordered (sequence, kv head, token), so the reads are
// contiguous and consecutive tokens of one page land in consecutive slots. Broken metadata never turns into a
// stray write: a sequence whose context is shorter than its new tokens is
// skipped, and so is a row whose position falls past the block table or
// whose page id is not a page of the pool.

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

struct AppendArgs {
  const uint16_t* key_new;
  const uint16_t* value_new;
  uint16_t* key_pages;
  uint16_t* value_pages;
  const int32_t* block_table;
  const int32_t* context_lens;
  int64_t rows;  // batch * num_kv_heads * new_len
  int num_kv_heads, new_len, num_pages, page_size, ps_log2, max_pages;
  int dv;  // row length in elements (<= D; lanes past it copy nothing)
};

// D/8 lanes copy one row of dv <= D bf16 values (16 bytes each; a head dim
// that is not 64, 128 or 256 runs the next larger instance with its last
// lanes idle).
template <int D>
__global__ void __launch_bounds__(kThreads) pa_kv_append(AppendArgs a) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerItem = kThreads / kLanesPerRow;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerItem + threadIdx.x / kLanesPerRow;
  if (row >= a.rows) return;
  const int chunk = threadIdx.x % kLanesPerRow;
  if (chunk * 8 >= a.dv) return;
  // row -> (sequence b, head h, token l); the same for every lane of the
  // launch, the branch takes 32-bit division (a few instructions, not the
  // long 64-bit sequence) whenever the row count fits
  int l, h, b;
  if (a.rows <= INT32_MAX) {
    const int r = (int)row;
    const int bh = r / a.new_len;
    l = r - bh * a.new_len;
    h = bh % a.num_kv_heads;
    b = bh / a.num_kv_heads;
  } else {
    const int64_t bh = row / a.new_len;
    l = (int)(row - bh * a.new_len);
    h = (int)(bh % a.num_kv_heads);
    b = (int)(bh / a.num_kv_heads);
  }
  int ctx = a.context_lens[b];
  // the new rows are loaded right after the context length: their addresses
  // need no metadata (every row below `rows` is in the inputs), so the loads
  // overlap the two dependent metadata reads instead of following them, and
  // waiting for the context length (issued first; loads complete in order)
  // does not wait for them. The empty asm statement emits no instruction: as a
  // compiler memory barrier it keeps the loads above it (otherwise they sink
  // below the metadata checks, the only path that uses them), and taking the
  // context length as an operand puts its wait after both loads are issued.
  const size_t src = (size_t)row * a.dv + chunk * 8;
  const u32x4_t k = *reinterpret_cast<const u32x4_t*>(a.key_new + src);
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.value_new + src);
  asm volatile("" : "+v"(ctx) : : "memory");
  if (ctx < a.new_len) return;  // the sequence cannot hold its new tokens: none is written
  const int s = ctx - a.new_len + l;
  const int lp = a.ps_log2 >= 0 ? (s >> a.ps_log2) : s / a.page_size;
  if (lp >= a.max_pages) return;
  const int32_t page = a.block_table[(size_t)b * a.max_pages + lp];
  if (page < 0 || page >= a.num_pages) return;
  const int slot = s - lp * a.page_size;
  const size_t dst = (((size_t)page * a.num_kv_heads + h) * a.page_size + slot) * a.dv + chunk * 8;
  // The page rows are written once here and read by a later attention
  // launch, not by this one: non-temporal stores (the streaming hint) let them
  // drain to HBM without holding cache lines (measured 14.2 -> 11.8 us for
  // 64 MiB of K/V; the same hint on the loads gave nothing).
  __builtin_nontemporal_store(k, reinterpret_cast<u32x4_t*>(a.key_pages + dst));
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(a.value_pages + dst));
}

template <int D>
hipError_t launch_dim(const AppendArgs& a, hipStream_t stream) {
  constexpr int kRowsPerItem = kThreads / (D / 8);
  const int64_t items = (a.rows + kRowsPerItem - 1) / kRowsPerItem;
  hipLaunchKernelGGL(pa_kv_append<D>, dim3((unsigned)items), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendKernelArgs& k, hipStream_t stream) {
  AppendArgs a;
  a.key_new = static_cast<const uint16_t*>(k.key_new);
  a.value_new = static_cast<const uint16_t*>(k.value_new);
  a.key_pages = static_cast<uint16_t*>(k.key_pages);
  a.value_pages = static_cast<uint16_t*>(k.value_pages);
  a.block_table = k.block_table;
  a.context_lens = k.context_lens;
  a.rows = (int64_t)k.batch * k.num_kv_heads * k.new_len;
  a.num_kv_heads = k.num_kv_heads;
  a.new_len = k.new_len;
  a.num_pages = k.num_pages;
  a.page_size = k.page_size;
  a.ps_log2 = -1;
  for (int e = 0; e < 31; ++e)
    if ((1 << e) == k.page_size) a.ps_log2 = e;
  a.max_pages = k.max_pages;
  a.dv = k.head_dim;
  switch (instance_dim(k.head_dim)) {
    case 64: return launch_dim<64>(a, stream);
    case 256: return launch_dim<256>(a, stream);
    default: return launch_dim<128>(a, stream);
  }
}

}  // namespace pa
