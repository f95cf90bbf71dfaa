// compact.hip - KV-slot compaction of one request (Tier 1 defragmentation).
//
// "The Execution Phase" (section "Tier 0 KV Defragmentation") names the next
// tier: live relocation of a request's fragmented page_size=1 KV slots under
// a copy budget; "The Architecture Detective" (section "Deconstructing the
// K/V Defrag Hypothesis") describes it as moving a request's KV entries to
// contiguous slots so that its rows are read as one run.  The pages leave
// the policy open; this file implements the plainest one:
//
//   Logical position k of the request's slot table belongs at slot
//   dst_begin + k of a free run the caller reserved.  Walking k upward, every
//   row not yet at its place is copied there and its table entry rewritten,
//   until `budget` rows have been copied.  Rows already in place are not
//   copied and do not count against the budget.
//
// Four launches on one stream, all sized from n and budget (so the step can
// be captured in a HIP graph): per-block counts of rows that need a move and
// precondition checks; one block that scans the counts; per-block
// compaction of the selected (position, source slot) pairs; and the copy,
// one 16-byte piece per thread, 72 pieces per 1152-byte row.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "verify_attn.h"

namespace {

constexpr int CB = 1024;           // table entries per block of the count/select passes
constexpr int ROW_PIECES = VA_D_QK * 2 / 16;   // 72 pieces of 16 bytes per row
constexpr int COPY_THREADS = 256;
typedef uint32_t vec4u __attribute__((ext_vector_type(4)));

// Arguments of the compaction kernels besides the leading ones (CompactLead
// below): the table [n] (read through CompactLead::table, rewritten by the
// copy through table_w), n, dst_begin, budget, nblocks = ceil(n / CB),
// block_need / block_bad [nblocks] (rows of each block that need a move, its
// precondition bits), result [2] (rows to copy or -bits on failure, total
// bits) and num_slots come there.
struct CompactArgs {
  uint16_t* kv;
  int32_t stride;          // bf16 elements between rows
  int32_t* table_w;        // the table, for the copy's rewrite of moved entries
  int32_t* block_off;      // [nblocks] exclusive prefix of block_need
  int32_t* sel_pos;        // [budget] logical positions to move, in order
  int32_t* sel_src;        // [budget] their current slots
  int32_t* copied;         // caller's device int: the same count / -bits
};

// The arguments the kernels' first loads need.  Every compaction kernel takes
// them as leading scalar parameters (COMPACT_LEAD), which the library's build
// preloads into scalar registers, so those loads need no kernel-argument load
// first; the rest come in CompactArgs.
struct CompactLead {
  const int32_t* table;
  int32_t* block_need;
  uint32_t* block_bad;
  int32_t* result;
  int64_t num_slots;
  int32_t n;
  int32_t dst_begin;
  int32_t nblocks;
  int32_t budget;
};
#define COMPACT_LEAD                                                                        \
  const int32_t *table, int32_t *block_need, uint32_t *block_bad, int32_t *result,         \
      int64_t num_slots, int32_t n, int32_t dst_begin, int32_t nblocks, int32_t budget
#define COMPACT_LEAD_INIT \
  const CompactLead l{table, block_need, block_bad, result, num_slots, n, dst_begin, nblocks, budget}

// needs[k]: table[k] != dst_begin + k.  Precondition bits: a slot outside the
// pool, or a slot inside the destination run but not at its own place (its
// row could be overwritten before it is read).
__device__ __forceinline__ void classify(const CompactLead& a, int k, bool* need, uint32_t* bad) {
  const int32_t sl = a.table[k];
  *need = sl != a.dst_begin + k;
  uint32_t b = 0u;
  if (sl < 0 || (int64_t)sl >= a.num_slots) b |= VA_COMPACT_BAD_SLOT;
  const int64_t rel = (int64_t)sl - a.dst_begin;
  if (rel >= 0 && rel < a.n && rel != k) b |= VA_COMPACT_RUN_OCCUPIED;
  *bad = b;
}

__global__ __launch_bounds__(CB) void compact_count_kernel(COMPACT_LEAD) {
  COMPACT_LEAD_INIT;
  __shared__ int cnt[CB / 64];
  __shared__ uint32_t bb[CB / 64];
  const int k = blockIdx.x * CB + threadIdx.x;
  bool need = false;
  uint32_t bad = 0u;
  if (k < l.n) classify(l, k, &need, &bad);
  const uint64_t m = __ballot(need);
  uint32_t wb = bad;
  for (int o = 32; o >= 1; o >>= 1) wb |= __shfl_xor(wb, o);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    cnt[wave] = __popcll(m);
    bb[wave] = wb;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0;
    uint32_t b = 0u;
    for (int i = 0; i < CB / 64; ++i) {
      c += cnt[i];
      b |= bb[i];
    }
    l.block_need[blockIdx.x] = c;
    l.block_bad[blockIdx.x] = b;
  }
}

// One block: exclusive scan of the per-block counts (sequential over
// waves of 1024), the number of rows to copy and the precondition bits.
__global__ __launch_bounds__(1024) void compact_scan_kernel(COMPACT_LEAD, CompactArgs a) {
  COMPACT_LEAD_INIT;
  __shared__ int part[1024];
  __shared__ uint32_t bits[1024];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  uint32_t b_all = 0u;
  __syncthreads();
  for (int base = 0; base < l.nblocks; base += 1024) {
    const int i = base + threadIdx.x;
    const int v = i < l.nblocks ? l.block_need[i] : 0;
    b_all |= i < l.nblocks ? l.block_bad[i] : 0u;
    part[threadIdx.x] = v;
    __syncthreads();
    // Hillis-Steele inclusive scan over the 1024 entries
    for (int o = 1; o < 1024; o <<= 1) {
      const int add = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < l.nblocks) a.block_off[i] = carry + part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
  bits[threadIdx.x] = b_all;
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
    if (threadIdx.x < o) bits[threadIdx.x] |= bits[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const uint32_t b = bits[0];
    const int todo = carry < l.budget ? carry : l.budget;
    l.result[0] = b ? -(int)b : todo;
    l.result[1] = (int)b;
    *a.copied = l.result[0];
  }
}

// The selected (position, slot) pairs in logical order: entry k that needs a
// move has rank block_off + (needing entries before it in its block).
__global__ __launch_bounds__(CB) void compact_select_kernel(COMPACT_LEAD, CompactArgs a) {
  COMPACT_LEAD_INIT;
  __shared__ int wcnt[CB / 64];
  if (l.result[0] <= 0) return;
  const int k = blockIdx.x * CB + threadIdx.x;
  bool need = false;
  uint32_t bad = 0u;
  if (k < l.n) classify(l, k, &need, &bad);
  const uint64_t m = __ballot(need);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (lane == 0) wcnt[wave] = __popcll(m);
  __syncthreads();
  int before = a.block_off[blockIdx.x];
  for (int i = 0; i < wave; ++i) before += wcnt[i];
  const int rank = before + __popcll(m & ((1ull << lane) - 1ull));
  if (need && rank < l.result[0]) {
    a.sel_pos[rank] = k;
    a.sel_src[rank] = l.table[k];
  }
}

// The same selection without the scan launch, for tables of at most CB
// count blocks: every block reduces the (at most CB) per-block counts itself
// to its own offset, the total and the precondition bits; block 0 publishes
// the result.
__global__ __launch_bounds__(CB) void compact_select_fused_kernel(COMPACT_LEAD, CompactArgs a) {
  COMPACT_LEAD_INIT;
  __shared__ int w_before[CB / 64];
  __shared__ int w_total[CB / 64];
  __shared__ uint32_t w_bits[CB / 64];
  __shared__ int wcnt[CB / 64];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  // this thread's count block (nblocks <= CB)
  const int cnt = t < l.nblocks ? l.block_need[t] : 0;
  const uint32_t cbad = t < l.nblocks ? l.block_bad[t] : 0u;
  int before = t < (int)blockIdx.x ? cnt : 0;
  int total = cnt;
  uint32_t bits = cbad;
  for (int o = 32; o >= 1; o >>= 1) {
    before += __shfl_xor(before, o);
    total += __shfl_xor(total, o);
    bits |= __shfl_xor(bits, o);
  }
  if (lane == 0) {
    w_before[wave] = before;
    w_total[wave] = total;
    w_bits[wave] = bits;
  }
  __syncthreads();
  int off = 0, tot = 0;
  uint32_t b = 0u;
  for (int i = 0; i < CB / 64; ++i) {
    off += w_before[i];
    tot += w_total[i];
    b |= w_bits[i];
  }
  const int todo = b ? -(int)b : (tot < l.budget ? tot : l.budget);
  if (blockIdx.x == 0 && t == 0) {
    l.result[0] = todo;
    l.result[1] = (int)b;
    *a.copied = todo;
  }
  if (todo <= 0) return;
  const int k = blockIdx.x * CB + t;
  bool need = false;
  uint32_t bad = 0u;
  if (k < l.n) classify(l, k, &need, &bad);
  const uint64_t m = __ballot(need);
  if (lane == 0) wcnt[wave] = __popcll(m);
  __syncthreads();
  for (int i = 0; i < wave; ++i) off += wcnt[i];
  const int rank = off + __popcll(m & ((1ull << lane) - 1ull));
  if (need && rank < todo) {
    a.sel_pos[rank] = k;
    a.sel_src[rank] = l.table[k];
  }
}

// Copy piece p of selected row i (thread i * 72 + p), then rewrite the table
// entry.  The copy reads only sel_src, never the table it rewrites.
__global__ __launch_bounds__(COPY_THREADS) void compact_copy_kernel(COMPACT_LEAD, CompactArgs a) {
  COMPACT_LEAD_INIT;
  const int todo = l.result[0];
  const int64_t t = (int64_t)blockIdx.x * COPY_THREADS + threadIdx.x;
  const int64_t i = t / ROW_PIECES;
  const int p = (int)(t - i * ROW_PIECES);
  if (todo <= 0 || i >= todo) return;
  const int32_t k = a.sel_pos[i];
  const int64_t src = a.sel_src[i];
  const int64_t dst = (int64_t)l.dst_begin + k;
  // streaming: each source row is read once and each destination written once
  const vec4u v = __builtin_nontemporal_load(reinterpret_cast<const vec4u*>(a.kv + src * a.stride + p * 8));
  __builtin_nontemporal_store(v, reinterpret_cast<vec4u*>(a.kv + dst * a.stride + p * 8));
  if (p == 0) a.table_w[k] = (int32_t)dst;
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

struct CompactLayout {
  int64_t need, off, bad, pos, src, result, total;
};

int32_t compact_blocks(int32_t n) {   // blocks of the count/select passes (>= 1)
  const int64_t nb = ((int64_t)n + CB - 1) / CB;
  return (int32_t)(nb > 0 ? nb : 1);
}

CompactLayout compact_layout(int32_t n, int32_t budget) {
  const int64_t nb = compact_blocks(n);
  CompactLayout l;
  l.need = 0;
  l.off = l.need + align256(nb * 4);
  l.bad = l.off + align256(nb * 4);
  l.pos = l.bad + align256(nb * 4);
  l.src = l.pos + align256((int64_t)budget * 4);
  l.result = l.src + align256((int64_t)budget * 4);
  l.total = l.result + 256;
  return l;
}

}  // namespace

extern "C" {

size_t verify_attn_compact_workspace_bytes(int32_t n, int32_t budget) {
  if (n < 0 || budget < 0) return 0;
  return (size_t)compact_layout(n, budget).total;
}

int verify_attn_compact(uint16_t* kv_pool, int64_t num_slots, int32_t kv_row_stride,
                        int32_t* slot_table, int32_t n, int32_t dst_begin, int32_t budget,
                        void* workspace, size_t workspace_bytes, int32_t* copied,
                        va_stream_t stream) {
  if (kv_pool == nullptr || (slot_table == nullptr && n > 0) || workspace == nullptr ||
      copied == nullptr)
    return VA_ERR_NULL;
  if (n < 0 || budget < 0 || num_slots < 1 || num_slots > (int64_t)INT32_MAX + 1 ||
      kv_row_stride < VA_D_QK || dst_begin < 0 || (int64_t)dst_begin + n > num_slots)
    return VA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(kv_pool) & 15u) != 0 || (kv_row_stride % 8) != 0)
    return VA_ERR_ALIGN;
  const CompactLayout l = compact_layout(n, budget);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || (int64_t)workspace_bytes < l.total)
    return VA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const int32_t nblocks = compact_blocks(n);
  int32_t* const block_need = reinterpret_cast<int32_t*>(ws + l.need);
  uint32_t* const block_bad = reinterpret_cast<uint32_t*>(ws + l.bad);
  int32_t* const result = reinterpret_cast<int32_t*>(ws + l.result);
  CompactArgs a;
  a.kv = kv_pool;
  a.stride = kv_row_stride;
  a.table_w = slot_table;
  a.block_off = reinterpret_cast<int32_t*>(ws + l.off);
  a.sel_pos = reinterpret_cast<int32_t*>(ws + l.pos);
  a.sel_src = reinterpret_cast<int32_t*>(ws + l.src);
  a.copied = copied;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned nb = (unsigned)nblocks;
#define VA_LEAD slot_table, block_need, block_bad, result, num_slots, n, dst_begin, nblocks, budget
  hipLaunchKernelGGL(compact_count_kernel, dim3(nb), dim3(CB), 0, st, VA_LEAD);
  if (nb <= CB) {   // every block can reduce the counts itself: no scan launch
    hipLaunchKernelGGL(compact_select_fused_kernel, dim3(nb), dim3(CB), 0, st, VA_LEAD, a);
  } else {
    hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(1024), 0, st, VA_LEAD, a);
    hipLaunchKernelGGL(compact_select_kernel, dim3(nb), dim3(CB), 0, st, VA_LEAD, a);
  }
  const int64_t threads = (int64_t)budget * ROW_PIECES;
  const unsigned copy_blocks = (unsigned)((threads + COPY_THREADS - 1) / COPY_THREADS);
  if (copy_blocks > 0)
    hipLaunchKernelGGL(compact_copy_kernel, dim3(copy_blocks), dim3(COPY_THREADS), 0, st, VA_LEAD, a);
#undef VA_LEAD
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

}  // extern "C"
