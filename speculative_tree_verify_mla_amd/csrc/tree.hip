// tree.hip - draft-tree marshaling on the GPU.
//
// The verify call needs, per request, the draft nodes in an order where every
// parent precedes its children, the parent array in that order, and the
// slot-table entries of the draft tokens after the prefix.  The pages build
// the tree and its mask on the host ("The Execution Phase", section "The
// Methodology: Evidence-Driven Engineering": tree build 1.8 ms and mask build
// 0.18 ms of CPU time per step); doing it on the device keeps the whole
// verify step inside one HIP graph.
//
// Input per request r (T_r <= 64 nodes): raw_parent[j] in [-1, T_r) for raw
// node j in any order (-1: attached to the prefix), and raw_slot[j], the pool
// slot holding node j's KV row.  Output, in verify order = sorted by (depth,
// raw index) (breadth first, so parents come first):
//   perm[i]       raw node at verify position i
//   parent[i]     verify position of its parent, or -1
//   anc[i]        bit k set iff verify node k is i or an ancestor of i
//   slot_table[slot_indptr[r] + prefix_len[r] + i] = raw_slot[perm[i]]
// One wave per request, lane j = raw node j.  A parent outside [-1, T_r) or
// a cycle sets the request's status bit (VA_TREE_BAD_PARENT); its outputs are
// then unspecified, and nothing is written outside the request's own ranges.
//
// permute_rows_kernel then gathers per-node rows (the queries, H x 576 bf16
// per node) from raw order into verify order through perm;
// build_tree_rows_kernel does both in one launch.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "verify_attn.h"

namespace {

typedef uint32_t vec4u __attribute__((ext_vector_type(4)));

// The rest of the arguments (the inputs come as leading scalar parameters).
struct TreeArgs {
  int32_t* slot_table;
  int32_t slot_table_len;
  int32_t* perm;               // [sum T_r]
  int32_t* parent;             // [sum T_r]
  uint64_t* anc;               // [sum T_r]
  uint32_t* status;            // [B]
  int32_t tree_begin[VA_MAX_REQUESTS + 1];
};

// Verify position of raw node `lane` of a request (one 64-lane wave, lane j =
// raw node j, live = j < T): the rank of (depth, raw index) among the live
// nodes.  p is the node's parent (lane) after the range check, -1 for a
// root; bad gets VA_TREE_BAD_PARENT for a parent outside [-1, T) or a cycle.
// Depth comes from walking up the chains through the wave: every lane holds
// its node's parent (one load), and a walk still going after 64 steps (more
// than T) is a cycle.
struct TreeRank {
  int p;
  int rank;
  uint32_t bad;
};
__device__ __forceinline__ TreeRank tree_rank(int p, bool live, int T, int lane) {
  TreeRank tr;
  tr.bad = 0u;
  if (live && (p < -1 || p >= T)) {
    tr.bad = VA_TREE_BAD_PARENT;
    p = -1;
  }
  int depth = 0;
  {
    int x = p;
    for (int step = 0; step < VA_MAX_TREE && __any(x >= 0); ++step) {   // uniform
      const int nx = __shfl(p, x >= 0 ? x : 0);
      if (x >= 0) {
        ++depth;
        x = nx;
      }
    }
    if (x >= 0) tr.bad = VA_TREE_BAD_PARENT;
  }
  // rank: the live nodes at a smaller depth, plus those at the same depth
  // with a smaller raw index, one ballot per depth level (depths are at most
  // 64, so the loop ends by then even for a cycle)
  const uint64_t below = lane == 0 ? 0ull : ~0ull >> (64 - lane);
  const int n_live = __popcll(__ballot(live));
  int rank = 0;
  int counted = 0;
  for (int d = 0; d <= VA_MAX_TREE && counted < n_live; ++d) {   // uniform
    const uint64_t at = __ballot(live && depth == d);
    if (depth > d) rank += __popcll(at);
    else if (depth == d) rank += __popcll(at & below);
    counted += __popcll(at);
  }
  tr.p = p;
  tr.rank = rank;
  return tr;
}

// Request r's tree, on one 64-lane wave (lane = raw node).
template <bool ONE>
__device__ __forceinline__ void build_tree_body(const int32_t* raw_parent, const int32_t* raw_slot,
                                                const int32_t* prefix_len,
                                                const int32_t* slot_indptr, int r, int t_first,
                                                const TreeArgs& a, int lane) {
  const int t0 = ONE ? 0 : a.tree_begin[r];
  const int T = ONE ? t_first : a.tree_begin[r + 1] - t0;
  const bool live = lane < T;

  // every load up front: the walk, the ranking and the table write then need
  // no further round trip to memory
  const int p_raw = live ? raw_parent[t0 + lane] : -1;
  const int32_t my_slot = live ? raw_slot[t0 + lane] : 0;
  const int32_t tab_base = slot_indptr[r];
  const int64_t tab_lo = (int64_t)tab_base + prefix_len[r];
  const int32_t tab_hi = slot_indptr[r + 1];
  const TreeRank tr = tree_rank(p_raw, live, T, lane);
  const int p = tr.p;
  const int rank = tr.rank;
  uint32_t bad = tr.bad;
  const int prank = __shfl(rank, p < 0 ? 0 : p);
  // ancestor mask in verify positions: walk the chain again, mapping raw ids
  // to verify positions through the wave (every lane takes part in the
  // shuffles; lanes with x = -1 idle; the walk stops when every chain ended)
  uint64_t m = 0ull;
  {
    int x = (live && bad == 0u) ? lane : -1;
    for (int step = 0; step < VA_MAX_TREE && __any(x >= 0); ++step) {   // uniform
      const int rx = __shfl(rank, x < 0 ? 0 : x);
      const int nx = __shfl(p, x < 0 ? 0 : x);
      if (x >= 0) {
        m |= 1ull << (rx & 63);
        x = nx;
      }
    }
  }
  if (live) {
    const int o = t0 + rank;
    a.perm[o] = lane;
    a.parent[o] = p < 0 ? -1 : prank;
    a.anc[o] = m;
    const int64_t e = tab_lo + rank;
    // only inside the request's own range [slot_indptr[r], slot_indptr[r+1]):
    // a negative device prefix length must not reach the previous request
    if (e >= 0 && e >= tab_base && e < a.slot_table_len && e < tab_hi)
      a.slot_table[e] = my_slot;
    else
      bad |= VA_TREE_BAD_TABLE;
  }
  uint32_t bits = bad;
  for (int o = 32; o >= 1; o >>= 1) bits |= __shfl_xor(bits, o);
  if (lane == 0) a.status[r] = bits;
}

// The inputs of the first loads come as leading scalar parameters, which the
// library's build preloads into scalar registers (no kernel-argument load
// before them); ONE (a single request) also takes its node count from there.
template <bool ONE>
__global__ __launch_bounds__(64) void build_tree_kernel(const int32_t* raw_parent,
                                                        const int32_t* raw_slot,
                                                        const int32_t* prefix_len,
                                                        const int32_t* slot_indptr,
                                                        int32_t num_requests, int32_t t_first,
                                                        TreeArgs a) {
  const int r = blockIdx.x;
  if (r >= num_requests) return;
  build_tree_body<ONE>(raw_parent, raw_slot, prefix_len, slot_indptr, r, t_first, a, threadIdx.x);
}

// dst row t0 + i = src row t0 + perm[t0 + i]: block (x, R) copies 16-byte
// pieces 256 x .. 256 x + 255 of verify row R.  Pointers and sizes come as
// leading (preloaded) arguments; ONE (a single request) needs no table.
struct PermuteArgs {
  int32_t num_requests;
  int32_t tree_begin[VA_MAX_REQUESTS + 1];
};
constexpr int PERMUTE_THREADS = 256;

template <bool ONE>
__global__ __launch_bounds__(PERMUTE_THREADS) void permute_rows_kernel(
    const int32_t* perm, const vec4u* src, vec4u* dst, int64_t pieces, int32_t t_first,
    PermuteArgs a) {
  const int R = blockIdx.y;
  const int64_t p = (int64_t)blockIdx.x * PERMUTE_THREADS + threadIdx.x;
  if (p >= pieces) return;
  int t0 = 0, T = t_first;
  if (!ONE) {
    int r = 0;
    while (r + 1 < a.num_requests && a.tree_begin[r + 1] <= R) ++r;
    t0 = a.tree_begin[r];
    T = a.tree_begin[r + 1] - t0;
  }
  const int j = perm[R];
  vec4u v = {0u, 0u, 0u, 0u};
  // each source row is read once
  if (j >= 0 && j < T) v = __builtin_nontemporal_load(src + (int64_t)(t0 + j) * pieces + p);
  dst[(int64_t)R * pieces + p] = v;
}

// Tree and row gather in one launch: blocks 0 .. B-1 build request b's tree
// (wave 0, as build_tree_kernel); block B + x R + c gathers pieces
// 256 c .. 256 c + 255 of verify row R (x blocks per row).  A gather block
// needs the raw node at its verify position, so each of its waves ranks its
// request's nodes again (the same tree_rank, on the same parent loads)
// instead of waiting for the tree blocks: nothing passes between blocks.
// The leading (preloaded) parameters are what a gather block needs first.
template <bool ONE>
__global__ __launch_bounds__(PERMUTE_THREADS) void build_tree_rows_kernel(
    const int32_t* raw_parent, const int32_t* raw_slot, const int32_t* prefix_len,
    const int32_t* slot_indptr, int32_t num_requests, int32_t xblocks, int32_t t_first,
    int64_t pieces, const vec4u* src, vec4u* dst, TreeArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  if (b < num_requests) {
    if (threadIdx.x < 64) build_tree_body<ONE>(raw_parent, raw_slot, prefix_len, slot_indptr, b,
                                               t_first, a, lane);
    return;
  }
  const int g = b - num_requests;
  const int R = g / xblocks;   // verify row
  const int c = g - R * xblocks;
  int r = 0;
  if (!ONE)
    while (r + 1 < num_requests && a.tree_begin[r + 1] <= R) ++r;
  const int t0 = ONE ? 0 : a.tree_begin[r];
  const int T = ONE ? t_first : a.tree_begin[r + 1] - t0;
  const bool live = lane < T;
  const TreeRank tr = tree_rank(live ? raw_parent[t0 + lane] : -1, live, T, lane);
  // the raw node ranked at position R - t0 (none, in a flagged request,
  // gives a row of zeros)
  const uint64_t at = __ballot(live && tr.rank == R - t0);
  const int j = at ? __builtin_ctzll(at) : -1;
  const int64_t p = (int64_t)c * PERMUTE_THREADS + threadIdx.x;
  if (p >= pieces) return;
  vec4u v = {0u, 0u, 0u, 0u};
  // each source row is read once
  if (j >= 0) v = __builtin_nontemporal_load(src + (int64_t)(t0 + j) * pieces + p);
  dst[(int64_t)R * pieces + p] = v;
}

// Plan checks shared by the tree entry points: the kernels index the
// caller's arrays through tree_begin, which must start at 0 and step by each
// request's tree size, as the planner writes it.
bool tree_plan_ok(const va_plan* plan) {
  if (plan->magic != VA_PLAN_MAGIC || plan->version != VA_PLAN_VERSION ||
      plan->num_requests < 1 || plan->num_requests > VA_MAX_REQUESTS || plan->tree_begin[0] != 0 ||
      plan->total_tree != plan->tree_begin[plan->num_requests] || plan->total_tree < 1)
    return false;
  for (int r = 0; r < plan->num_requests; ++r)
    if (plan->num_tree[r] < 1 || plan->num_tree[r] > VA_MAX_TREE ||
        plan->tree_begin[r + 1] - plan->tree_begin[r] != plan->num_tree[r])
      return false;
  return true;
}

}  // namespace

extern "C" {

int verify_attn_build_tree(const va_plan* plan, const int32_t* raw_parent, const int32_t* raw_slot,
                           const int32_t* prefix_len, const int32_t* slot_indptr,
                           int32_t* slot_table, int32_t slot_table_len, int32_t* perm,
                           int32_t* parent, uint64_t* anc, uint32_t* status, va_stream_t stream) {
  if (plan == nullptr || raw_parent == nullptr || raw_slot == nullptr || prefix_len == nullptr ||
      slot_indptr == nullptr || slot_table == nullptr || perm == nullptr || parent == nullptr ||
      anc == nullptr || status == nullptr)
    return VA_ERR_NULL;
  if (!tree_plan_ok(plan)) return VA_ERR_PLAN;
  if (slot_table_len < 0) return VA_ERR_SHAPE;
  TreeArgs a;
  a.slot_table = slot_table;
  a.slot_table_len = slot_table_len;
  a.perm = perm;
  a.parent = parent;
  a.anc = anc;
  a.status = status;
  for (int r = 0; r <= plan->num_requests; ++r) a.tree_begin[r] = plan->tree_begin[r];
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan->num_requests == 1)
    hipLaunchKernelGGL(build_tree_kernel<true>, dim3(1), dim3(64), 0, st, raw_parent, raw_slot,
                       prefix_len, slot_indptr, plan->num_requests, plan->num_tree[0], a);
  else
    hipLaunchKernelGGL(build_tree_kernel<false>, dim3(plan->num_requests), dim3(64), 0, st,
                       raw_parent, raw_slot, prefix_len, slot_indptr, plan->num_requests,
                       plan->num_tree[0], a);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

int verify_attn_permute_rows(const va_plan* plan, const int32_t* perm, const uint16_t* src,
                             uint16_t* dst, int64_t row_elems, va_stream_t stream) {
  if (plan == nullptr || perm == nullptr || src == nullptr || dst == nullptr) return VA_ERR_NULL;
  if (!tree_plan_ok(plan)) return VA_ERR_PLAN;
  if (row_elems < 8 || (row_elems % 8) != 0 || row_elems > ((int64_t)1 << 40)) return VA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15u) != 0)
    return VA_ERR_ALIGN;
  const int64_t pieces = row_elems / 8;
  const int64_t xblocks = (pieces + PERMUTE_THREADS - 1) / PERMUTE_THREADS;
  if (xblocks > INT32_MAX) return VA_ERR_SHAPE;
  PermuteArgs a;
  a.num_requests = plan->num_requests;
  for (int r = 0; r <= plan->num_requests; ++r) a.tree_begin[r] = plan->tree_begin[r];
  const dim3 grid((unsigned)xblocks, (unsigned)plan->total_tree);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const vec4u* s4 = reinterpret_cast<const vec4u*>(src);
  vec4u* d4 = reinterpret_cast<vec4u*>(dst);
  if (plan->num_requests == 1)
    hipLaunchKernelGGL(permute_rows_kernel<true>, grid, dim3(PERMUTE_THREADS), 0, st, perm, s4, d4,
                       pieces, plan->num_tree[0], a);
  else
    hipLaunchKernelGGL(permute_rows_kernel<false>, grid, dim3(PERMUTE_THREADS), 0, st, perm, s4,
                       d4, pieces, plan->num_tree[0], a);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

int verify_attn_build_tree_rows(const va_plan* plan, const int32_t* raw_parent,
                                const int32_t* raw_slot, const int32_t* prefix_len,
                                const int32_t* slot_indptr, int32_t* slot_table,
                                int32_t slot_table_len, int32_t* perm, int32_t* parent,
                                uint64_t* anc, uint32_t* status, const uint16_t* src,
                                uint16_t* dst, int64_t row_elems, va_stream_t stream) {
  if (plan == nullptr || raw_parent == nullptr || raw_slot == nullptr || prefix_len == nullptr ||
      slot_indptr == nullptr || slot_table == nullptr || perm == nullptr || parent == nullptr ||
      anc == nullptr || status == nullptr || src == nullptr || dst == nullptr)
    return VA_ERR_NULL;
  if (!tree_plan_ok(plan)) return VA_ERR_PLAN;
  if (slot_table_len < 0) return VA_ERR_SHAPE;
  if (row_elems < 8 || (row_elems % 8) != 0 || row_elems > ((int64_t)1 << 40)) return VA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15u) != 0)
    return VA_ERR_ALIGN;
  const int64_t pieces = row_elems / 8;
  const int64_t xblocks = (pieces + PERMUTE_THREADS - 1) / PERMUTE_THREADS;
  const int64_t blocks = plan->num_requests + xblocks * plan->total_tree;
  if (blocks > INT32_MAX) return VA_ERR_SHAPE;
  TreeArgs a;
  a.slot_table = slot_table;
  a.slot_table_len = slot_table_len;
  a.perm = perm;
  a.parent = parent;
  a.anc = anc;
  a.status = status;
  for (int r = 0; r <= plan->num_requests; ++r) a.tree_begin[r] = plan->tree_begin[r];
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const vec4u* s4 = reinterpret_cast<const vec4u*>(src);
  vec4u* d4 = reinterpret_cast<vec4u*>(dst);
  if (plan->num_requests == 1)
    hipLaunchKernelGGL(build_tree_rows_kernel<true>, dim3((unsigned)blocks), dim3(PERMUTE_THREADS),
                       0, st, raw_parent, raw_slot, prefix_len, slot_indptr, plan->num_requests,
                       (int32_t)xblocks, plan->num_tree[0], pieces, s4, d4, a);
  else
    hipLaunchKernelGGL(build_tree_rows_kernel<false>, dim3((unsigned)blocks), dim3(PERMUTE_THREADS),
                       0, st, raw_parent, raw_slot, prefix_len, slot_indptr, plan->num_requests,
                       (int32_t)xblocks, plan->num_tree[0], pieces, s4, d4, a);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

}  // extern "C"
