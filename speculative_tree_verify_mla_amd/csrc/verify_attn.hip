// verify_attn.hip - tree-verify MLA attention for MI355X (gfx950, CDNA4).
//
// Split-KV partial pass + log-sum-exp reduce ("The Verify Kernel
// Breakthrough", section "The Message in Context": partial+reduce;
// "The Architecture Detective", section "The Split Verify Design": LSE
// merge), with the KV tile loaded once and shared by every head and draft
// node of a row group ("The Execution Phase", section "The Core Design: A
// Streaming Flash Attention Kernel": KV-tile outer, heads inner), 16-byte
// gathers of the page_size=1 rows (same page, section "The Optimization That
// Unlocked 3-6x Speedup": 128-bit loads) and graph-capture-safe launches
// (same page, section "Making the Kernel CUDA Graph Capture-Safe").
//
// gfx950 mapping of one work item (request r, row group g, KV split s):
//   - 256 threads = 4 wave64s; each wave owns 16 query rows (node, head).
//   - Per 32-key tile the block gathers 32 pool rows (72 x 16 B each) into
//     LDS twice: row-major K[key][576] for the score contraction and a
//     transposed V^T[col][key] (8x8 register transposes) for the value
//     contraction, so both MFMA operands are single 16-byte LDS reads.
//   - S^T[key][row] = K . Q^T on v_mfma_f32_16x16x32_bf16 (A = K tile from
//     LDS, B = the wave's Q rows held in VGPRs).  The MFMA output layout puts
//     one query row per lane (lane % 16), so the online softmax needs only
//     two cross-lane steps per tile and the probabilities are already the B
//     operand of O^T[col][row] = V^T . P^T (keys reordered consistently on
//     both operands).
//   - The tree mask is one 64-bit ancestor mask per draft node, built in the
//     prologue from parent[]; only draft positions (>= L) consult it.
//   - Each work item writes o/l (fp32) and lse (base 2) for its rows; the
//     reduce merges a row's splits and writes bf16 out and natural-log lse.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "verify_attn.h"

namespace {

constexpr int DQK = VA_D_QK;   // 576
constexpr int DV = VA_D_V;     // 512
constexpr int TILE = 32;       // keys per tile
constexpr int THREADS = 256;   // 4 waves
constexpr int ROWS = 64;       // query rows per work item (16 per wave)
constexpr int KS_STRIDE = DQK + 8;   // bf16 per K row in LDS (1168 B: conflict-free 16-row reads)
constexpr int VT_STRIDE = TILE + 8;  // bf16 per V^T row in LDS (80 B)
constexpr int QK_STEPS = DQK / 32;   // 18 MFMA k-steps for the score
constexpr int O_BLOCKS = DV / 16;    // 32 MFMA column blocks for the output
constexpr int MIN_KEYS_PER_SPLIT = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct PartialArgs {
  const uint16_t* q;
  const uint16_t* kv;
  int64_t num_slots;
  int32_t stride;
  int32_t num_requests;
  int32_t num_heads;
  float scale_log2;   // sm_scale * log2(e): scores are kept in base 2
  const int32_t* slot_table;
  int32_t slot_table_len;
  const int32_t* slot_indptr;
  const int32_t* prefix_len;
  const int32_t* parent;
  float* part_o;      // [work][ROWS][DV]
  float* part_lse;    // [work][ROWS]
  uint32_t* status;   // [work]
  int32_t num_tree[VA_MAX_REQUESTS];
  int32_t max_prefix[VA_MAX_REQUESTS];
  int32_t nsplit[VA_MAX_REQUESTS];
  int32_t tree_begin[VA_MAX_REQUESTS + 1];
  int32_t work_begin[VA_MAX_REQUESTS + 1];
};

struct ReduceArgs {
  const float* part_o;
  const float* part_lse;
  const uint32_t* status;
  uint16_t* out;
  float* lse;
  int32_t num_requests;
  int32_t num_heads;
  int32_t nsplit[VA_MAX_REQUESTS];
  int32_t tree_begin[VA_MAX_REQUESTS + 1];
  int32_t work_begin[VA_MAX_REQUESTS + 1];
};

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// One 16-byte piece (8 bf16 columns starting at col8*8) of pool row `slot`.
// Slots outside the pool are never dereferenced: *ok is cleared and zeros
// are returned.
__device__ __forceinline__ u32x4 gather16(const uint16_t* __restrict__ kv, int64_t num_slots,
                                          int32_t stride, int32_t slot, int col8, bool* ok) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (slot >= 0 && (int64_t)slot < num_slots) {
    v = *reinterpret_cast<const u32x4*>(kv + (int64_t)slot * stride + col8 * 8);
  } else {
    *ok = false;
  }
  return v;
}

// Key of a tile that loader quad kq stages as its j-th row (j = 0..7).  The
// same order is the key order of the value contraction: V^T slot 8*kq + j
// holds this key, and the lane group kq of the score MFMA output holds keys
// 4*kq + i (first 16-key block) and 16 + 4*kq + i (second block).
__device__ __forceinline__ int stage_key(int kq, int j) {
  return j < 4 ? 4 * kq + j : 16 + 4 * kq + (j - 4);
}

__global__ __launch_bounds__(THREADS, 1) void va_partial_kernel(PartialArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[TILE * KS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t vt[DV * VT_STRIDE];
  __shared__ uint64_t anc[VA_MAX_TREE];
  __shared__ uint32_t status_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 15;   // MFMA column index: this lane's query row
  const int lgrp = lane >> 4;   // MFMA k-group of this lane
  const int w = blockIdx.x;

  // ---- decode the work item: request r, row group g, split s
  int r = 0;
  while (r + 1 < a.num_requests && a.work_begin[r + 1] <= w) ++r;
  const int ns = a.nsplit[r];
  const int local = w - a.work_begin[r];
  const int g = local / ns;
  const int s = local - g * ns;
  const int T = a.num_tree[r];
  const int H = a.num_heads;
  const int rows_r = T * H;

  if (tid == 0) status_sh = 0u;
  __syncthreads();

  uint32_t st = 0u;
  int L = a.prefix_len[r];
  if (L < 0 || L > a.max_prefix[r]) {
    st |= VA_STATUS_BAD_PREFIX;
    L = L < 0 ? 0 : a.max_prefix[r];
  }
  const int n = L + T;
  const int tab0 = a.slot_indptr[r];
  const int tab1 = a.slot_indptr[r + 1];
  int n_read = n;   // keys whose table entry exists
  if (tab0 < 0 || tab1 < tab0 || tab1 > a.slot_table_len || tab1 - tab0 < n) {
    st |= VA_STATUS_SHORT_TABLE;
    n_read = (tab0 < 0 || tab1 < tab0 || tab0 >= a.slot_table_len)
                 ? 0 : min(tab1, a.slot_table_len) - tab0;
  }
  const int chunk = ((n + ns - 1) / ns + TILE - 1) / TILE * TILE;
  const int k0 = s * chunk;
  const int k1 = min(n, k0 + chunk);

  // ---- ancestor masks (bit j of anc[i]: draft node j is i or an ancestor of i)
  if (tid < VA_MAX_TREE) {
    uint64_t m = 0;
    if (tid < T) {
      const int32_t* par = a.parent + a.tree_begin[r];
      int x = tid;
      while (x != -1) {
        m |= 1ull << x;
        const int p = par[x];
        if (p < -1 || p >= x) {   // also guarantees the walk ends
          st |= VA_STATUS_BAD_PARENT;
          break;
        }
        x = p;
      }
    }
    anc[tid] = m;
  }

  // ---- this lane's query row and its Q fragment (B operand of the score MFMA)
  const int rho = g * ROWS + wave * 16 + lrow;
  const bool row_ok = rho < rows_r;
  bf16x8 qf[QK_STEPS];
  {
    const int64_t qrow = (int64_t)a.tree_begin[r] * H + (row_ok ? rho : 0);
    const uint16_t* qp = a.q + qrow * DQK + lgrp * 8;
#pragma unroll
    for (int k = 0; k < QK_STEPS; ++k) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4*>(qp + k * 32);
      qf[k] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();   // anc[] ready
  const uint64_t anc_row = row_ok ? anc[rho / H] : 0ull;

  // ---- loader roles: quad kq = tid & 3 stages 8 keys x latent block fb;
  //      every thread also stages one 16-byte rope piece.
  const int kq = tid & 3;
  const int fb = tid >> 2;        // 0..63: latent columns fb*8 .. fb*8+7
  const int rkey = tid >> 3;      // rope piece: key 0..31
  const int rcol = 64 + (tid & 7);  // 16-byte column index 64..71 (cols 512..575)
  const int32_t* table = a.slot_table + (tab0 < 0 ? 0 : tab0);

  u32x4 lat[8];
  u32x4 rope;
  bool ok = true;
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = kt + stage_key(kq, j);
      lat[j] = u32x4{0u, 0u, 0u, 0u};
      if (k < n && k < n_read) lat[j] = gather16(a.kv, a.num_slots, a.stride, table[k], fb, &ok);
    }
    const int k = kt + rkey;
    rope = u32x4{0u, 0u, 0u, 0u};
    if (k < n && k < n_read) rope = gather16(a.kv, a.num_slots, a.stride, table[k], rcol, &ok);
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x4*>(&ks[stage_key(kq, j) * KS_STRIDE + fb * 8]) = lat[j];
    *reinterpret_cast<u32x4*>(&ks[rkey * KS_STRIDE + rcol * 8]) = rope;
    // 8x8 transpose: column fb*8+c gets this quad's 8 keys in stage order.
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int d = c >> 1;
      u32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = lat[2 * e][d];
        const uint32_t y = lat[2 * e + 1][d];
        t[e] = (c & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
      }
      *reinterpret_cast<u32x4*>(&vt[(fb * 8 + c) * VT_STRIDE + kq * 8]) = t;
    }
  };

  f32x4 o[O_BLOCKS];
#pragma unroll
  for (int c = 0; c < O_BLOCKS; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max of base-2 scores of this row
  // Partial sums over this lane's keys (summed across the 4 lane groups at the
  // end): l_run of the fp32 probabilities gives the lse; lb_run of the bf16
  // probabilities that enter the value MFMA normalises the output, so the
  // output is an exact weighted average of the value rows it was built from.
  float l_run = 0.f;
  float lb_run = 0.f;

  if (k0 < k1) load_tile(k0);
  for (int kt = k0; kt < k1; kt += TILE) {
    __syncthreads();   // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (kt + TILE < k1) load_tile(kt + TILE);   // in flight during the math below

    // S^T = K . Q^T for the two 16-key blocks of the tile
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int k = 0; k < QK_STEPS; ++k) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(&ks[(kb * 16 + lrow) * KS_STRIDE + k * 32 + lgrp * 8]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[k], sacc[kb], 0, 0, 0);
      }
    }

    // mask + online softmax (base 2); lane holds 8 keys of row lrow
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kp = kt + (j < 4 ? 4 * lgrp + j : 16 + 4 * lgrp + (j - 4));
      bool vis = kp < n;
      if (kp >= L) vis = vis && ((anc_row >> ((kp - L) & 63)) & 1ull);
      sv[j] = vis ? sacc[j >> 2][j & 3] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    bf16x8 pf;
    float psum = 0.f;
    float pbsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = exp2f(sv[j] - m_use);
      const __bf16 pb = (__bf16)p;
      pf[j] = pb;
      psum += p;
      pbsum += (float)pb;
    }
    l_run = l_run * alpha + psum;
    lb_run = lb_run * alpha + pbsum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int c = 0; c < O_BLOCKS; ++c) o[c] *= alpha;
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int c = 0; c < O_BLOCKS; ++c) {
      const bf16x8 vf =
          *reinterpret_cast<const bf16x8*>(&vt[(c * 16 + lrow) * VT_STRIDE + lgrp * 8]);
      o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[c], 0, 0, 0);
    }
  }

  // ---- epilogue: normalise and store this work item's partial
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float lb_tot = lb_run + __shfl_xor(lb_run, 16);
  lb_tot += __shfl_xor(lb_tot, 32);
  const float inv = lb_tot > 0.f ? 1.f / lb_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
  if (row_ok) {
    const int64_t prow = (int64_t)w * ROWS + wave * 16 + lrow;
    float* po = a.part_o + prow * DV + lgrp * 4;
#pragma unroll
    for (int c = 0; c < O_BLOCKS; ++c) *reinterpret_cast<f32x4*>(po + c * 16) = o[c] * inv;
    if (lgrp == 0) a.part_lse[prow] = lse2;
  }
  if (!ok) st |= VA_STATUS_BAD_SLOT;
  if (st) atomicOr(&status_sh, st);
  __syncthreads();
  if (tid == 0) a.status[w] = status_sh;
}

// One block per query row: merge the row's splits by log-sum-exp.
__global__ __launch_bounds__(128) void va_reduce_kernel(ReduceArgs a) {
  const int row = blockIdx.x;   // global (node, head) row
  const int tid = threadIdx.x;  // 4 output columns each
  const int H = a.num_heads;
  int r = 0;
  while (r + 1 < a.num_requests && a.tree_begin[r + 1] * H <= row) ++r;
  const int rho = row - a.tree_begin[r] * H;
  const int g = rho / ROWS;
  const int ri = rho - g * ROWS;
  const int ns = a.nsplit[r];
  const int64_t wb = (int64_t)a.work_begin[r] + (int64_t)g * ns;

  uint32_t st = 0u;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) {
    st |= a.status[wb + s];
    M = fmaxf(M, a.part_lse[(wb + s) * ROWS + ri]);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < ns; ++s) {
      const float ls = a.part_lse[(wb + s) * ROWS + ri];
      if (ls == -INFINITY) continue;
      const float wt = exp2f(ls - M);
      wsum += wt;
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.part_o + ((wb + s) * ROWS + ri) * DV + tid * 4);
      acc += wt * v;
    }
  }
  float res[4];
  float lse_out;
  if (st != 0u) {
    res[0] = res[1] = res[2] = res[3] = NAN;
    lse_out = NAN;
  } else if (wsum > 0.f) {
    const float inv = 1.f / wsum;
    res[0] = acc[0] * inv; res[1] = acc[1] * inv; res[2] = acc[2] * inv; res[3] = acc[3] * inv;
    lse_out = (M + log2f(wsum)) * LN2;
  } else {
    res[0] = res[1] = res[2] = res[3] = 0.f;
    lse_out = -INFINITY;
  }
  uint32_t lo = (uint32_t)f32_to_bf16_rne(res[0]) | ((uint32_t)f32_to_bf16_rne(res[1]) << 16);
  uint32_t hi = (uint32_t)f32_to_bf16_rne(res[2]) | ((uint32_t)f32_to_bf16_rne(res[3]) << 16);
  *reinterpret_cast<uint2*>(a.out + (int64_t)row * DV + tid * 4) = make_uint2(lo, hi);
  if (tid == 0) a.lse[row] = lse_out;
}

// Diagnostic: pool rows through the partial pass's 16-byte gather.
__global__ __launch_bounds__(256) void va_gather_kernel(const uint16_t* kv, int64_t num_slots,
                                                        int32_t stride, const int32_t* table,
                                                        int32_t n, uint16_t* dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)n * (DQK / 8)) return;
  const int k = (int)(i / (DQK / 8));
  const int c8 = (int)(i - (int64_t)k * (DQK / 8));
  bool ok = true;
  u32x4 v = gather16(kv, num_slots, stride, table[k], c8, &ok);
  if (!ok) v = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
  *reinterpret_cast<u32x4*>(dst + (int64_t)k * DQK + c8 * 8) = v;
}

// ------------------------------------------------------------------ host side
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

int query_num_cus(int32_t* out) {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VA_ERR_HIP;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) {
    *out = cached[dev];
    return VA_OK;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return VA_ERR_HIP;
  if (dev >= 0 && dev < 64) cached[dev] = v;
  *out = v;
  return VA_OK;
}

bool plan_ok(const va_plan* p) {
  return p != nullptr && p->magic == VA_PLAN_MAGIC && p->version == VA_PLAN_VERSION &&
         p->num_requests >= 1 && p->num_requests <= VA_MAX_REQUESTS && p->total_work >= 1 &&
         p->rows_per_group == ROWS && p->tile_keys == TILE;
}

}  // namespace

extern "C" {

int verify_attn_plan(int32_t num_requests, int32_t num_heads, const int32_t* h_prefix_len,
                     const int32_t* h_num_tree, int32_t num_cus, va_plan* plan,
                     size_t* workspace_bytes) {
  if (h_prefix_len == nullptr || h_num_tree == nullptr || plan == nullptr) return VA_ERR_NULL;
  if (num_requests < 1 || num_requests > VA_MAX_REQUESTS) return VA_ERR_SHAPE;
  if (num_heads < 1 || num_heads > VA_MAX_HEADS) return VA_ERR_SHAPE;
  if (num_cus < 0) return VA_ERR_SHAPE;
  for (int r = 0; r < num_requests; ++r) {
    if (h_num_tree[r] < 1 || h_num_tree[r] > VA_MAX_TREE) return VA_ERR_SHAPE;
    if (h_prefix_len[r] < 0 || h_prefix_len[r] > INT32_MAX - VA_MAX_TREE - TILE) return VA_ERR_SHAPE;
  }
  if (num_cus == 0) {
    const int rc = query_num_cus(&num_cus);
    if (rc != VA_OK) return rc;
  }
  va_plan p;
  std::memset(&p, 0, sizeof p);
  p.magic = VA_PLAN_MAGIC;
  p.version = VA_PLAN_VERSION;
  p.num_requests = num_requests;
  p.num_heads = num_heads;
  p.rows_per_group = ROWS;
  p.tile_keys = TILE;
  p.num_cus = num_cus;

  // Split count: balance keys x row groups over the compute units.
  int64_t units = 0;
  for (int r = 0; r < num_requests; ++r) {
    const int64_t groups = ((int64_t)h_num_tree[r] * num_heads + ROWS - 1) / ROWS;
    units += groups * ((int64_t)h_prefix_len[r] + h_num_tree[r]);
  }
  int64_t keys_per_item = (units + num_cus - 1) / num_cus;
  if (keys_per_item < MIN_KEYS_PER_SPLIT) keys_per_item = MIN_KEYS_PER_SPLIT;
  int forced = 0;
  if (const char* e = std::getenv("VA_NSPLIT")) forced = std::atoi(e);

  int64_t work = 0;
  int64_t tree = 0;
  p.tree_begin[0] = 0;
  p.work_begin[0] = 0;
  for (int r = 0; r < num_requests; ++r) {
    const int64_t n = (int64_t)h_prefix_len[r] + h_num_tree[r];
    const int64_t groups = ((int64_t)h_num_tree[r] * num_heads + ROWS - 1) / ROWS;
    int64_t ns = forced > 0 ? forced : (n + keys_per_item - 1) / keys_per_item;
    const int64_t max_ns = (n + TILE - 1) / TILE;
    if (ns > max_ns) ns = max_ns;
    if (ns > VA_MAX_SPLITS) ns = VA_MAX_SPLITS;
    if (ns < 1) ns = 1;
    p.num_tree[r] = h_num_tree[r];
    p.max_prefix[r] = h_prefix_len[r];
    p.nsplit[r] = (int32_t)ns;
    p.num_groups[r] = (int32_t)groups;
    work += groups * ns;
    tree += h_num_tree[r];
    if (work > INT32_MAX / ROWS || tree * num_heads > INT32_MAX / DV) return VA_ERR_SHAPE;
    p.tree_begin[r + 1] = (int32_t)tree;
    p.work_begin[r + 1] = (int32_t)work;
  }
  p.total_work = (int32_t)work;
  p.total_tree = (int32_t)tree;
  p.total_rows = (int32_t)(tree * num_heads);
  const int64_t o_bytes = align256(work * ROWS * DV * (int64_t)sizeof(float));
  const int64_t lse_bytes = align256(work * ROWS * (int64_t)sizeof(float));
  const int64_t st_bytes = align256(work * (int64_t)sizeof(uint32_t));
  p.lse_offset = o_bytes;
  p.status_offset = o_bytes + lse_bytes;
  p.workspace_bytes = o_bytes + lse_bytes + st_bytes;
  *plan = p;
  if (workspace_bytes != nullptr) *workspace_bytes = (size_t)p.workspace_bytes;
  return VA_OK;
}

int verify_attn_run(const va_plan* plan, const uint16_t* q, const uint16_t* kv_pool,
                    int64_t num_slots, int32_t kv_row_stride, const int32_t* slot_table,
                    int32_t slot_table_len, const int32_t* slot_indptr,
                    const int32_t* prefix_len, const int32_t* parent,
                    float sm_scale, void* workspace, size_t workspace_bytes, va_stream_t stream) {
  if (plan == nullptr || q == nullptr || kv_pool == nullptr || slot_table == nullptr ||
      slot_indptr == nullptr || prefix_len == nullptr || parent == nullptr)
    return VA_ERR_NULL;
  if (!plan_ok(plan)) return VA_ERR_PLAN;
  if (num_slots < 1 || num_slots > (int64_t)INT32_MAX + 1 || kv_row_stride < DQK ||
      slot_table_len < 0)
    return VA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(kv_pool) || (kv_row_stride % 8) != 0) return VA_ERR_ALIGN;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
      (int64_t)workspace_bytes < plan->workspace_bytes)
    return VA_ERR_WORKSPACE;

  PartialArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = q;
  a.kv = kv_pool;
  a.num_slots = num_slots;
  a.stride = kv_row_stride;
  a.num_requests = plan->num_requests;
  a.num_heads = plan->num_heads;
  a.scale_log2 = sm_scale * LOG2E;
  a.slot_table = slot_table;
  a.slot_table_len = slot_table_len;
  a.slot_indptr = slot_indptr;
  a.prefix_len = prefix_len;
  a.parent = parent;
  char* ws = static_cast<char*>(workspace);
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_lse = reinterpret_cast<float*>(ws + plan->lse_offset);
  a.status = reinterpret_cast<uint32_t*>(ws + plan->status_offset);
  for (int r = 0; r < plan->num_requests; ++r) {
    a.num_tree[r] = plan->num_tree[r];
    a.max_prefix[r] = plan->max_prefix[r];
    a.nsplit[r] = plan->nsplit[r];
  }
  for (int r = 0; r <= plan->num_requests; ++r) {
    a.tree_begin[r] = plan->tree_begin[r];
    a.work_begin[r] = plan->work_begin[r];
  }
  hipLaunchKernelGGL(va_partial_kernel, dim3(plan->total_work), dim3(THREADS), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

int verify_attn_reduce(const va_plan* plan, const void* workspace, uint16_t* out, float* lse,
                       va_stream_t stream) {
  if (plan == nullptr || workspace == nullptr || out == nullptr || lse == nullptr)
    return VA_ERR_NULL;
  if (!plan_ok(plan)) return VA_ERR_PLAN;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return VA_ERR_ALIGN;
  ReduceArgs a;
  std::memset(&a, 0, sizeof a);
  const char* ws = static_cast<const char*>(workspace);
  a.part_o = reinterpret_cast<const float*>(ws);
  a.part_lse = reinterpret_cast<const float*>(ws + plan->lse_offset);
  a.status = reinterpret_cast<const uint32_t*>(ws + plan->status_offset);
  a.out = out;
  a.lse = lse;
  a.num_requests = plan->num_requests;
  a.num_heads = plan->num_heads;
  for (int r = 0; r < plan->num_requests; ++r) a.nsplit[r] = plan->nsplit[r];
  for (int r = 0; r <= plan->num_requests; ++r) {
    a.tree_begin[r] = plan->tree_begin[r];
    a.work_begin[r] = plan->work_begin[r];
  }
  hipLaunchKernelGGL(va_reduce_kernel, dim3(plan->total_rows), dim3(DV / 4), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

int verify_attn_read_status(const va_plan* plan, const void* workspace, va_stream_t stream,
                            uint32_t* h_status) {
  if (plan == nullptr || workspace == nullptr || h_status == nullptr) return VA_ERR_NULL;
  if (!plan_ok(plan)) return VA_ERR_PLAN;
  const int n = plan->total_work;
  uint32_t* host = static_cast<uint32_t*>(std::malloc(sizeof(uint32_t) * n));
  if (host == nullptr) return VA_ERR_HIP;
  const char* ws = static_cast<const char*>(workspace) + plan->status_offset;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = VA_OK;
  if (hipMemcpyAsync(host, ws, sizeof(uint32_t) * n, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    rc = VA_ERR_HIP;
  } else {
    uint32_t acc = 0u;
    for (int i = 0; i < n; ++i) acc |= host[i];
    *h_status = acc;
  }
  std::free(host);
  return rc;
}

int verify_attn_check_tree(const int32_t* h_parent, int32_t T) {
  if (h_parent == nullptr) return VA_ERR_NULL;
  if (T < 1 || T > VA_MAX_TREE) return VA_ERR_TREE;
  for (int32_t i = 0; i < T; ++i)
    if (h_parent[i] < -1 || h_parent[i] >= i) return VA_ERR_TREE;
  return VA_OK;
}

int verify_attn_gather_rows(const uint16_t* kv_pool, int64_t num_slots, int32_t kv_row_stride,
                            const int32_t* slot_table, int32_t n, uint16_t* dst,
                            va_stream_t stream) {
  if (kv_pool == nullptr || slot_table == nullptr || dst == nullptr) return VA_ERR_NULL;
  if (n < 0 || num_slots < 1 || kv_row_stride < DQK) return VA_ERR_SHAPE;
  if (!aligned16(kv_pool) || !aligned16(dst) || (kv_row_stride % 8) != 0) return VA_ERR_ALIGN;
  if (n == 0) return VA_OK;
  const int64_t pieces = (int64_t)n * (DQK / 8);
  const int64_t blocks = (pieces + 255) / 256;
  hipLaunchKernelGGL(va_gather_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), kv_pool, num_slots, kv_row_stride,
                     slot_table, n, dst);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

const char* verify_attn_error_string(int code) {
  switch (code) {
    case VA_OK: return "ok";
    case VA_ERR_NULL: return "a required pointer is NULL";
    case VA_ERR_SHAPE: return "a count or size is out of range";
    case VA_ERR_ALIGN: return "a buffer is not 16-byte aligned or the row stride is not a multiple of 8";
    case VA_ERR_WORKSPACE: return "workspace is NULL, not 256-byte aligned or smaller than the plan needs";
    case VA_ERR_PLAN: return "plan was not produced by verify_attn_plan of this library version";
    case VA_ERR_HIP: return "a HIP call or kernel launch failed";
    case VA_ERR_TREE: return "parent array is not a topological forest (parent[i] must be in [-1, i-1])";
    case VA_ERR_DEVICE_DATA: return "device-resident inputs failed the in-kernel checks";
    default: return "unknown error code";
  }
}

size_t verify_attn_plan_struct_size(void) { return sizeof(va_plan); }

}  // extern "C"
