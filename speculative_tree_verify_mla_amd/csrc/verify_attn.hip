// verify_attn.hip - tree-verify MLA attention for MI355X (gfx950, CDNA4).
//
// Split-KV partial pass + log-sum-exp reduce ("The Verify Kernel
// Breakthrough", section "The Message in Context": partial+reduce;
// "The Architecture Detective", section "The Split Verify Design": LSE
// merge), with each KV tile loaded once and shared by every head and draft
// node of a row group ("The Execution Phase", section "The Core Design: A
// Streaming Flash Attention Kernel": KV-tile outer, heads inner), 16-byte
// gathers of the page_size=1 rows (same page, section "The Optimization That
// Unlocked 3-6x Speedup": 128-bit loads) and graph-capture-safe launches
// (same page, section "Making the Kernel CUDA Graph Capture-Safe").
//
// gfx950 mapping of one work item (request r, row group g of 64 query rows,
// KV split s):
//   - 256 threads = 4 wave64s, one per SIMD.  Wave w owns row half
//     rh = w & 1 (32 query rows, the MFMA N dimension) and half kh = w >> 1
//     of the work: for the score, keys 32*kh .. +31 of every 64-key tile over
//     all 576 columns (the full Q of its rows stays in accumulation
//     registers, so no partial scores are exchanged); for the output, columns
//     256*kh .. +255 over all 64 keys.  The two key halves hand each other
//     their bf16 probabilities through an 8 KB LDS buffer: one barrier per
//     tile besides the tile barrier.  Each wave runs the output MFMAs of its
//     own key half before that barrier and the other half's after it.
//   - The group's Q rows are copied once into the second tile buffer in the
//     tile layout, each wave reads its fragments from there, and the first
//     tile's barrier frees the buffer for the second tile.  The first tile's
//     copies go out as soon as its slot-table entries have landed, while Q
//     is still in flight.
//   - Tiles of 64 pool rows go straight from HBM into LDS with
//     global_load_lds_dwordx4 (1 KB per wave instruction: one 128-byte line
//     of 8 rows, each lane holding its row's address, so a copy costs three
//     instructions), double-buffered: one tile is in flight while the other
//     is consumed.  The slot-table entries of a tile are copied into a small
//     LDS ring two tiles ahead of its rows.  All these copies are inline asm
//     counted by hand (see vm_wait), so the compiler never makes an LDS read
//     wait for them.  In LDS a tile is stored line by line with the 16-byte
//     pieces of each row XOR-swizzled (piece_off), so both MFMA read patterns
//     below are free of LDS bank conflicts.
//   - S^T[key][row] = K . Q^T on v_mfma_f32_32x32x16_bf16 (A = K fragment
//     from LDS, B = Q rows held in accumulation registers).  The output layout gives each lane
//     one query row (lane % 32) and, per register quad, 4 of the wave's keys,
//     so the probabilities of keys 16*ks .. +15 are, register for register,
//     the B operand of O^T = V^T . P^T for k-step ks.  That operand's A side
//     comes from the same K tile through ds_read_b64_tr_b16 (transpose reads:
//     no transposed copy of V).
//   - Each row's probabilities are taken against a fixed reference: the
//     row's first finite tile max.  Probabilities may then exceed 1 (up to
//     2^64), which bf16 and the fp32 accumulators hold without loss of
//     relative precision, and the accumulators are never rescaled.  If a
//     later tile beats a row's reference by more than 2^64 (only adversarial
//     inputs do), the work item sweeps its split once for each row's exact
//     max (scores only) and then computes the split again against that max,
//     so every input takes at most three passes.
//   - The tree mask is one 64-bit ancestor mask per draft node, built in the
//     prologue from parent[] (copied into the slot ring's last row beside the
//     first slot entries); only tiles reaching past the prefix consult it.
//   - Each work item writes its normalised output o / lb (lb = the sum of the
//     bf16 weights) in fp16 with a per-row power-of-two scale, in the MFMA
//     output layout (512 B per wave store, streaming stores: only the merge
//     reads them), and its lse (base 2); the reduce merges a row's splits
//     with one round of loads and writes bf16 out and natural-log lse.

#include <hip/hip_runtime.h>
// m0 is set inside the copy asm (nothing else in these kernels uses it)
#pragma clang diagnostic ignored "-Winline-asm"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <utility>

#include "verify_attn.h"

// Scratch of verify_attn_forward_static: the partials, lse pairs and status
// words of up to VA_STATIC_SCRATCH_WORK work items, laid out as a workspace.
// Each device holds its own copy for the life of the process.  Host code
// takes its device address from hipGetSymbolAddress (static_scratch below)
// and never passes the name itself to a kernel.
static __device__ __align__(256) unsigned char scratch[VA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int DQK = VA_D_QK;      // 576
constexpr int DV = VA_D_V;        // 512: value columns = latent columns
constexpr int DROPE = DQK - DV;   // 64 rope columns
constexpr int TILE = 64;          // keys per LDS tile
constexpr int HALF = TILE / 2;    // keys of a tile one wave owns (the MFMA M dimension)
constexpr int SPLIT_ALIGN = 32;   // split lengths are multiples of this many keys
constexpr int THREADS = 256;      // 4 waves, one per SIMD
constexpr int ROWS = 64;          // query rows per work item
constexpr int NPIECE = DQK / 8;                   // 16-byte pieces of a key row: 64 latent, 8 rope
constexpr int NLINE = NPIECE / 8;                 // 128-byte lines of a key row: 8 latent, 1 rope
constexpr int CHUNK = 8 * 128;                    // one line of 8 keys (one copy instruction)
constexpr int LINE = (TILE / 8) * CHUNK;          // one line of all the keys of a tile
constexpr int BUF_BYTES = NLINE * LINE;           // one tile buffer: 73,728 B
constexpr int BUF_ELEMS = BUF_BYTES / 2;
constexpr int QK_STEPS = DQK / 16;   // 36 MFMA k-steps (16 columns each) for the score
constexpr int LAT_STEPS = DV / 16;   // the first 32 are latent columns, the last 4 rope
constexpr int O_BLK = DV / 32;       // 16 MFMA column blocks (32 columns) of the output
constexpr int O_HALF = O_BLK / 2;    // 8 of them per wave (one column half)
constexpr int PART_VEC = ROWS * DV / 4;  // 4-column entries of one work item's partial output
constexpr int SLOT_RING = 4;         // LDS ring of per-tile slot-table entries (3 live)
constexpr int COPIES = 2 * NLINE;    // copies one wave issues per tile: 9 lines of 2 key groups
constexpr int MIN_KEYS_PER_SPLIT = 128;
constexpr float REF_SLACK = 64.f;  // log2 units: probabilities stay <= 2^64
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct PartialArgs {
  const uint16_t* q;
  const uint16_t* kv;
  int64_t num_slots;
  int32_t stride;
  int32_t num_requests;
  int32_t num_heads;
  int32_t total_work;
  float scale_log2;   // sm_scale * log2(e): scores are kept in base 2
  const int32_t* slot_table;
  int32_t slot_table_len;
  const int32_t* slot_indptr;
  const int32_t* prefix_len;
  const int32_t* parent;
  uint32_t* part_o;   // [work][PART_VEC] 4 x fp16 (o / lb scaled by 2^-e), MFMA layout
  float* part_lse;    // [work][ROWS][2]: lse (base 2), scale exponent e
  uint32_t* status;   // [work]
  int32_t num_tree[VA_MAX_REQUESTS];
  int32_t max_prefix[VA_MAX_REQUESTS];
  int32_t nsplit[VA_MAX_REQUESTS];
  int32_t num_groups[VA_MAX_REQUESTS];
  int32_t tree_begin[VA_MAX_REQUESTS + 1];
  int32_t work_begin[VA_MAX_REQUESTS + 1];
};

struct ReduceArgs {
  const uint32_t* part_o;  // [work][PART_VEC] 4 x fp16 (o / lb scaled by 2^-e), MFMA layout
  const float* part_lse;   // [work][ROWS][2]: lse (base 2), scale exponent e
  const uint32_t* status;
  uint16_t* out;
  float* lse;
  int32_t num_requests;
  int32_t num_heads;
  int32_t nsplit[VA_MAX_REQUESTS];
  int32_t num_groups[VA_MAX_REQUESTS];
  int32_t tree_begin[VA_MAX_REQUESTS + 1];
  int32_t work_begin[VA_MAX_REQUESTS + 1];
};

// Source of the pieces of keys that are missing (past the split end) or
// whose slot is outside the pool: a row of zeros.
__device__ const uint16_t va_zero_row[DQK] = {};

// Two fp32 values as packed bf16 bits (a in the low half), rounded to
// nearest even by the hardware conversion.
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)a, (__bf16)b});
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// Asynchronous copy of 16 bytes per lane from global memory into LDS: lane i
// writes lds_base + 16*i (global_load_lds_dwordx4; lds_base is wave-uniform).
__device__ __forceinline__ void dma16(const uint16_t* src, uint16_t* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// The partial kernel issues its copies into LDS as inline asm, so the
// compiler sees no vector-memory operation in the tile loop: it would
// otherwise make every LDS read wait for all outstanding copies (vmcnt(0)),
// serialising the copy of tiles t+1, t+2 with the compute of tile t.  The
// kernel counts its own copies instead (vm_wait) and every wait/barrier is a
// compiler memory fence.  `nt` marks the KV rows as streamed once.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// 4 bytes per lane from a per-lane address (lane i writes lds + 4 i)
__device__ __forceinline__ void dma4_v(uint32_t lds, const void* addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds), "v"(addr) : "memory", "m0");
}
// Copy of line J of key group 2 w + E (w = wave) of a tile: the lane's
// address (addr) points at its key row's piece (lane % 8) ^ swz(key) of line
// 0; lds_w = tile buffer + 2 w CHUNK.  The instruction offset 128 J advances
// both the global address (by one line) and the LDS address, so
// m0 = lds_w + E CHUNK + (LINE - 128) J puts lane l at
// buffer + J LINE + (2 w + E) CHUNK + 16 l.
template <int E, int J>
__device__ __forceinline__ void dma_line(uint32_t lds_w, const void* addr) {
  asm volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%3 nt"
               :: "s"(lds_w), "v"(addr), "n"(E * CHUNK + (LINE - 128) * J), "n"(128 * J)
               : "memory", "m0", "scc");
}
template <int E, int J>
__device__ __forceinline__ void dma_line_keep(uint32_t lds_w, const void* addr) {
  asm volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%3"
               :: "s"(lds_w), "v"(addr), "n"(E * CHUNK + (LINE - 128) * J), "n"(128 * J)
               : "memory", "m0", "scc");
}
// all 18 copies of a wave (addr[e]: key group 2 w + e)
template <int... J>
__device__ __forceinline__ void dma_lines_keep(uint32_t lds_w, const void* addr0, const void* addr1,
                                               std::integer_sequence<int, J...>) {
  (dma_line_keep<0, J>(lds_w, addr0), ...);
  (dma_line_keep<1, J>(lds_w, addr1), ...);
}
// copy C of a wave's 18: key group 2 w + C / 9, line C % 9
template <int C>
__device__ __forceinline__ void dma_copy(uint32_t lds_w, const void* addr0, const void* addr1) {
  if (C < NLINE) dma_line<0, C % NLINE>(lds_w, addr0);
  else dma_line<1, C % NLINE>(lds_w, addr1);
}
// copies 2 part and 2 part + 1 (part is a constant once the caller's loop is unrolled)
template <int... P>
__device__ __forceinline__ void dma_part(int part, uint32_t lds_w, const void* addr0,
                                         const void* addr1, std::integer_sequence<int, P...>) {
  ((part == P ? (dma_copy<2 * P>(lds_w, addr0, addr1), dma_copy<2 * P + 1>(lds_w, addr0, addr1))
              : void()), ...);
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// barrier that is also a compiler memory fence, after this wave's own LDS
// operations have completed
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane block,
// lane i receives element (i % 4) of the 8-byte pieces addressed by lanes
// i/4, i/4+4, i/4+8 and i/4+12.  A block whose lane i addresses
// K[k0 + i/4][c0 + 4*(i%4)] therefore hands lane i the column c0 + i of the
// four keys k0..k0+3: half of a value-MFMA operand, read from the row-major
// key tile without a transposed copy.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Table entry of logical key k with the index clamped into [0, k_end) so the
// load stays inside the request's table (k_end >= 1).
__device__ __forceinline__ int32_t table_entry(const int32_t* __restrict__ table, int k,
                                               int k_end) {
  return table[k < k_end ? k : k_end - 1];
}

// LDS tile layout: piece p (columns 8p .. 8p+7, 16 bytes) of key k lies at
//   (p / 8) LINE + (k / 8) CHUNK + (k % 8) 128 + ((p % 8) ^ swz(k)) 16.
// A copy instruction moves one 128-byte line of 8 keys (8 lanes per key, one
// global line each).  swz keeps the score reads (one piece of 16
// consecutive keys) and the transposed value reads (4 pieces of 4 keys) on
// distinct LDS banks.
__device__ __forceinline__ constexpr int swz(int k) { return (((k >> 1) & 1) << 2) | ((k >> 2) & 3); }
// byte offset of piece p of key k within a tile buffer
__device__ __forceinline__ constexpr int piece_off(int k, int p) {
  return (p >> 3) * LINE + (k >> 3) * CHUNK + (k & 7) * 128 + (((p & 7) ^ swz(k)) << 4);
}

// The tile loader's lane roles.  Wave w copies the 9 lines of tile keys
// 16w .. 16w+15 (18 copies of 1 KB: 8 keys x 128 bytes); lane l takes key
// tile_key(w, e, l) (e = 0, 1), whose slot it reads from the slot ring, and
// the 16-byte piece (l % 8) ^ swz(key) of each of that key's lines.
__device__ __forceinline__ int tile_key(int wave, int e, int lane) {
  return 16 * wave + 8 * e + (lane >> 3);
}
// Global source of the lane's piece of line 0 of tile key `key`: the slot's
// pool row, or the zero row for a key past the split end (exists false) or a
// slot outside the pool (which also sets VA_STATUS_BAD_SLOT in bad).  The
// copy of line J then reads 128 J bytes further.
__device__ __forceinline__ const uint16_t* copy_source(const uint16_t* kv, int64_t num_slots,
                                                       int32_t stride, int32_t slot, bool exists,
                                                       int key, int lane, uint32_t& bad) {
  const bool inside = slot >= 0 && (int64_t)slot < num_slots;
  if (exists && !inside) bad = VA_STATUS_BAD_SLOT;
  return (exists && inside ? kv + (int64_t)slot * stride : va_zero_row) + 8 * ((lane & 7) ^ swz(key));
}

// Which keys a launch of the partial kernel covers.
//   FUSED:  every split of a request covers a slice of its L + T keys; tiles
//           reaching into the draft block apply the tree mask.
//   PREFIX: splits 0 .. ns-2 cover slices of the L prefix keys only, with no
//           tree mask; split ns-1 (the tree block) is left to TREE.
//   TREE:   one work item per (request, row group): the T draft keys, with
//           the tree mask.
// PREFIX + TREE is the split-verify decomposition ("The Architecture
// Detective", section "The Split Verify Design": a dense prefix pass and a
// small masked tree-block pass joined by the log-sum-exp merge); the reduce
// is the same for both.
enum KernelMode { FUSED = 0, PREFIX = 1, TREE = 2 };

// LDS of one work item (157,200 bytes of the 160 KB).
struct PartialSmem {
  __attribute__((aligned(16))) uint16_t tiles[2 * BUF_ELEMS];
  // bf16 probabilities [row half][key half][lane] (two value-MFMA operands per
  // lane); before the first tile the same bytes hold the ancestor masks
  __attribute__((aligned(16))) bf16x8 xp[2][2][2][64];
  int32_t sring[SLOT_RING][TILE];   // slot-table entries of upcoming tiles
  float xm[2][2][32];               // per-row maxima [row half][key half][row]
  uint32_t status_sh;
  uint32_t restart_sh;
};
static_assert(sizeof(PartialSmem::xp) >= VA_MAX_TREE * sizeof(uint64_t), "ancestor masks fit");

// The arguments the prologue's first loads depend on.  The kernels take them
// as leading scalar parameters, ahead of the argument struct, and the library
// is built with kernel-argument preloading, so they arrive in scalar
// registers at wave launch: the request-length and slot-table loads go out
// without first waiting for a kernel-argument load.  ONE (a plan with a
// single request) also takes that request's split count, row groups, draft
// nodes and prefix bound from here instead of the struct's arrays.  14
// dwords are preloaded (16 user SGPRs less the argument-segment pointer):
// the parameters are ordered so that only the last ones, needed after the
// first loads return, come from memory.
struct Lead {
  const int32_t* prefix_len;
  const int32_t* slot_indptr;
  const int32_t* slot_table;
  const uint16_t* q;
  int32_t total_work;
  int32_t num_heads;
  int32_t slot_table_len;
  int32_t ns0, g0, t0, max_prefix0;   // request 0 (used when ONE)
};

template <int MODE, bool ONE>
__device__ __forceinline__ void partial_body(const PartialArgs& a, const Lead& f, int block,
                                             PartialSmem& sm);

// FUSED launch: one block per work item (XCD-ordered, see partial_body).
template <bool ONE>
__global__ __launch_bounds__(THREADS, 1) void va_partial_kernel(
    const int32_t* prefix_len, const int32_t* slot_indptr, const int32_t* slot_table,
    const uint16_t* q, int32_t total_work, int32_t num_heads, int32_t slot_table_len, int32_t ns0,
    int32_t g0, int32_t t0, int32_t max_prefix0, PartialArgs a) {
  __shared__ PartialSmem sm;
  const Lead f{prefix_len, slot_indptr, slot_table, q, total_work, num_heads, slot_table_len,
               ns0, g0, t0, max_prefix0};
  partial_body<FUSED, ONE>(a, f, blockIdx.x, sm);
}

// SPLIT_TREE launch: the tree-block work items (blocks 0 .. tree_blocks-1)
// and the prefix work items share one grid, so the small tree block runs on
// its own compute units alongside the prefix splits instead of before them.
template <bool ONE>
__global__ __launch_bounds__(THREADS, 1) void va_split_kernel(
    const int32_t* prefix_len, const int32_t* slot_indptr, const int32_t* slot_table,
    const uint16_t* q, int32_t tree_blocks, int32_t total_work, int32_t num_heads,
    int32_t slot_table_len, int32_t ns0, int32_t g0, int32_t t0, int32_t max_prefix0, PartialArgs a) {
  __shared__ PartialSmem sm;
  const Lead f{prefix_len, slot_indptr, slot_table, q, total_work, num_heads, slot_table_len,
               ns0, g0, t0, max_prefix0};
  if ((int)blockIdx.x < tree_blocks) partial_body<TREE, ONE>(a, f, blockIdx.x, sm);
  else partial_body<PREFIX, ONE>(a, f, blockIdx.x - tree_blocks, sm);
}

template <int MODE, bool ONE>
__device__ __forceinline__ void partial_body(const PartialArgs& a, const Lead& f, int block,
                                             PartialSmem& sm) {
  uint16_t* const tiles = sm.tiles;
  bf16x8 (&xp)[2][2][2][64] = sm.xp;
  int32_t (&sring)[SLOT_RING][TILE] = sm.sring;
  float (&xm)[2][2][32] = sm.xm;
  uint32_t& status_sh = sm.status_sh;
  uint32_t& restart_sh = sm.restart_sh;
  uint64_t* anc = reinterpret_cast<uint64_t*>(&xp[0][0][0][0]);   // [VA_MAX_TREE]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = wave & 1;      // row half of the work item's 64 rows
  const int kh = wave >> 1;     // key half of every tile for the score; column half of the output
  const int lrow = lane & 31;   // MFMA column: this lane's query row within the row half
  const int lh = lane >> 5;     // MFMA k-half of this lane

  // Work items are ordered (request, split, row group); block b runs on XCD
  // b % 8, so each XCD takes a contiguous run of work items and the row
  // groups that read the same KV split share that XCD's L2.
  int w, r = 0;
  if (MODE == TREE) {
    // block b -> (request, row group) of the tree-block work items
    int b = block;
    if (ONE) {
      if (b >= f.g0) return;
      w = (f.ns0 - 1) * f.g0 + b;
    } else {
      while (r + 1 < a.num_requests && b >= a.num_groups[r]) {
        b -= a.num_groups[r];
        ++r;
      }
      if (b >= a.num_groups[r]) return;
      w = a.work_begin[r] + (a.nsplit[r] - 1) * a.num_groups[r] + b;
    }
  } else {
    const int per_xcd = (f.total_work + 7) >> 3;
    w = (block & 7) * per_xcd + (block >> 3);
    if (w >= f.total_work) return;
    if (!ONE) while (r + 1 < a.num_requests && a.work_begin[r + 1] <= w) ++r;
  }
  const int G = ONE ? f.g0 : a.num_groups[r];
  const int local = w - (ONE ? 0 : a.work_begin[r]);
  const int s = local / G;
  const int g = local - s * G;
  const int ns = ONE ? f.ns0 : a.nsplit[r];
  if (MODE == PREFIX && s == ns - 1) return;   // the tree block
  const int T = ONE ? f.t0 : a.num_tree[r];
  const int H = f.num_heads;
  const int tb = ONE ? 0 : a.tree_begin[r];
  const int rows_r = T * H;

  if (tid == 0) status_sh = 0u;

  uint32_t st = 0u;
  const int maxp = ONE ? f.max_prefix0 : a.max_prefix[r];
  int L = f.prefix_len[r];
  if (L < 0 || L > maxp) {
    st |= VA_STATUS_BAD_PREFIX;
    L = L < 0 ? 0 : maxp;
  }
  const int n = L + T;
  const int tab0 = f.slot_indptr[r];
  const int tab1 = f.slot_indptr[r + 1];
  int n_valid = n;   // keys whose table entry exists
  if (tab0 < 0 || tab1 < tab0 || tab1 > f.slot_table_len || tab1 - tab0 < n) {
    st |= VA_STATUS_SHORT_TABLE;
    n_valid = (tab0 < 0 || tab1 < tab0 || tab0 >= f.slot_table_len)
                  ? 0 : min(min(tab1, f.slot_table_len) - tab0, n);
  }
  int k0, k1;   // key range of this split (keys past a short table dropped)
  if (MODE == FUSED) {
    // the L prefix keys in ns slices of whole SPLIT_ALIGN blocks; the T
    // draft keys go with the last slice
    const int chunk = ((L + ns - 1) / ns + SPLIT_ALIGN - 1) / SPLIT_ALIGN * SPLIT_ALIGN;
    k0 = min(s * chunk, L);
    k1 = min(n_valid, s == ns - 1 ? n : min(k0 + chunk, L));
  } else if (MODE == PREFIX) {
    const int np = ns - 1;   // >= 1 here
    const int chunk = ((L + np - 1) / np + SPLIT_ALIGN - 1) / SPLIT_ALIGN * SPLIT_ALIGN;
    k0 = min(s * chunk, L);
    k1 = min(min(n_valid, L), k0 + chunk);
  } else {
    k0 = L;
    k1 = min(n_valid, n);
  }
  const int ntiles = k1 > k0 ? (k1 - k0 + TILE - 1) / TILE : 0;
  const int32_t* table = f.slot_table + (n_valid > 0 ? tab0 : 0);

  // ---- slot-table entries of the first two tiles: the first copies wait on
  // them, so they go out before everything else.  Wave 0 copies the 64
  // entries of tile u into sring[u % SLOT_RING] (one 4-byte copy per lane;
  // keys past the split end read the split's last entry, which is in bounds).
  auto issue_slots = [&](int u) {
    if (wave == 0) {
      const int k = min(k0 + u * TILE + lane, k1 - 1);
      dma4_v(lds_addr(&sring[u & (SLOT_RING - 1)][0]), table + k);
    }
  };
  if (ntiles > 0) {
    issue_slots(0);
    issue_slots(1);
  }
  // the parent entries of the request's draft nodes go to the slot ring's
  // last row (free until the first tile is consumed); lanes past T re-read
  // entry T-1
  if (MODE != PREFIX && wave == 0)
    dma4_v(lds_addr(&sring[SLOT_RING - 1][0]), a.parent + tb + min(lane, T - 1));

  // ---- Q, all 576 score columns of the group's rows
  const int rho = g * ROWS + rh * 32 + lrow;
  const bool row_ok = rho < rows_r;
  bf16x8 qf[QK_STEPS];
  // The group's 64 Q rows are copied once into the second tile buffer, in
  // the layout of a key tile (each row is read by the two key-half waves of
  // its row half; one copy per block halves the Q traffic of loading the
  // fragments per wave).  Rows past the group's end copy row 0 of the
  // request: they repeat its scores exactly (so raise no restart of their
  // own) and their partial rows are never merged.  Wave w copies rows
  // 16w .. 16w+15.  The first tile goes into the first buffer;
  // the second tile's copies start after the barrier at the top of the
  // first tile, when every wave has read its fragments.
  {
    const uint16_t* const q0 = f.q + (int64_t)tb * H * DQK;
    const uint16_t* src[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 16 * wave + 8 * e + (lane >> 3);   // row of the group this lane copies
      const int rr = g * ROWS + i < rows_r ? g * ROWS + i : 0;
      src[e] = q0 + (int64_t)rr * DQK + 8 * ((lane & 7) ^ swz(i));
    }
    dma_lines_keep(lds_addr(tiles + BUF_ELEMS) + 2 * wave * CHUNK, src[0], src[1],
                   std::make_integer_sequence<int, NLINE>{});
  }

  // ---- tile loader.  Wave w copies the 9 lines of keys 16w .. 16w+15 (18
  // copies of 1 KB: 8 keys x 128 bytes); lane l takes key 16w + 8e + l/8
  // (e = 0, 1), whose slot it reads from the ring.  Keys past the split end
  // and slots outside the pool copy the zero row.
  uint32_t bad = 0u;
  // The copies of a tile are issued in 9 parts of 2 spread over the score
  // MFMAs of the previous tile: a burst of all of them stalls the wave on
  // memory back-pressure while the MFMA pipe idles.
  struct TileIssue {
    const uint16_t* src[2];   // this lane's piece of line 0 of its two key rows
    uint32_t lds_w;           // LDS byte address of chunk 2 w of the tile buffer
  };
  struct SlotPair {
    int32_t v[2];
  };
  auto read_slots = [&](int u) -> SlotPair {
    SlotPair sp;
#pragma unroll
    for (int e = 0; e < 2; ++e) sp.v[e] = sring[u & (SLOT_RING - 1)][tile_key(wave, e, lane)];
    return sp;
  };
  // vslot: read_slots(u), read ahead by the caller
  auto prepare_tile = [&](int u, const SlotPair& vslot, uint16_t* buf) -> TileIssue {
    TileIssue ti;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = tile_key(wave, e, lane);
      ti.src[e] = copy_source(a.kv, a.num_slots, a.stride, vslot.v[e], k0 + u * TILE + key < k1,
                              key, lane, bad);
    }
    ti.lds_w = lds_addr(buf) + 2 * wave * CHUNK;
    return ti;
  };
  // copies 2 part, 2 part + 1 of the tile
  auto issue_part = [&](const TileIssue& ti, int part) {
    dma_part(part, ti.lds_w, ti.src[0], ti.src[1], std::make_integer_sequence<int, COPIES / 2>{});
  };
  static_assert(COPIES == 2 * 9, "copies of a tile = 2 per score MFMA group");


  f32x16 o[O_HALF];
  // The reference this row's probabilities are taken against (common to the
  // two key-half waves of a row half), the largest tile max this wave has
  // seen, and the sums over this wave's keys (lane ^ 32 holds the other
  // half of the row's keys).  l sums the fp32 probabilities and gives the
  // lse; lb sums the bf16 probabilities that enter the value MFMA and
  // normalises the output, so the output is an exact weighted average of its
  // value rows.
  float m_ref = -INFINITY;
  bf16x8 pown[2];   // this wave's own probabilities of the current tile (P operand)
  float m_seen = -INFINITY;
  float l_run = 0.f;
  float lb_run = 0.f;

  // per-lane LDS byte offsets of the MFMA operands within a tile buffer.
  // Score k-step k reads piece 2k + lh of key krow: LINE (k / 4) + kb[k % 4].
  const int krow = kh * HALF + lrow;                      // this lane's key row for the score
  uint32_t kb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kb[i] = piece_off(krow, 2 * i + lh);
  // value operand: block b = lane/16 reads keys 16*ks + 4*(b>>1) + i/4 (+8)
  // and columns 16*(b&1) + 4*(i%4) of each 32-column block (i = lane%16) of
  // this wave's column half
  // (key 16 ks' + 8n + 4 (b>>1) + i/4, piece 32 kh + 4 cb + 2 (b&1) + (i%4)/2,
  // byte 8 (i%2): vb[cb % 2][n] below, plus LINE (4 kh + cb / 2) and 2 CHUNK ks')
  uint32_t vb[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int n = 0; n < 2; ++n)
      vb[c][n] = piece_off(8 * n + 4 * lh + ((lane & 15) >> 2),
                           4 * c + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + (lane & 1) * 8;
  }
  const int qkey = kh * HALF + 4 * lh;   // tile key of register 4*qd+i is qkey + 8*qd + i

  // Consumes tile t (one buffer).  `first` is set on the first tile of a
  // pass: the two key-half waves then agree on each row's reference.
  // In the sweep pass (`sweep`) only the scores and their max are taken.
  auto compute = [&](int t, const uint16_t* buf, uint64_t anc_row, bool first,
                     const TileIssue& nxt, bool sweep) {
    const int kt = k0 + t * TILE;
    // keep every Q fragment in an accumulation register for the whole loop:
    // the score MFMAs read them there directly, where the allocator would
    // otherwise copy most of them to VGPRs before each use
#pragma unroll
    for (int k = 0; k < QK_STEPS; ++k) asm volatile("" : "+a"(qf[k]));
    // S^T = K . Q^T for this wave's 32 keys over all 576 score columns
    f32x16 sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
    // K fragments in groups of QG k-steps, the next group's LDS reads issued
    // ahead of the current group's MFMAs
    constexpr int QG = 4;
    auto load_k = [&](bf16x8* kf, int k0s) {
#pragma unroll
      for (int kk = 0; kk < QG; ++kk) {
        const int k = k0s + kk;
        kf[kk] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint8_t*>(buf) +
                                                  LINE * (k >> 2) + kb[k & 3]);
      }
    };
    // after each group's MFMAs, 2 of the next tile's copies
    bf16x8 kfa[QG], kfb[QG];
    load_k(kfa, 0);
#pragma unroll
    for (int g = 0; g < QK_STEPS / QG; ++g) {
      bf16x8* cur = (g & 1) ? kfb : kfa;
      bf16x8* ahead = (g & 1) ? kfa : kfb;
      if (g + 1 < QK_STEPS / QG) load_k(ahead, (g + 1) * QG);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < QG; ++kk)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[kk], qf[g * QG + kk], sacc, 0, 0, 0);
      issue_part(nxt, g);
      __builtin_amdgcn_sched_barrier(0);
    }

    // mask (only on tiles reaching past the prefix or the split end)
    if (MODE == PREFIX ? kt + TILE > k1 : (kt + TILE > L || kt + TILE > k1)) {   // uniform
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kp = kt + qkey + 8 * (e >> 2) + (e & 3);
        const int d = kp - L;
        const bool in_tree = MODE == PREFIX || d < 0 || ((anc_row >> (d & 63)) & 1ull);
        sacc[e] = (kp < k1 && in_tree) ? sacc[e] : -INFINITY;
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
    {   // this wave's 32 keys of the row: lanes l and l ^ 32 hold the two halves
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                       __builtin_bit_cast(uint32_t, mx), false, false);
      mx = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
    }
    mx *= a.scale_log2;
    m_seen = fmaxf(m_seen, mx);
    if (sweep) return;   // uniform
    if (first) {
      // reference = the row's max over the whole tile (both key halves)
      if (lh == 0) xm[rh][kh][lrow] = mx;
      lds_barrier();
      const float r2 = fmaxf(xm[rh][0][lrow], xm[rh][1][lrow]);
      if (m_ref == -INFINITY) m_ref = r2;
    } else if (mx > m_ref + REF_SLACK) {
      restart_sh = 1u;   // all waves stop the pass; the sweep for the exact max follows
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    // probabilities exp2(s * scale - m); register quads 2ks, 2ks+1 form the
    // B operand of value k-step ks of this key half
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * ks + i], a.scale_log2, -m_use));
      l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      bf16x2 pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = bf16x2{(__bf16)p[2 * i], (__bf16)p[2 * i + 1]};
        lb_run = __builtin_amdgcn_fdot2_f32_bf16(pb[i], ones, lb_run, false);
      }
      pown[ks] = __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(uint32_t, pb[0]),
                                                   __builtin_bit_cast(uint32_t, pb[1]),
                                                   __builtin_bit_cast(uint32_t, pb[2]),
                                                   __builtin_bit_cast(uint32_t, pb[3])});
      xp[rh][kh][ks][lane] = pown[ks];
    }
  };

  // O^T += V^T . P^T for this wave's 256 output columns over the 32 keys of
  // key half `half` (value k-steps 2 half, 2 half + 1, P operand ph): 8
  // column blocks x 2 k-steps, V^T fragments by transpose reads one block
  // ahead.  Each tile runs it twice: first for the wave's own key half, whose
  // probabilities are still in registers, while the other key-half wave
  // finishes its scores; then, after the exchange barrier, for the other half.
  auto value_half = [&](const uint16_t* buf, int half, const bf16x8* ph) {
    auto load_v2 = [&](bf16x8* vf, int cb) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint8_t* p0 = reinterpret_cast<const uint8_t*>(buf) + (4 * kh + (cb >> 1)) * LINE +
                            (2 * half + j) * (2 * CHUNK);
        const i16x4 v0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(p0 + vb[cb & 1][0]));
        const i16x4 v1 = lds_read_tr16(reinterpret_cast<const uint16_t*>(p0 + vb[cb & 1][1]));
        const i16x8 v8 = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        vf[j] = __builtin_bit_cast(bf16x8, v8);
      }
    };
    bf16x8 vfa[2], vfb[2];
    load_v2(vfa, 0);
#pragma unroll
    for (int cb = 0; cb < O_HALF; cb += 2) {
      load_v2(vfb, cb + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfa[j], ph[j], o[cb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (cb + 2 < O_HALF) load_v2(vfa, cb + 2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        o[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfb[j], ph[j], o[cb + 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline over the split's tiles (two buffers; tile u in buffer u % 2).
  // Per wave the copies are issued in the order
  //   [slots 0, 1] [parents] [Q] (wait for all but Q) [tile 0] [slots 2]
  //   (wait for Q) | loop t: [slots t+3] [tile t+1]
  // (slot and parent copies on wave 0 only; Q goes to the second buffer in
  // the first pass; the copies of tile t+1 are spread over the score MFMAs of
  // tile t).  The waits before the loop rely on a wave's copies completing
  // in the order they were issued.
  // At the top of iteration t every wave waits for all its copies, which are
  // those of tile t and the slots up to t+2.  The barrier then publishes tile
  // t and slots t+1 and ends all use of tile t-1 (or of the Q staging), whose
  // buffer tile t+1 overwrites while tile t is consumed.
  //
  // Passes: pass 0 computes the split against each row's first tile max.  If
  // a later tile beats that reference by more than REF_SLACK, pass 0 stops
  // and pass 1 sweeps every tile of the split for each row's exact max
  // (scores only, nothing accumulated); pass 2 then computes the split
  // against that max, which no tile can exceed, so no input needs a fourth.
  uint64_t anc_row = 0ull;
  for (int pass = 0;; ++pass) {
    const bool sweep = pass == 1;
#pragma unroll
    for (int c = 0; c < O_HALF; ++c) {
#pragma unroll
      for (int e = 0; e < 16; ++e) o[c][e] = 0.f;
    }
    l_run = 0.f;
    lb_run = 0.f;
    if (tid == 0) restart_sh = 0u;
    if (pass > 0) {
      if (ntiles > 0) {
        issue_slots(0);
        issue_slots(1);
      }
      wait_vmcnt<0>();
      __syncthreads();   // slots 0, 1 and restart_sh ready
    } else {
      // wave 0's slot and parent entries went out before its 18 Q copies
      vm_wait<COPIES>();
      __syncthreads();   // slots 0, 1, parents, status_sh and restart_sh ready
    }
    if (ntiles > 0) {
      // tile 0 goes out without waiting for Q, which fills the other buffer
      const TileIssue first_tile = prepare_tile(0, read_slots(0), tiles);
#pragma unroll
      for (int g = 0; g < 9; ++g) issue_part(first_tile, g);
      issue_slots(2);
    }
    if (pass == 0) {
      if (MODE != PREFIX && wave == 0) {
        int p = lane < T ? sring[SLOT_RING - 1][lane] : -1;
        if (p < -1 || p >= lane) {   // parents precede their children
          st |= VA_STATUS_BAD_PARENT;
          p = -1;
        }
        uint64_t m = lane < T ? 1ull << lane : 0ull;
        // every step moves to a smaller index, so the walk ends within T steps
        int x = p;
        while (__any(x >= 0)) {
          const int nx = __shfl(p, x >= 0 ? x : 0);
          if (x >= 0) {
            m |= 1ull << x;
            x = nx;
          }
        }
        anc[lane] = m;
      }
      // this wave's Q copies precede its tile-0 copies (and wave 0's slot copy)
      if (ntiles > 0) {
        if (wave == 0) vm_wait<COPIES + 1>();
        else vm_wait<COPIES>();
      } else {
        vm_wait<0>();
      }
      __syncthreads();   // Q and anc[] ready
      if (MODE != PREFIX) anc_row = row_ok ? anc[rho / H] : 0ull;
      const uint8_t* const qb = reinterpret_cast<const uint8_t*>(tiles + BUF_ELEMS);
      const int qr = rh * HALF + lrow;
#pragma unroll
      for (int k = 0; k < QK_STEPS; ++k)
        qf[k] = *reinterpret_cast<const bf16x8*>(qb + piece_off(qr, 2 * k + lh));
    }

    bool restart = false;
    bool restart_seen = false;   // restart_sh as of the last mid-tile barrier
    // slots of tile 1 (landed before the barrier above); each iteration reads
    // the slots of the tile after next, which landed at its top wait
    SlotPair vslot_next = read_slots(1);
    for (int t = 0; t < ntiles; ++t) {
      vm_wait<0>();
      lds_barrier();   // tile t is in LDS; every wave is done with tile t-1
      if (restart_seen && pass == 0) {   // uniform
        restart = true;
        break;
      }
      // the next tile's copies; after the last tile they copy the zero row
      // (every key lies past the split end) into the free buffer
      const TileIssue nxt = prepare_tile(t + 1, vslot_next, tiles + ((t + 1) & 1) * BUF_ELEMS);
      vslot_next = read_slots(t + 2);
      issue_slots(t + 3);
      compute(t, tiles + (t & 1) * BUF_ELEMS, anc_row, t == 0, nxt, sweep);
      if (!sweep) value_half(tiles + (t & 1) * BUF_ELEMS, kh, pown);
      lds_barrier();   // both key halves' probabilities are in LDS
      // every write of restart_sh (in compute) precedes the barrier above
      const uint32_t rs = restart_sh;
      if (!sweep) {
        bf16x8 poth[2];
        poth[0] = xp[rh][kh ^ 1][0][lane];
        poth[1] = xp[rh][kh ^ 1][1][lane];
        value_half(tiles + (t & 1) * BUF_ELEMS, kh ^ 1, poth);
      }
      restart_seen = __builtin_amdgcn_readfirstlane(rs) != 0u;
    }
    vm_wait<0>();
    __syncthreads();   // all copies landed and all waves are done with the tiles
    if (!restart) restart = sweep || (pass == 0 && restart_sh != 0u);
    if (!restart) break;
    // the reference of the next pass: the largest tile max either key half
    // has seen (after the sweep, the row's max over the whole split)
    if (lh == 0) xm[rh][kh][lrow] = m_seen;
    __syncthreads();
    m_ref = fmaxf(xm[rh][0][lrow], xm[rh][1][lrow]);
    __syncthreads();
  }

  // ---- store the normalised partial o / lb in fp16, in the MFMA output
  // layout: entry (rh * 16 + cb) * 4 + qd, lane holds the 4 columns qd of
  // register block cb: row rh*32 + lane%32, columns 32*cb + 8*qd +
  // 4*(lane/32) .. +3 (rows past T*H are never read).  Wave (rh, kh) holds
  // blocks 8*kh .. 8*kh+7.  Each row is scaled by 2^-e so that its largest
  // entry lies in [2^14, 2^15): any value range fits fp16, and fp16 keeps 11
  // significant bits, finer than the bf16 output.
  {
    // the row sums and largest |o| of the two column halves (the tile
    // buffers are free now)
    float* xr = reinterpret_cast<float*>(tiles);   // [rh][kh][3][32]: l, lb, max |o|
    const float l = l_run + __shfl_xor(l_run, 32);
    const float lb = lb_run + __shfl_xor(lb_run, 32);
    float amax = 0.f;
#pragma unroll
    for (int cb = 0; cb < O_HALF; ++cb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(o[cb][e]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (lh == 0) {
      xr[((rh * 2 + kh) * 3 + 0) * 32 + lrow] = l;
      xr[((rh * 2 + kh) * 3 + 1) * 32 + lrow] = lb;
      xr[((rh * 2 + kh) * 3 + 2) * 32 + lrow] = amax;
    }
    __syncthreads();
    const float lt = xr[((rh * 2 + 0) * 3 + 0) * 32 + lrow] + xr[((rh * 2 + 1) * 3 + 0) * 32 + lrow];
    const float lbt = xr[((rh * 2 + 0) * 3 + 1) * 32 + lrow] + xr[((rh * 2 + 1) * 3 + 1) * 32 + lrow];
    const float amx = fmaxf(xr[((rh * 2 + 0) * 3 + 2) * 32 + lrow], xr[((rh * 2 + 1) * 3 + 2) * 32 + lrow]);
    int ex = 0;
    float scale = 0.f;   // a row without visible keys stores zeros (its weight is 0)
    if (lbt > 0.f && amx > 0.f) {
      ex = ilogbf(amx / lbt) - 14;
      scale = ldexpf(1.f / lbt, -ex);
    }
    u32x2* po = reinterpret_cast<u32x2*>(a.part_o) + (int64_t)w * PART_VEC +
                (rh * O_BLK + kh * O_HALF) * 4 * 64 + lane;
#pragma unroll
    for (int cb = 0; cb < O_HALF; ++cb) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const f16x4 h = {(_Float16)(o[cb][4 * qd] * scale), (_Float16)(o[cb][4 * qd + 1] * scale),
                         (_Float16)(o[cb][4 * qd + 2] * scale), (_Float16)(o[cb][4 * qd + 3] * scale)};
        // streaming stores: the partials are read once, by the merge, and
        // leave no dirty lines for the end-of-kernel write-back
        __builtin_nontemporal_store(__builtin_bit_cast(u32x2, h), &po[(cb * 4 + qd) * 64]);
      }
    }
    if (kh == 0 && lh == 0) {
      const float lse2 = lt > 0.f ? m_ref + log2f(lt) : -INFINITY;
      *reinterpret_cast<float2*>(a.part_lse + ((int64_t)w * ROWS + rh * 32 + lrow) * 2) =
          make_float2(lse2, (float)ex);
    }
  }
  st |= bad;
  if (st) atomicOr(&status_sh, st);
  __syncthreads();
  if (tid == 0) a.status[w] = status_sh;
}

// ---- 128-row blocks over 32-key tiles (fused mode) ---------------------------
// The streaming design loads each KV tile once and computes every head on it
// ("The Execution Phase", section "The Core Design: A Streaming Flash
// Attention Kernel").  With many rows and long splits (a block's share of
// the prefix at least WIDE_MIN_KEYS keys, see verify_attn_plan_ex) a block
// here takes the two 64-row work items of a split that share a row
// pair (groups 2 gw and 2 gw + 1), so every KV row of the split enters the
// CU once for 128 rows instead of once per 64.  Wave w owns rows
// 32 w .. 32 w + 31 of the block entirely: the score of every key of a tile
// over all 576 columns (Q k-steps 0 .. QV-1 in VGPRs, the rest from LDS),
// its own softmax, and all 512 output columns (accumulators in the 256
// AGPRs).  No probabilities change hands, so a tile needs one barrier.
// Two 32-key tile buffers: a tile's copies go out during the score phase of
// the tile before (with three buffers and two tiles in flight, more of Q
// had to stay in registers and the kernel spilled more).  The partials are
// written as the two 64-row work items in the layout of va_partial_kernel,
// so the merge is the same.
//
// The value products are inline-asm MFMAs that accumulate in AGPRs: the
// compiler's hazard tracking does not see them, so the accumulators are
// zeroed and read only behind acc_settle, which gives the wait states and
// ties every later access of the accumulators to that point, and the
// probabilities (written by VALU instructions) get their wait states before
// the first value MFMA reads them.
constexpr int WROWS = 128;
// Prefix keys per block from which the planner picks these blocks.  Below,
// the doubled split count (partials to write and merge) and the larger Q
// prologue per block cost more than the halved KV ingest saves.
constexpr int WIDE_MIN_KEYS = 2048;
constexpr int WTILE = 32;
constexpr int WLINE = (WTILE / 8) * CHUNK;      // one line of all keys of a tile: 4 KB
constexpr int WBUF_BYTES = NLINE * WLINE;       // 36,864 B
constexpr int WBUF_ELEMS = WBUF_BYTES / 2;
constexpr int WNBUF = 2;                        // the next tile in flight while one is consumed
constexpr int WCOPIES = NLINE;                  // copies per wave per tile: 9 lines of its 8 keys
constexpr int WSLOT_RING = 4;
constexpr int QV = 16;   // score k-steps whose Q fragments stay in VGPRs; the rest are read from LDS

struct WideSmem {
  __attribute__((aligned(16))) uint16_t tiles[WNBUF * WBUF_ELEMS];
  // Q fragments of score k-steps QV .. 35 per wave, [wave][k - QV][lane]
  __attribute__((aligned(16))) bf16x8 qt[4][QK_STEPS - QV][64];
  int32_t sring[WSLOT_RING][WTILE];
  int32_t parents[64];
  uint64_t anc[VA_MAX_TREE];
  uint32_t status_sh;
  uint32_t restart_sh[2];   // set by tile t's waves in entry t % 2, read after the next barrier
};

__device__ __forceinline__ constexpr int wpiece_off(int k, int p) {
  return (p >> 3) * WLINE + (k >> 3) * CHUNK + (k & 7) * 128 + (((p & 7) ^ swz(k)) << 4);
}
// copy of line J of the wave's 8 keys: m0 = lds_w + (WLINE - 128) J, with the
// instruction offset 128 J advancing both addresses
template <int J>
__device__ __forceinline__ void wdma_line(uint32_t lds_w, const void* addr) {
  asm volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%3 nt"
               :: "s"(lds_w), "v"(addr), "n"((WLINE - 128) * J), "n"(128 * J)
               : "memory", "m0", "scc");
}
template <int... J>
__device__ __forceinline__ void wdma_copy(int c, uint32_t lds_w, const void* addr,
                                          std::integer_sequence<int, J...>) {
  ((c == J ? wdma_line<J>(lds_w, addr) : void()), ...);
}
// 16 bytes per lane from a per-lane address (lane i writes lds + 16 i)
__device__ __forceinline__ void dma16v(uint32_t lds, const void* addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(addr) : "memory", "m0");
}
// Wait states after the accumulating MFMAs (inline asm, which the compiler's
// hazard tracking does not see) before any other instruction touches the
// accumulators: the operands tie every later access of o to this point.
__device__ __forceinline__ void acc_settle(f32x16 (&o)[O_BLK]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                 "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
}
// O^T block += V^T fragment . P^T fragment, accumulating in AGPRs
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

template <bool ONE>
__device__ __forceinline__ void wide_body(const PartialArgs& a, const Lead& f, int block,
                                          WideSmem& sm) {
  uint16_t* const tiles = sm.tiles;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31;
  const int lh = lane >> 5;

  // blocks ordered (request, split, row pair); consecutive blocks in that
  // order go to one XCD (block b runs on XCD b % 8), as in va_partial_kernel
  const int items = f.total_work;   // blocks of this launch: sum of ns * ceil(G / 2)
  const int per_xcd = (items + 7) >> 3;
  int it = (block & 7) * per_xcd + (block >> 3);
  if (it >= items) return;
  int r = 0;
  if (!ONE) {
    for (;;) {   // uniform
      const int nb = a.nsplit[r] * ((a.num_groups[r] + 1) >> 1);
      if (r + 1 >= a.num_requests || it < nb) break;
      it -= nb;
      ++r;
    }
  }
  const int G = ONE ? f.g0 : a.num_groups[r];   // 64-row groups of the request
  const int GW = (G + 1) >> 1;                    // row pairs
  const int s = it / GW;
  const int gw = it - s * GW;
  const int ns = ONE ? f.ns0 : a.nsplit[r];
  const int T = ONE ? f.t0 : a.num_tree[r];
  const int H = f.num_heads;
  const int tb = ONE ? 0 : a.tree_begin[r];
  const int wb = ONE ? 0 : a.work_begin[r];       // the request's first work item
  const int rows_r = T * H;

  if (tid == 0) sm.status_sh = 0u;
  uint32_t st = 0u;
  const int maxp = ONE ? f.max_prefix0 : a.max_prefix[r];
  int L = f.prefix_len[r];
  if (L < 0 || L > maxp) {
    st |= VA_STATUS_BAD_PREFIX;
    L = L < 0 ? 0 : maxp;
  }
  const int n = L + T;
  const int tab0 = f.slot_indptr[r];
  const int tab1 = f.slot_indptr[r + 1];
  int n_valid = n;
  if (tab0 < 0 || tab1 < tab0 || tab1 > f.slot_table_len || tab1 - tab0 < n) {
    st |= VA_STATUS_SHORT_TABLE;
    n_valid = (tab0 < 0 || tab1 < tab0 || tab0 >= f.slot_table_len)
                  ? 0 : min(min(tab1, f.slot_table_len) - tab0, n);
  }
  // the split ranges of the fused mode: the L prefix keys in ns slices of
  // whole SPLIT_ALIGN blocks; the T draft keys go with the last slice
  const int chunk = ((L + ns - 1) / ns + SPLIT_ALIGN - 1) / SPLIT_ALIGN * SPLIT_ALIGN;
  const int k0 = min(s * chunk, L);
  const int k1 = min(n_valid, s == ns - 1 ? n : min(k0 + chunk, L));
  const int ntiles = k1 > k0 ? (k1 - k0 + WTILE - 1) / WTILE : 0;
  const int32_t* table = f.slot_table + (n_valid > 0 ? tab0 : 0);

  auto issue_slots = [&](int u) {
    if (wave == 0 && lane < WTILE) {
      const int k = min(k0 + u * WTILE + lane, k1 - 1);
      dma4_v(lds_addr(&sm.sring[u & (WSLOT_RING - 1)][0]), table + k);
    }
  };
  if (ntiles > 0) {
    issue_slots(0);
    issue_slots(1);
  }
  if (wave == 0) dma4_v(lds_addr(&sm.parents[0]), a.parent + tb + min(lane, T - 1));

  // ---- Q: this wave's 32 rows, all 576 score columns, straight into VGPRs
  // (B operand of S^T = K . Q^T: lane l holds row l % 32, columns
  // 16 k + 8 (l / 32) .. +7 of k-step k).  Rows past the request's end read
  // row 0: they repeat its scores and are never merged.
  const int rho = gw * WROWS + wave * 32 + lrow;   // row of the request
  const bool row_ok = rho < rows_r;
  bf16x8 qf[QV];
  {
    const uint16_t* qrow = f.q + ((int64_t)tb * H + (row_ok ? rho : 0)) * DQK + 8 * lh;
    // the tail k-steps into this wave's LDS area, lane l at 16 l (one copy each)
#pragma unroll
    for (int k = QV; k < QK_STEPS; ++k) dma16v(lds_addr(&sm.qt[wave][k - QV][0]), qrow + 16 * k);
#pragma unroll
    for (int k = 0; k < QV; ++k) qf[k] = *reinterpret_cast<const bf16x8*>(qrow + 16 * k);
  }

  // ---- tile loader: wave w copies the 9 lines of tile keys 8 w .. 8 w + 7;
  // lane l takes key 8 w + l / 8 and its piece (l % 8) ^ swz(key)
  uint32_t bad = 0u;
  struct WIssue {
    const uint16_t* src;
    uint32_t lds_w;
  };
  const int wkey = 8 * wave + (lane >> 3);
  auto prepare = [&](int u, int slot, int buf) -> WIssue {
    WIssue wi;
    wi.src = copy_source(a.kv, a.num_slots, a.stride, slot, k0 + u * WTILE + wkey < k1, wkey,
                         lane, bad);
    wi.lds_w = lds_addr(tiles + buf * WBUF_ELEMS) + wave * CHUNK;
    return wi;
  };
  auto issue_copy = [&](const WIssue& wi, int c) {
    wdma_copy(c, wi.lds_w, wi.src, std::make_integer_sequence<int, WCOPIES>{});
  };

  f32x16 o[O_BLK];
  float m_ref = -INFINITY;
  float m_seen = -INFINITY;
  float l_run = 0.f;
  float lb_run = 0.f;
  bf16x8 pown[2];

  uint32_t kb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kb[i] = wpiece_off(lrow, 2 * i + lh);
  uint32_t vb[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int nn = 0; nn < 2; ++nn)
      vb[c][nn] = wpiece_off(8 * nn + 4 * lh + ((lane & 15) >> 2),
                             4 * c + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + (lane & 1) * 8;
  }
  const int qkey = 4 * lh;   // tile key of register 4 qd + i is qkey + 8 qd + i

  auto compute = [&](int t, int buf, uint64_t anc_row, bool first, const WIssue& nxt, bool sweep) {
    const uint8_t* const bp = reinterpret_cast<const uint8_t*>(tiles + buf * WBUF_ELEMS);
    const int kt = k0 + t * WTILE;
    f32x16 sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
    constexpr int QG = 4;
    // per-tile LDS addresses of this lane's K pieces, opaque to the compiler so
    // that each read is base + an instruction offset (no hoisted address per read)
    uint32_t kbase[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kbase[i] = lds_addr(bp) + kb[i];
      asm volatile("" : "+v"(kbase[i]));
    }
    auto load_k = [&](bf16x8* kf, bf16x8* qx, int k0s) {
#pragma unroll
      for (int kk = 0; kk < QG; ++kk) {
        const int k = k0s + kk;
        kf[kk] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            (uintptr_t)(kbase[k & 3] + WLINE * (k >> 2)));
        if (k >= QV) qx[kk] = sm.qt[wave][k - QV][lane];
      }
    };
    bf16x8 kfa[QG], kfb[QG], qxa[QG], qxb[QG];
    load_k(kfa, qxa, 0);
#pragma unroll
    for (int g = 0; g < QK_STEPS / QG; ++g) {
      bf16x8* cur = (g & 1) ? kfb : kfa;
      bf16x8* ahead = (g & 1) ? kfa : kfb;
      bf16x8* qcur = (g & 1) ? qxb : qxa;
      bf16x8* qahead = (g & 1) ? qxa : qxb;
      if (g + 1 < QK_STEPS / QG) load_k(ahead, qahead, (g + 1) * QG);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < QG; ++kk) {
        const int k = g * QG + kk;
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[kk], k < QV ? qf[k < QV ? k : 0] : qcur[kk],
                                                       sacc, 0, 0, 0);
      }
      issue_copy(nxt, g);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + WTILE > L || kt + WTILE > k1) {   // uniform
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kp = kt + qkey + 8 * (e >> 2) + (e & 3);
        const int d = kp - L;
        const bool in_tree = d < 0 || ((anc_row >> (d & 63)) & 1ull);
        sacc[e] = (kp < k1 && in_tree) ? sacc[e] : -INFINITY;
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                       __builtin_bit_cast(uint32_t, mx), false, false);
      mx = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
    }
    mx *= a.scale_log2;
    m_seen = fmaxf(m_seen, mx);
    if (sweep) return;
    if (first) {
      if (m_ref == -INFINITY) m_ref = mx;
    } else if (mx > m_ref + REF_SLACK) {
      sm.restart_sh[t & 1] = 1u;
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * ks + i], a.scale_log2, -m_use));
      l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      bf16x2 pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = bf16x2{(__bf16)p[2 * i], (__bf16)p[2 * i + 1]};
        lb_run = __builtin_amdgcn_fdot2_f32_bf16(pb[i], ones, lb_run, false);
      }
      pown[ks] = __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(uint32_t, pb[0]),
                                                   __builtin_bit_cast(uint32_t, pb[1]),
                                                   __builtin_bit_cast(uint32_t, pb[2]),
                                                   __builtin_bit_cast(uint32_t, pb[3])});
    }
  };

  // O^T += V^T . P^T over the tile's 32 keys: 16 column blocks x 2 k-steps,
  // V^T fragments by transpose reads one block ahead
  auto value = [&](int buf) {
    uint32_t vbase[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        vbase[c][nn] = lds_addr(tiles + buf * WBUF_ELEMS) + vb[c][nn];
        asm volatile("" : "+v"(vbase[c][nn]));
      }
    }
    auto load_v2 = [&](bf16x8* vf, int cb) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t off = (cb >> 1) * WLINE + j * (2 * CHUNK);
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vbase[cb & 1][0] + off));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(vbase[cb & 1][1] + off));
        const i16x8 v8 = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        vf[j] = __builtin_bit_cast(bf16x8, v8);
      }
    };
    bf16x8 vfa[2], vfb[2];
    load_v2(vfa, 0);
    // the probabilities were just written by vector ALU instructions
    asm volatile("s_nop 4" : "+v"(pown[0]), "+v"(pown[1]));
#pragma unroll
    for (int cb = 0; cb < O_BLK; cb += 2) {
      load_v2(vfb, cb + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j) mfma_acc(o[cb], vfa[j], pown[j]);
      __builtin_amdgcn_sched_barrier(0);
      if (cb + 2 < O_BLK) load_v2(vfa, cb + 2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j) mfma_acc(o[cb + 1], vfb[j], pown[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  uint64_t anc_row = 0ull;
  for (int pass = 0;; ++pass) {
    const bool sweep = pass == 1;
    // accumulator writes after the last pass's accumulating MFMAs, and the
    // first accumulating MFMA after the writes
    if (pass > 0) acc_settle(o);
#pragma unroll
    for (int c = 0; c < O_BLK; ++c) {
#pragma unroll
      for (int e = 0; e < 16; ++e) o[c][e] = 0.f;
    }
    acc_settle(o);
    l_run = 0.f;
    lb_run = 0.f;
    if (tid == 0) {
      sm.restart_sh[0] = 0u;
      sm.restart_sh[1] = 0u;
    }
    if (pass > 0) {
      if (ntiles > 0) {
        issue_slots(0);
        issue_slots(1);
      }
      vm_wait<0>();
    } else {
      // wave 0: slots 0, 1 and the parents went out before its 36 Q copies and loads
      vm_wait<QK_STEPS>();
    }
    __syncthreads();   // slots 0, 1 (and parents) in LDS; status_sh, restart_sh set
    if (ntiles > 0) {
      const WIssue t0i = prepare(0, sm.sring[0][wkey], 0);
#pragma unroll
      for (int c = 0; c < WCOPIES; ++c) issue_copy(t0i, c);
    }
    if (pass == 0 && wave == 0) {
      int p = lane < T ? sm.parents[lane] : -1;
      if (p < -1 || p >= lane) {   // parents precede their children
        st |= VA_STATUS_BAD_PARENT;
        p = -1;
      }
      uint64_t m = lane < T ? 1ull << lane : 0ull;
      int x = p;
      while (__any(x >= 0)) {
        const int nx = __shfl(p, x >= 0 ? x : 0);
        if (x >= 0) {
          m |= 1ull << x;
          x = nx;
        }
      }
      sm.anc[lane] = m;
    }

    bool restart = false;
    for (int t = 0; t < ntiles; ++t) {
      // tile t (and the slots of tile t + 1) landed: nothing else is in flight
      vm_wait<0>();
      lds_barrier();   // tile t and slots t + 1 in LDS; every wave is done with tile t - 1
      if (t == 0 && pass == 0) anc_row = row_ok ? sm.anc[rho / H] : 0ull;
      // tile t - 1's restart requests: all written before the barrier above,
      // and entry (t - 1) % 2 is not written again before the next barrier
      if (pass == 0 && t > 0 &&
          __builtin_amdgcn_readfirstlane(sm.restart_sh[(t - 1) & 1]) != 0u) {   // uniform
        restart = true;
        break;
      }
      // tile t + 1 goes into the buffer tile t - 1 left
      const WIssue nxt = prepare(t + 1, sm.sring[(t + 1) & (WSLOT_RING - 1)][wkey], (t + 1) % WNBUF);
      issue_slots(t + 2);
      compute(t, t % WNBUF, anc_row, t == 0, nxt, sweep);
      if (!sweep) value(t % WNBUF);
    }
    vm_wait<0>();
    __syncthreads();
    if (!restart) restart = sweep || (pass == 0 && (sm.restart_sh[0] | sm.restart_sh[1]) != 0u);
    if (!restart) break;
    m_ref = m_seen;
    __syncthreads();
  }
  acc_settle(o);

  // ---- store o / lb in fp16 as the block's two 64-row work items
  {
    const float l = l_run + __shfl_xor(l_run, 32);
    const float lb = lb_run + __shfl_xor(lb_run, 32);
    float amax = 0.f;
#pragma unroll
    for (int cb = 0; cb < O_BLK; ++cb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(o[cb][e]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    int ex = 0;
    float scale = 0.f;
    if (lb > 0.f && amax > 0.f) {
      ex = ilogbf(amax / lb) - 14;
      scale = ldexpf(1.f / lb, -ex);
    }
    const int vg = 2 * gw + (wave >> 1);        // this wave's row group
    const int rh = wave & 1;
    if (vg < G) {
      const int w = wb + s * G + vg;   // the 64-row work item
      u32x2* po = reinterpret_cast<u32x2*>(a.part_o) + (int64_t)w * PART_VEC + rh * O_BLK * 4 * 64 + lane;
#pragma unroll
      for (int cb = 0; cb < O_BLK; ++cb) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f16x4 h = {(_Float16)(o[cb][4 * qd] * scale), (_Float16)(o[cb][4 * qd + 1] * scale),
                           (_Float16)(o[cb][4 * qd + 2] * scale), (_Float16)(o[cb][4 * qd + 3] * scale)};
          __builtin_nontemporal_store(__builtin_bit_cast(u32x2, h), &po[(cb * 4 + qd) * 64]);
        }
      }
      if (lh == 0) {
        const float lse2 = l > 0.f ? m_ref + log2f(l) : -INFINITY;
        *reinterpret_cast<float2*>(a.part_lse + ((int64_t)w * ROWS + rh * 32 + lrow) * 2) =
            make_float2(lse2, (float)ex);
      }
    }
  }
  st |= bad;
  if (st) atomicOr(&sm.status_sh, st);
  __syncthreads();
  if (tid < 2) {
    const int vg = 2 * gw + tid;
    if (vg < G) a.status[wb + s * G + vg] = sm.status_sh;
  }
}

template <bool ONE>
__global__ __launch_bounds__(THREADS, 1) void va_wide_kernel(
    const int32_t* prefix_len, const int32_t* slot_indptr, const int32_t* slot_table,
    const uint16_t* q, int32_t items, int32_t num_heads, int32_t slot_table_len, int32_t ns0,
    int32_t g0, int32_t t0, int32_t max_prefix0, PartialArgs a) {
  __shared__ WideSmem sm;
  const Lead f{prefix_len, slot_indptr, slot_table, q, items, num_heads, slot_table_len,
               ns0, g0, t0, max_prefix0};
  wide_body<ONE>(a, f, blockIdx.x, sm);
}

// Log-sum-exp merge of the splits.  One block per (request, row group, row
// half, 32-column block, 4-column quad): 32 rows x 8 columns, read as one
// contiguous 512-byte piece per split; with QPB = 4, all four quads of the
// 32-column block (four consecutive pieces, wave q finishing quad q).  The
// block has 256 threads for up to 64 splits and 512 beyond (red_threads):
// with few splits the shorter barriers of four waves pay, with many the
// eight waves' loads in flight.  All of the block's loads go out together,
// so the merge costs one memory round trip: thread (split group sg, row)
// loads the (lse, scale exponent e) pairs of splits sg, sg + SG, ...
// (SG = threads / 32), wave v the pieces of splits v, v + W, ...
// (W = threads / 64), and thread i the status word of split i.  Loads past
// the request's last split re-read that split (in bounds, no branch around
// any load): they leave the row max unchanged and enter the sums with
// coefficient 0.  Then, on registers and LDS: the row max over the splits,
// the coefficients exp2(lse_s - max) * 2^e_s, each wave's weighted sum of
// its pieces, and the sum over the waves.
constexpr int RED_PIECES = 2 * O_BLK * 4;   // blocks per row group
constexpr int red_threads(int maxs) { return maxs <= 64 ? 256 : 512; }

// MAXS: a bound on every request's split count, a multiple of the split
// groups (red_threads(MAXS) / 32).
// The pointers and, when ONE (a single request), that request's split count,
// row groups and rows come as leading scalar parameters, preloaded into
// scalar registers like the partial kernel's (see Lead), so the first loads
// need no kernel-argument load.
template <int MAXS, int QPB, bool ONE>
__global__ __launch_bounds__(red_threads(MAXS)) void va_reduce_kernel(
    const uint32_t* part_o, const float* part_lse, const uint32_t* status, uint16_t* out,
    float* lse, int32_t ns0, int32_t g0, int32_t rows0, int32_t num_heads, ReduceArgs a) {
  constexpr int RED_WAVES = red_threads(MAXS) / 64;
  constexpr int RED_SG = red_threads(MAXS) / 32;    // split groups of the lse loads
  static_assert(MAXS % RED_SG == 0 && MAXS % RED_WAVES == 0, "split bound");
  constexpr int RED_LSE = MAXS / RED_SG;           // lse pairs per thread
  constexpr int RED_PER_WAVE = MAXS / RED_WAVES;   // splits per wave
  constexpr int BPG = RED_PIECES / QPB;            // blocks per row group
  static_assert(QPB == 1 || (QPB == 4 && RED_WAVES >= 4), "quads per block");
  __shared__ float coef[MAXS][32];
  __shared__ float red_m[RED_SG][32];
  __shared__ float red_w[RED_SG][32];
  __shared__ f32x4 part[RED_WAVES][QPB][64];
  __shared__ uint32_t bad_w[RED_WAVES];   // per wave: a split status it loaded is nonzero

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform: the split of each partial load, its address and its
  // bounds test are scalar work
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int b = blockIdx.x;
  int r = 0;
  // block ranges: request r owns num_groups[r] * BPG blocks
  if (!ONE) {
    while (r + 1 < a.num_requests && b >= a.num_groups[r] * BPG) {
      b -= a.num_groups[r] * BPG;
      ++r;
    }
  }
  const int g = b / BPG;
  const int piece = (b - g * BPG) * QPB;   // first piece: (rh * 16 + cb) * 4 + qd
  const int rh = piece / (O_BLK * 4);
  const int cb = (piece >> 2) % O_BLK;
  const int qd = piece & 3;
  const int ns = ONE ? ns0 : a.nsplit[r];
  const int G = ONE ? g0 : a.num_groups[r];
  const int H = num_heads;
  const int rows_r = ONE ? rows0 : (a.tree_begin[r + 1] - a.tree_begin[r]) * H;
  const int tb = ONE ? 0 : a.tree_begin[r];
  const int64_t wbase = (int64_t)(ONE ? 0 : a.work_begin[r]) + g;   // work item of split s: wbase + s * G

  const int row = tid & 31;
  const int sg = tid >> 5;   // 2 wave + lane / 32
  const int prow = lane & 31;
  // lse pair of split s: plse[s * lse_step] (s * lse_step < 2^31: at most
  // 256 splits of at most 1024 row groups of 64 rows)
  const float2* plse = reinterpret_cast<const float2*>(part_lse) + wbase * ROWS + rh * 32 + row;
  const int lse_step = G * ROWS;
  const u32x2* src = reinterpret_cast<const u32x2*>(part_o) + wbase * PART_VEC + piece * 64;
  const int64_t split_step = (int64_t)G * PART_VEC;
  float2 lv[RED_LSE];
  {
    const float2* const last = plse + (ns - 1) * lse_step;
    const float2* lp = plse + sg * lse_step;
#pragma unroll
    for (int i = 0; i < RED_LSE; ++i) {
      lv[i] = *(sg + i * RED_SG < ns ? lp : last);
      lp += RED_SG * lse_step;
    }
  }
  const uint32_t st = status[wbase + (int64_t)min(tid, ns - 1) * G];
  u32x2 v[RED_PER_WAVE][QPB];
  {
    // uniform addresses: split wave + u W by steps of W splits, the request's
    // last split once past it
    const u32x2* const last = src + (ns - 1) * split_step;
    const u32x2* ps = src + wave * split_step;
#pragma unroll
    for (int u = 0; u < RED_PER_WAVE; ++u) {
      const u32x2* const pu = wave + u * RED_WAVES < ns ? ps : last;
#pragma unroll
      for (int q = 0; q < QPB; ++q) v[u][q] = __builtin_nontemporal_load(pu + q * 64 + lane);   // read once
      ps += RED_WAVES * split_step;
    }
  }

  // per-row max over the splits (the re-read copies of the last split
  // leave it unchanged)
  float m = lv[0].x;
#pragma unroll
  for (int i = 1; i < RED_LSE; ++i) m = fmaxf(m, lv[i].x);
  red_m[sg][row] = m;
  // the status words: one flag per wave, read by the finishing waves after
  // the barriers below (a block-wide reduction would cost barriers of its own)
  const bool wave_bad = __builtin_amdgcn_ballot_w64(st != 0u) != 0ull;
  if (lane == 0) bad_w[wave] = wave_bad ? 1u : 0u;
  __syncthreads();
  float M = red_m[0][row];
#pragma unroll
  for (int i = 1; i < RED_SG; ++i) M = fmaxf(M, red_m[i][row]);
  // coefficients and weight sums, without branches: splits past the
  // request's last (s < MAXS, so inside the table) get coefficient 0, as do
  // empty splits (lse -inf) and every split of a row without keys (M -inf).
  // The hardware exp2 (no rescaling below 2^-126) may return 0 for weights
  // under 2^-126 of the largest: a term that small moves the output only if
  // the split's values exceed the output's by a factor near 2^126.
  const bool row_on = M != -INFINITY;
  float wsum = 0.f;
#pragma unroll
  for (int i = 0; i < RED_LSE; ++i) {
    const int s = sg + i * RED_SG;
    const float e = __builtin_amdgcn_exp2f(s < ns && row_on ? lv[i].x - M : -INFINITY);
    wsum += e;
    coef[s][row] = ldexpf(e, (int)lv[i].y);
  }
  red_w[sg][row] = wsum;
  __syncthreads();

  // weighted sum of this wave's pieces.  Partials are finite (a row without
  // visible keys stores zeros), so a split whose coefficient is 0, including
  // the re-read copies of the last split, adds an exact 0.
  f32x4 acc[QPB];
#pragma unroll
  for (int q = 0; q < QPB; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < RED_PER_WAVE; ++u) {
    const float c = coef[wave + u * RED_WAVES][prow];
#pragma unroll
    for (int q = 0; q < QPB; ++q) {
      const f16x4 h = __builtin_bit_cast(f16x4, v[u][q]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[q][i] = __builtin_fmaf(c, (float)h[i], acc[q][i]);
    }
  }
#pragma unroll
  for (int q = 0; q < QPB; ++q) part[wave][q][lane] = acc[q];
  __syncthreads();
  // wave q < QPB finishes quad qd + q
  if (wave < QPB) {
    const int qq = QPB == 1 ? 0 : wave;
    f32x4 tot = part[0][qq][lane];
#pragma unroll
    for (int i = 1; i < RED_WAVES; ++i) tot += part[i][qq][lane];
    // this thread's row is prow, whose max M it took above
    float W = 0.f;
    uint32_t Sr = 0u;
#pragma unroll
    for (int i = 0; i < RED_WAVES; ++i) Sr |= bad_w[i];
#pragma unroll
    for (int i = 0; i < RED_SG; ++i) W += red_w[i][prow];
    const int rr = g * ROWS + rh * 32 + prow;   // row within the request
    if (rr < rows_r) {
      float res[4];
      float lse_out;
      if (Sr != 0u) {
        res[0] = res[1] = res[2] = res[3] = NAN;
        lse_out = NAN;
      } else if (W > 0.f) {
        const float inv = 1.f / W;
        res[0] = tot[0] * inv; res[1] = tot[1] * inv; res[2] = tot[2] * inv; res[3] = tot[3] * inv;
        lse_out = (M + log2f(W)) * LN2;
      } else {
        res[0] = res[1] = res[2] = res[3] = 0.f;
        lse_out = -INFINITY;
      }
      const int64_t orow = (int64_t)tb * H + rr;
      const int col = cb * 32 + 8 * (qd + qq) + 4 * (lane >> 5);
      // round to nearest even (v_cvt_pk_bf16_f32)
      const uint32_t lo = bf16_pair(res[0], res[1]);
      const uint32_t hi = bf16_pair(res[2], res[3]);
      *reinterpret_cast<uint2*>(out + orow * DV + col) = make_uint2(lo, hi);
      if (((piece + qq) & (O_BLK * 4 - 1)) == 0 && lane < 32) lse[orow] = lse_out;   // once per row
    }
  }
}

// Measurement helper: the read ceiling the partial pass is compared with.
// Every 16-byte word of buf is read once (streaming loads, four in flight
// per thread); block b folds the XOR of the 32-bit words it read into
// sink[b % sink_words], so the reads cannot be dropped and a test can check
// that each word was read exactly once.  With sink_words at least the grid
// size no two blocks share a sink word (atomics on one word serialise).
constexpr int STREAM_THREADS = 256;
constexpr int STREAM_BLOCKS_PER_CU = 8;
__global__ __launch_bounds__(STREAM_THREADS) void va_stream_read_kernel(const u32x4* buf, int64_t n16,
                                                                          uint32_t* sink, int sink_words) {
  __shared__ uint32_t part[STREAM_THREADS / 64];
  const int64_t stride = (int64_t)gridDim.x * STREAM_THREADS;
  int64_t i = (int64_t)blockIdx.x * STREAM_THREADS + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    const u32x4 b = __builtin_nontemporal_load(buf + i + stride);
    const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0u;
    for (int w = 0; w < STREAM_THREADS / 64; ++w) t ^= part[w];
    atomicXor(sink + blockIdx.x % sink_words, t);
  }
}

// Diagnostic: pool rows through the partial kernel's own tile loader, one
// block per 64-key tile: its slot-ring copy of the table entries, its lane
// roles and copy sources (tile_key, copy_source), its copy instructions
// (dma_part) and its LDS tile layout (piece_off), then the rows read back out
// of the tile in table order.
__global__ __launch_bounds__(THREADS) void va_gather_kernel(const uint16_t* kv, int64_t num_slots,
                                                            int32_t stride, const int32_t* table,
                                                            int32_t n, uint16_t* dst) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[BUF_ELEMS];
  __shared__ int32_t ring[TILE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k0 = blockIdx.x * TILE;
  const int k1 = min(n, k0 + TILE);
  // the slot entries of the tile, as the partial kernel's slot ring gets them
  if (wave == 0) dma4_v(lds_addr(ring), table + min(k0 + lane, k1 - 1));
  wait_vmcnt<0>();
  __syncthreads();
  // the partial kernel's copies of one tile: its lane roles, sources and
  // copy instructions, into its LDS layout
  uint32_t bad = 0u;
  const uint16_t* src[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int key = tile_key(wave, e, lane);
    src[e] = copy_source(kv, num_slots, stride, ring[key], k0 + key < k1, key, lane, bad);
  }
  const uint32_t lds_w = lds_addr(tile) + 2 * wave * CHUNK;
#pragma unroll
  for (int part = 0; part < COPIES / 2; ++part)
    dma_part(part, lds_w, src[0], src[1], std::make_integer_sequence<int, COPIES / 2>{});
  vm_wait<0>();
  __syncthreads();
  // rows back out of the tile layout (NaN rows for slots outside the pool)
  for (int i = tid; i < TILE * NPIECE; i += THREADS) {
    const int key = i / NPIECE;
    const int p = i - key * NPIECE;
    if (k0 + key >= k1) continue;
    const int32_t slot = ring[key];
    u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(tile) + piece_off(key, p));
    if (slot < 0 || (int64_t)slot >= num_slots) v = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
    *reinterpret_cast<u32x4*>(dst + (int64_t)(k0 + key) * DQK + p * 8) = v;
  }
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
  if (p == nullptr || p->magic != VA_PLAN_MAGIC || p->version != VA_PLAN_VERSION ||
      p->num_requests < 1 || p->num_requests > VA_MAX_REQUESTS || p->total_work < 1 ||
      p->rows_per_group != ROWS || p->tile_keys != TILE ||
      (p->mode != VA_MODE_FUSED && p->mode != VA_MODE_SPLIT_TREE))
    return false;
  // 128-row blocks: fused mode only
  if (p->groups_per_block != 1 && (p->groups_per_block != 2 || p->mode != VA_MODE_FUSED))
    return false;
  // the derived tables must be the ones the planner writes: the kernels
  // index through them without further checks
  if (p->num_heads < 1 || p->work_begin[0] != 0 || p->tree_begin[0] != 0) return false;
  const int min_ns = p->mode == VA_MODE_SPLIT_TREE ? 2 : 1;   // split: a prefix split + the tree block
  for (int r = 0; r < p->num_requests; ++r) {
    const int T = p->num_tree[r];
    if (T < 1 || T > VA_MAX_TREE || p->tree_begin[r + 1] - p->tree_begin[r] != T) return false;
    if (p->nsplit[r] < min_ns || p->nsplit[r] > VA_MAX_SPLITS) return false;
    if (p->num_groups[r] != (T * p->num_heads + ROWS - 1) / ROWS) return false;
    if ((int64_t)p->work_begin[r + 1] - p->work_begin[r] != (int64_t)p->nsplit[r] * p->num_groups[r])
      return false;
  }
  const int64_t work = p->total_work;
  const int64_t o_bytes = align256(work * ROWS * DV * (int64_t)sizeof(uint16_t));
  const int64_t lse_bytes = align256(work * ROWS * 2 * (int64_t)sizeof(float));
  const int64_t st_bytes = align256(work * (int64_t)sizeof(uint32_t));
  return p->work_begin[p->num_requests] == p->total_work &&
         p->total_tree == p->tree_begin[p->num_requests] &&
         (int64_t)p->total_rows == (int64_t)p->total_tree * p->num_heads &&
         p->lse_offset == o_bytes && p->status_offset == o_bytes + lse_bytes &&
         p->workspace_bytes == o_bytes + lse_bytes + st_bytes;
}

// Checks of the launch arguments verify_attn_run and verify_attn_forward_static share.
int check_run_args(const va_plan* plan, const uint16_t* q, const uint16_t* kv_pool,
                   int64_t num_slots, int32_t kv_row_stride, const int32_t* slot_table,
                   int32_t slot_table_len, const int32_t* slot_indptr, const int32_t* prefix_len,
                   const int32_t* parent, float sm_scale) {
  if (plan == nullptr || q == nullptr || kv_pool == nullptr || slot_table == nullptr ||
      slot_indptr == nullptr || prefix_len == nullptr || parent == nullptr)
    return VA_ERR_NULL;
  if (!plan_ok(plan)) return VA_ERR_PLAN;
  if (num_slots < 1 || num_slots > (int64_t)INT32_MAX + 1 || kv_row_stride < DQK ||
      slot_table_len < 0 || !std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return VA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(kv_pool) || (kv_row_stride % 8) != 0) return VA_ERR_ALIGN;
  return VA_OK;
}

// The partial pass into workspace ws (checked by the caller).
int launch_partial(const va_plan* plan, const uint16_t* q, const uint16_t* kv_pool,
                   int64_t num_slots, int32_t kv_row_stride, const int32_t* slot_table,
                   int32_t slot_table_len, const int32_t* slot_indptr, const int32_t* prefix_len,
                   const int32_t* parent, float sm_scale, char* ws, hipStream_t st) {
  PartialArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = q;
  a.kv = kv_pool;
  a.num_slots = num_slots;
  a.stride = kv_row_stride;
  a.num_requests = plan->num_requests;
  a.num_heads = plan->num_heads;
  a.total_work = plan->total_work;
  a.scale_log2 = sm_scale * LOG2E;
  a.slot_table = slot_table;
  a.slot_table_len = slot_table_len;
  a.slot_indptr = slot_indptr;
  a.prefix_len = prefix_len;
  a.parent = parent;
  a.part_o = reinterpret_cast<uint32_t*>(ws);
  a.part_lse = reinterpret_cast<float*>(ws + plan->lse_offset);
  a.status = reinterpret_cast<uint32_t*>(ws + plan->status_offset);
  for (int r = 0; r < plan->num_requests; ++r) {
    a.num_tree[r] = plan->num_tree[r];
    a.max_prefix[r] = plan->max_prefix[r];
    a.nsplit[r] = plan->nsplit[r];
    a.num_groups[r] = plan->num_groups[r];
  }
  for (int r = 0; r <= plan->num_requests; ++r) {
    a.tree_begin[r] = plan->tree_begin[r];
    a.work_begin[r] = plan->work_begin[r];
  }
  const unsigned grid = 8u * (unsigned)((plan->total_work + 7) / 8);   // see the XCD work order
  // request 0's values for the single-request instantiations (see Lead)
  const int ns0 = plan->nsplit[0], g0 = plan->num_groups[0], t0 = plan->num_tree[0];
  const int mp0 = plan->max_prefix[0];
  if (plan->mode == VA_MODE_SPLIT_TREE) {
    int tree_blocks = 0;
    for (int r = 0; r < plan->num_requests; ++r) tree_blocks += plan->num_groups[r];
    if (plan->num_requests == 1)
      hipLaunchKernelGGL(va_split_kernel<true>, dim3(grid + (unsigned)tree_blocks), dim3(THREADS), 0,
                         st, prefix_len, slot_indptr, slot_table, q, tree_blocks, a.total_work,
                         a.num_heads, slot_table_len, ns0, g0, t0, mp0, a);
    else
      hipLaunchKernelGGL(va_split_kernel<false>, dim3(grid + (unsigned)tree_blocks), dim3(THREADS),
                         0, st, prefix_len, slot_indptr, slot_table, q, tree_blocks, a.total_work,
                         a.num_heads, slot_table_len, ns0, g0, t0, mp0, a);
  } else if (plan->groups_per_block == 2) {
    // one block per (request, split, row pair), in XCD order (see wide_body)
    int blocks = 0;
    for (int r = 0; r < plan->num_requests; ++r)
      blocks += plan->nsplit[r] * ((plan->num_groups[r] + 1) / 2);
    const unsigned wgrid = 8u * (unsigned)((blocks + 7) / 8);
    if (plan->num_requests == 1)
      hipLaunchKernelGGL(va_wide_kernel<true>, dim3(wgrid), dim3(THREADS), 0, st, prefix_len,
                         slot_indptr, slot_table, q, blocks, a.num_heads, slot_table_len, ns0, g0,
                         t0, mp0, a);
    else
      hipLaunchKernelGGL(va_wide_kernel<false>, dim3(wgrid), dim3(THREADS), 0, st, prefix_len,
                         slot_indptr, slot_table, q, blocks, a.num_heads, slot_table_len, ns0, g0,
                         t0, mp0, a);
  } else {
    if (plan->num_requests == 1)
      hipLaunchKernelGGL(va_partial_kernel<true>, dim3(grid), dim3(THREADS), 0, st, prefix_len,
                         slot_indptr, slot_table, q, a.total_work, a.num_heads, slot_table_len, ns0,
                         g0, t0, mp0, a);
    else
      hipLaunchKernelGGL(va_partial_kernel<false>, dim3(grid), dim3(THREADS), 0, st, prefix_len,
                         slot_indptr, slot_table, q, a.total_work, a.num_heads, slot_table_len, ns0,
                         g0, t0, mp0, a);
  }
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

// The merge of the partials in workspace ws (checked by the caller).
int launch_reduce(const va_plan* plan, const char* ws, uint16_t* out, float* lse, hipStream_t st) {
  ReduceArgs a;
  std::memset(&a, 0, sizeof a);
  a.part_o = reinterpret_cast<const uint32_t*>(ws);
  a.part_lse = reinterpret_cast<const float*>(ws + plan->lse_offset);
  a.status = reinterpret_cast<const uint32_t*>(ws + plan->status_offset);
  a.out = out;
  a.lse = lse;
  a.num_requests = plan->num_requests;
  a.num_heads = plan->num_heads;
  for (int r = 0; r < plan->num_requests; ++r) {
    a.nsplit[r] = plan->nsplit[r];
    a.num_groups[r] = plan->num_groups[r];
  }
  for (int r = 0; r <= plan->num_requests; ++r) {
    a.tree_begin[r] = plan->tree_begin[r];
    a.work_begin[r] = plan->work_begin[r];
  }
  int groups = 0;
  int max_ns = 1;
  for (int r = 0; r < plan->num_requests; ++r) {
    groups += plan->num_groups[r];
    max_ns = max(max_ns, plan->nsplit[r]);
  }
  // With up to 64 splits (four-wave blocks) and more one-quad blocks than
  // one round of the CUs holds (eight four-wave blocks each), a block takes
  // all four quads of a 32-column block: one round of blocks instead of
  // several.  The output is the same bit for bit (same splits per wave, same
  // summation order).
  const bool quads = max_ns <= 64 && groups * RED_PIECES > 8 * plan->num_cus;
  const bool one = plan->num_requests == 1;
  const int ns0 = plan->nsplit[0], g0 = plan->num_groups[0];
  const int rows0 = plan->num_tree[0] * plan->num_heads;
  auto launch = [&](auto k1, auto k0, int threads, int qpb) {
    const int blocks = groups * (RED_PIECES / qpb);
    if (one)
      hipLaunchKernelGGL(k1, dim3(blocks), dim3(threads), 0, st, a.part_o, a.part_lse,
                         a.status, out, lse, ns0, g0, rows0, a.num_heads, a);
    else
      hipLaunchKernelGGL(k0, dim3(blocks), dim3(threads), 0, st, a.part_o, a.part_lse,
                         a.status, out, lse, ns0, g0, rows0, a.num_heads, a);
  };
#define VA_RED(M) launch(va_reduce_kernel<M, 1, true>, va_reduce_kernel<M, 1, false>, red_threads(M), 1)
#define VA_RED4(M) launch(va_reduce_kernel<M, 4, true>, va_reduce_kernel<M, 4, false>, red_threads(M), 4)
  if (max_ns <= 16 && quads) VA_RED4(16);
  else if (max_ns <= 16) VA_RED(16);
  else if (max_ns <= 32 && quads) VA_RED4(32);
  else if (max_ns <= 32) VA_RED(32);
  else if (max_ns <= 64 && quads) VA_RED4(64);
  else if (max_ns <= 64) VA_RED(64);
  else if (max_ns <= 128) VA_RED(128);
  else VA_RED(VA_MAX_SPLITS);
#undef VA_RED
#undef VA_RED4
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept for the process.
static_assert(VA_STATIC_SCRATCH_BYTES ==
                  (int64_t)VA_STATIC_SCRATCH_WORK * (ROWS * DV * 2 + ROWS * 2 * 4) +
                      ((VA_STATIC_SCRATCH_WORK * 4 + 255) & ~255),
              "scratch = the workspace of VA_STATIC_SCRATCH_WORK work items");
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mutex;
void* scratch_ptr[SCRATCH_MAX_DEVICES] = {};

int static_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return VA_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return VA_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(scratch_ptr[dev]);
  return VA_OK;
}

}  // namespace

extern "C" {

int verify_attn_plan(int32_t num_requests, int32_t num_heads, const int32_t* h_prefix_len,
                     const int32_t* h_num_tree, int32_t num_cus, va_plan* plan,
                     size_t* workspace_bytes) {
  return verify_attn_plan_ex(num_requests, num_heads, h_prefix_len, h_num_tree, num_cus, 0u, plan,
                             workspace_bytes);
}

int verify_attn_plan_ex(int32_t num_requests, int32_t num_heads, const int32_t* h_prefix_len,
                        const int32_t* h_num_tree, int32_t num_cus, uint32_t flags,
                        va_plan* plan, size_t* workspace_bytes) {
  if (h_prefix_len == nullptr || h_num_tree == nullptr || plan == nullptr) return VA_ERR_NULL;
  if ((flags & ~(VA_PLAN_SPLIT_TREE | VA_PLAN_ROWS64 | VA_PLAN_ROWS128)) != 0u) return VA_ERR_SHAPE;
  const bool split_tree = (flags & VA_PLAN_SPLIT_TREE) != 0u;
  const bool rows64 = (flags & VA_PLAN_ROWS64) != 0u;
  const bool rows128 = (flags & VA_PLAN_ROWS128) != 0u;
  if (rows64 && rows128) return VA_ERR_SHAPE;
  if (rows128 && split_tree) return VA_ERR_SHAPE;
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
  p.mode = split_tree ? VA_MODE_SPLIT_TREE : VA_MODE_FUSED;
  // 128-row blocks (va_wide_kernel) when every request has at least two row
  // groups and a block would get at least WIDE_MIN_KEYS prefix keys: the
  // row pairs' prefix keys over the CUs, before any split-count override
  bool wide = rows128;
  if (!rows64 && !rows128 && !split_tree) {
    bool pairs_only = true;
    int64_t pair_keys = 0;
    for (int r = 0; r < num_requests; ++r) {
      const int64_t groups = ((int64_t)h_num_tree[r] * num_heads + ROWS - 1) / ROWS;
      pairs_only &= groups >= 2;
      pair_keys += (groups + 1) / 2 * (int64_t)h_prefix_len[r];
    }
    wide = pairs_only && pair_keys >= (int64_t)WIDE_MIN_KEYS * num_cus;
  }
  const int gpb = wide ? 2 : 1;
  p.groups_per_block = gpb;

  // Split count: balance prefix keys x blocks per split (row groups, or row
  // pairs with 128-row blocks) over the compute units.
  // The draft keys (at most one tile) go with each request's last split in
  // the fused mode, and to the tree block, one more split per request run by
  // its own small kernel, in the split-tree mode.
  int64_t units = 0;
  int64_t cus = num_cus;
  for (int r = 0; r < num_requests; ++r) {
    const int64_t groups = ((int64_t)h_num_tree[r] * num_heads + ROWS - 1) / ROWS;
    units += (groups + gpb - 1) / gpb * (int64_t)h_prefix_len[r];
    if (split_tree) cus -= groups;   // compute units the tree-block work items occupy
  }
  if (cus < 1) cus = 1;
  // A work item takes ceil(keys / TILE) tile iterations whatever the keys in
  // its last tile, so the split length is rounded up to whole tiles: the
  // same iterations on the critical path, fewer splits to write and merge.
  // (The 65k-prefix request, H = 8, T = 16: 128 splits of 512 prefix keys,
  // 8 tiles each, the last split 16 draft keys more.  Spreading all L + T
  // keys instead gave 114 splits of 576 keys, 9 tiles each.)
  auto whole_tiles = [](int64_t k) { return (k + TILE - 1) / TILE * TILE; };
  int64_t keys_per_item = whole_tiles((units + cus - 1) / cus);
  if (keys_per_item < MIN_KEYS_PER_SPLIT) keys_per_item = MIN_KEYS_PER_SPLIT;
  int forced = 0;
  if (const char* e = std::getenv("VA_NSPLIT")) forced = std::atoi(e);
  // prefix split count of request r for a given split length
  auto nsplit_of = [&](int r, int64_t kpi) -> int64_t {
    const int64_t n = h_prefix_len[r];
    int64_t ns = forced > 0 ? forced : (n + kpi - 1) / kpi;
    const int64_t max_ns = (n + SPLIT_ALIGN - 1) / SPLIT_ALIGN;
    const int64_t cap = split_tree ? VA_MAX_SPLITS - 1 : VA_MAX_SPLITS;
    if (ns > max_ns) ns = max_ns;
    if (ns > cap) ns = cap;
    return ns < 1 ? 1 : ns;
  };
  // Each request's split count is rounded up, so the work items can add up to
  // more than the CUs, and the blocks past them would run as a second round
  // on the machine, doubling the call.  Lengthen the splits until the items
  // fit (or every request is down to one split per row group).
  if (forced == 0) {
    for (;;) {
      int64_t items = 0;
      bool more = false;
      for (int r = 0; r < num_requests; ++r) {
        const int64_t groups = ((int64_t)h_num_tree[r] * num_heads + ROWS - 1) / ROWS;
        const int64_t ns = nsplit_of(r, keys_per_item);
        items += (groups + gpb - 1) / gpb * ns;   // blocks
        more |= ns > 1;
      }
      if (items <= cus || !more) break;
      keys_per_item = whole_tiles(keys_per_item + std::max<int64_t>(SPLIT_ALIGN, keys_per_item / 64));
    }
  }

  int64_t work = 0;
  int64_t tree = 0;
  p.tree_begin[0] = 0;
  p.work_begin[0] = 0;
  for (int r = 0; r < num_requests; ++r) {
    const int64_t groups = ((int64_t)h_num_tree[r] * num_heads + ROWS - 1) / ROWS;
    int64_t ns = nsplit_of(r, keys_per_item);
    if (split_tree) ns += 1;   // the tree block
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
  const int64_t o_bytes = align256(work * ROWS * DV * (int64_t)sizeof(uint16_t));
  const int64_t lse_bytes = align256(work * ROWS * 2 * (int64_t)sizeof(float));
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
  const int rc = check_run_args(plan, q, kv_pool, num_slots, kv_row_stride, slot_table,
                                slot_table_len, slot_indptr, prefix_len, parent, sm_scale);
  if (rc != VA_OK) return rc;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
      (int64_t)workspace_bytes < plan->workspace_bytes)
    return VA_ERR_WORKSPACE;
  return launch_partial(plan, q, kv_pool, num_slots, kv_row_stride, slot_table, slot_table_len,
                        slot_indptr, prefix_len, parent, sm_scale, static_cast<char*>(workspace),
                        static_cast<hipStream_t>(stream));
}

int verify_attn_reduce(const va_plan* plan, const void* workspace, uint16_t* out, float* lse,
                       va_stream_t stream) {
  if (plan == nullptr || workspace == nullptr || out == nullptr || lse == nullptr)
    return VA_ERR_NULL;
  if (!plan_ok(plan)) return VA_ERR_PLAN;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return VA_ERR_ALIGN;
  return launch_reduce(plan, static_cast<const char*>(workspace), out, lse,
                       static_cast<hipStream_t>(stream));
}

int verify_attn_forward_static(const va_plan* plan, const uint16_t* q, const uint16_t* kv_pool,
                               int64_t num_slots, int32_t kv_row_stride,
                               const int32_t* slot_table, int32_t slot_table_len,
                               const int32_t* slot_indptr, const int32_t* prefix_len,
                               const int32_t* parent, float sm_scale, uint16_t* out, float* lse,
                               va_stream_t stream) {
  int rc = check_run_args(plan, q, kv_pool, num_slots, kv_row_stride, slot_table,
                          slot_table_len, slot_indptr, prefix_len, parent, sm_scale);
  if (rc != VA_OK) return rc;
  if (out == nullptr || lse == nullptr) return VA_ERR_NULL;
  if (!aligned16(out)) return VA_ERR_ALIGN;
  if (plan->workspace_bytes > (int64_t)VA_STATIC_SCRATCH_BYTES) return VA_ERR_WORKSPACE;
  char* ws = nullptr;
  rc = static_scratch(&ws);
  if (rc != VA_OK) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  rc = launch_partial(plan, q, kv_pool, num_slots, kv_row_stride, slot_table, slot_table_len,
                      slot_indptr, prefix_len, parent, sm_scale, ws, st);
  if (rc != VA_OK) return rc;
  return launch_reduce(plan, ws, out, lse, st);
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
  hipLaunchKernelGGL(va_gather_kernel, dim3((unsigned)((n + TILE - 1) / TILE)), dim3(THREADS), 0,
                     static_cast<hipStream_t>(stream), kv_pool, num_slots, kv_row_stride,
                     slot_table, n, dst);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}

int verify_attn_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t sink_words,
                            va_stream_t stream) {
  if (buf == nullptr || sink == nullptr) return VA_ERR_NULL;
  if (bytes < 0 || (bytes & 15) != 0 || sink_words < 1) return VA_ERR_SHAPE;
  if (!aligned16(buf)) return VA_ERR_ALIGN;
  if (bytes == 0) return VA_OK;
  int32_t cus = 0;
  const int rc = query_num_cus(&cus);
  if (rc != VA_OK) return rc;
  const int64_t n16 = bytes / 16;
  const int64_t want = (n16 + STREAM_THREADS - 1) / STREAM_THREADS;
  const unsigned blocks = (unsigned)std::min<int64_t>(want, (int64_t)cus * STREAM_BLOCKS_PER_CU);
  hipLaunchKernelGGL(va_stream_read_kernel, dim3(blocks), dim3(STREAM_THREADS), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), n16, sink,
                     sink_words);
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
