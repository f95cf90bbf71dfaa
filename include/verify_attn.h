/*
 * verify_attn.h - C ABI of the MI355X (gfx950) tree-verify MLA attention library.
 *
 * The operation: for every draft-tree node i of a request and every head h,
 * weight-absorbed MLA attention of the 576-wide query q[i,h] (512 latent +
 * 64 rope columns) over the request's latent KV rows, which live one token
 * per slot (page_size 1) in a shared pool and are reached through a
 * per-token slot table.  Node i sees the whole prefix (no mask), itself and
 * its ancestors in the draft tree; it never sees siblings or descendants.
 *   score_k = sm_scale * <q[i,h], K_k>        (K_k = all 576 columns of row k)
 *   lse     = ln sum_k exp(score_k)           (over the visible keys)
 *   out     = sum_k exp(score_k - lse) * V_k  (V_k = first 512 columns of row k)
 *
 * Sources: "The Execution Phase: From Plan to 3-6x Decode Speedup on
 * Blackwell Consumer GPUs" (section "The Transition: From Planning to
 * Execution": a C API called through ctypes, around MLA-absorb attention
 * with a custom tree mask; section "Making the Kernel CUDA Graph
 * Capture-Safe": static buffers, no host sync, no device allocation, a
 * caller-owned workspace, a split count fixed ahead of capture); "The
 * Verify Kernel Breakthrough" (section "The Message in Context": split-KV
 * flash-decode with a partial pass and a reduce); "The Architecture
 * Detective" (section "The Split Verify Design": dense prefix, masked tree
 * block, log-sum-exp merge).
 *
 * Three calls make one verify step:
 *   verify_attn_plan   host only; sizes the split-KV work and the workspace.
 *   verify_attn_run    partial pass: every (request, row group, KV split)
 *                      work item writes a partial (o, lse) into the workspace.
 *   verify_attn_reduce log-sum-exp merge of the partials into out and lse.
 *
 * Conventions for every entry point:
 *   - Pointers named h_* are host pointers; every other data pointer is a
 *     device pointer.  bf16 tensors are passed as uint16_t bit patterns.
 *   - The caller owns all memory.  The library never allocates or frees
 *     device memory and never synchronises; run and reduce only enqueue
 *     kernels on `stream` (a hipStream_t; NULL = the default stream), so the
 *     pair can be captured into a HIP graph.  Call plan outside capture.
 *   - Return value: VA_OK (0) or a negative VA_ERR_* code.  No exception
 *     crosses the ABI.  Argument errors are found on the host before any
 *     launch; faulty device-resident data (a slot outside the pool, a bad
 *     parent, a prefix length above the planned bound, a short slot table)
 *     is never dereferenced: the affected rows come out as NaN and the
 *     workspace records the error (verify_attn_read_status).
 *   - One workspace serves one run/reduce pair at a time; concurrent steps
 *     need separate workspaces.
 */
#ifndef VERIFY_ATTN_H
#define VERIFY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VA_D_QK 576         /* query / key width: 512 latent + 64 rope */
#define VA_D_V 512          /* value width: the latent columns */
#define VA_MAX_TREE 64      /* draft nodes per request (one 64-bit ancestor mask) */
#define VA_MAX_REQUESTS 64  /* requests per plan */
#define VA_MAX_SPLITS 256   /* KV splits per request */
#define VA_MAX_HEADS 1024

/* Return codes. */
#define VA_OK 0
#define VA_ERR_NULL (-1)        /* a required pointer is NULL */
#define VA_ERR_SHAPE (-2)       /* count out of range (B, H, T, L, stride, num_slots) */
#define VA_ERR_ALIGN (-3)       /* q/kv/out not 16-byte aligned, or stride not a multiple of 8 */
#define VA_ERR_WORKSPACE (-4)   /* workspace NULL, misaligned or smaller than planned */
#define VA_ERR_PLAN (-5)        /* plan not produced by verify_attn_plan of this version */
#define VA_ERR_HIP (-6)         /* a HIP call or kernel launch failed */
#define VA_ERR_TREE (-7)        /* parent[] is not a topological forest */
#define VA_ERR_DEVICE_DATA (-8) /* device data failed the in-kernel checks (status word) */

/* Bits of the device status word (verify_attn_read_status). */
#define VA_STATUS_BAD_PREFIX 1u  /* prefix_len[r] < 0 or above the planned bound */
#define VA_STATUS_SHORT_TABLE 2u /* slot_indptr gives fewer than L + T entries or leaves the table */
#define VA_STATUS_BAD_SLOT 4u    /* a slot outside [0, num_slots) */
#define VA_STATUS_BAD_PARENT 8u  /* parent[i] outside [-1, i-1] */

typedef void* va_stream_t; /* a hipStream_t */

/*
 * Launch plan: a plain struct the caller allocates (stack, static or heap);
 * it owns no resources and is never freed.  Its content is filled by
 * verify_attn_plan and is read-only for the caller.
 */
typedef struct va_plan {
  uint32_t magic;            /* VA_PLAN_MAGIC when valid */
  uint32_t version;          /* VA_PLAN_VERSION */
  int32_t num_requests;      /* B */
  int32_t num_heads;         /* H */
  int32_t rows_per_group;    /* query rows (node, head) one work item holds */
  int32_t tile_keys;         /* keys per KV tile; split lengths are multiples of half of it */
  int32_t total_work;        /* work items of the partial pass (its grid) */
  int32_t total_tree;        /* sum of T_r */
  int32_t total_rows;        /* sum of T_r * H */
  int32_t num_cus;           /* compute units the plan was sized for */
  int32_t mode;              /* VA_MODE_FUSED or VA_MODE_SPLIT_TREE */
  int32_t groups_per_block;  /* row groups one partial-pass block holds: 1, or 2 (128-row blocks) */
  int64_t workspace_bytes;   /* bytes verify_attn_run needs */
  int64_t lse_offset;        /* byte offset of the partial-lse region */
  int64_t status_offset;     /* byte offset of the per-work-item status words */
  int32_t num_tree[VA_MAX_REQUESTS];        /* T_r */
  int32_t max_prefix[VA_MAX_REQUESTS];      /* planned upper bound of L_r */
  int32_t nsplit[VA_MAX_REQUESTS];          /* KV splits of request r */
  int32_t num_groups[VA_MAX_REQUESTS];      /* row groups of request r */
  int32_t tree_begin[VA_MAX_REQUESTS + 1];  /* prefix sums of T_r */
  int32_t work_begin[VA_MAX_REQUESTS + 1];  /* prefix sums of groups * splits */
} va_plan;

#define VA_PLAN_MAGIC 0x56415054u /* "VAPT" */
#define VA_PLAN_VERSION 3u

/* How verify_attn_run decomposes the keys of a request (va_plan.mode).
 * VA_MODE_FUSED: one partial kernel; its nsplit splits cover equal slices
 *   of the L prefix keys (whole 32-key blocks), the last one followed by the
 *   T draft keys, and the tiles that reach into the draft block apply the
 *   tree mask.
 * VA_MODE_SPLIT_TREE: the split-verify decomposition ("The Architecture
 *   Detective", section "The Split Verify Design": the draft queries attend
 *   the prefix densely, only the small tree block needs the custom mask, and
 *   a log-sum-exp merge joins the two).  A prefix kernel without any tree
 *   mask covers the L prefix keys in nsplit-1 splits, and a tree-block
 *   kernel covers the T draft keys as split nsplit-1.  The same reduce merges
 *   both.  Results agree with the fused mode to rounding. */
#define VA_MODE_FUSED 0
#define VA_MODE_SPLIT_TREE 1

/* verify_attn_plan_ex flags */
#define VA_PLAN_SPLIT_TREE 1u   /* plan VA_MODE_SPLIT_TREE instead of VA_MODE_FUSED */
#define VA_PLAN_ROWS64 2u       /* 64-row blocks (groups_per_block = 1) whatever the row count */
#define VA_PLAN_ROWS128 4u      /* 128-row blocks (groups_per_block = 2); fused mode only */

/*
 * verify_attn_plan - size the split-KV schedule and the workspace (host only).
 *
 * num_requests   B, 1..VA_MAX_REQUESTS.
 * num_heads      H, 1..VA_MAX_HEADS.
 * h_prefix_len   [B] host: prefix length L_r of each request, >= 0.  For a
 *                captured graph pass an upper bound; the device value given
 *                to run may be anything from 0 up to it.
 * h_num_tree     [B] host: draft nodes T_r, 1..VA_MAX_TREE.  Fixed by the plan.
 * num_cus        compute units to size the schedule for; 0 = ask the current
 *                HIP device (the only device call this function makes).
 * plan           out: caller-allocated plan.
 * workspace_bytes out (may be NULL): bytes of device workspace run needs
 *                (also plan->workspace_bytes).
 *
 * The number of KV splits per request (the grid dimension of the partial
 * pass; "The Verify Kernel Breakthrough", section "The Message in Context",
 * raised it from 16 to 64 for occupancy) is chosen from the compute-unit
 * count, the rows T_r*H and the prefix lengths so that every work item gets
 * a similar number of prefix keys in whole tiles (the T_r <= 64 draft keys
 * add at most one tile to the request's last split) and the work items fit
 * the compute units.  The environment variable VA_NSPLIT, read here
 * only, forces one split count for every request (for tuning sweeps; with
 * VA_PLAN_SPLIT_TREE it is the count of prefix splits).
 * In the fused mode, when every request has at least two row groups and
 * sum_r ceil(groups_r / 2) * L_r >= 2048 * num_cus (each block's share of
 * the prefix is at least 2048 keys), the plan uses 128-row blocks
 * (groups_per_block = 2): one block runs the two row groups 2j and 2j+1 of
 * a split, so each KV row enters a compute unit once per 128 rows, and the
 * splits are balanced over ceil(groups / 2) blocks per split (about twice
 * the splits of 64-row blocks).  The work items, the workspace and the
 * merge stay those of 64-row groups.  VA_NSPLIT does not enter this choice.
 * Errors: VA_ERR_NULL, VA_ERR_SHAPE, VA_ERR_HIP (device query failed).
 */
int verify_attn_plan(int32_t num_requests, int32_t num_heads, const int32_t* h_prefix_len,
                     const int32_t* h_num_tree, int32_t num_cus, va_plan* plan,
                     size_t* workspace_bytes);

/*
 * verify_attn_plan_ex - verify_attn_plan with flags.  flags = 0 is
 * verify_attn_plan (VA_MODE_FUSED); VA_PLAN_SPLIT_TREE plans the
 * split-verify decomposition (VA_MODE_SPLIT_TREE): nsplit[r] counts the
 * prefix splits plus the one tree-block split.  VA_PLAN_ROWS64 and
 * VA_PLAN_ROWS128 override the block-size rule of verify_attn_plan; both
 * together, or VA_PLAN_ROWS128 with VA_PLAN_SPLIT_TREE, are VA_ERR_SHAPE, as
 * are unknown flag bits.  Other arguments and errors as verify_attn_plan.
 */
int verify_attn_plan_ex(int32_t num_requests, int32_t num_heads, const int32_t* h_prefix_len,
                        const int32_t* h_num_tree, int32_t num_cus, uint32_t flags,
                        va_plan* plan, size_t* workspace_bytes);

/*
 * verify_attn_run - partial pass (enqueue only).
 *
 * plan           from verify_attn_plan (host pointer; read during the call only).
 * q              [sum T_r, H, 576] bf16, rows ordered (request, node, head);
 *                16-byte aligned.
 * kv_pool        [num_slots, kv_row_stride] bf16; columns 0..511 latent,
 *                512..575 rope; 16-byte aligned.
 * num_slots      rows in the pool (>= 1); slots are checked against it.
 * kv_row_stride  elements between pool rows, >= 576 and a multiple of 8.
 * slot_table     int32 [slot_table_len], per request L_r prefix slots in
 *                logical order then T_r draft slots in node order, requests
 *                concatenated.
 * slot_table_len entries in slot_table; every table read is checked against it.
 * slot_indptr    [B+1] int32: request r uses slot_table[slot_indptr[r] ...
 *                slot_indptr[r+1]), which must hold at least L_r + T_r entries.
 * prefix_len     [B] int32 device: actual L_r, 0..planned bound.
 * parent         [sum T_r] int32, request-local: parent[i] in [-1, i-1]
 *                (-1: the node hangs directly off the prefix).
 * sm_scale       softmax scale applied to <q, k> (the workloads use 1/sqrt(192));
 *                it must be finite and > 0 (the kernel takes the row max of the
 *                unscaled scores and masks with -inf before scaling), anything
 *                else is refused with VA_ERR_SHAPE.
 * workspace      device scratch of at least plan->workspace_bytes, 256-byte
 *                aligned; needs no initialisation.
 * stream         hipStream_t to enqueue on.
 * Errors: VA_ERR_NULL, VA_ERR_PLAN, VA_ERR_SHAPE, VA_ERR_ALIGN,
 *         VA_ERR_WORKSPACE, VA_ERR_HIP.
 */
int verify_attn_run(const va_plan* plan, const uint16_t* q, const uint16_t* kv_pool,
                    int64_t num_slots, int32_t kv_row_stride, const int32_t* slot_table,
                    int32_t slot_table_len, const int32_t* slot_indptr, const int32_t* prefix_len,
                    const int32_t* parent, float sm_scale, void* workspace,
                    size_t workspace_bytes, va_stream_t stream);

/*
 * verify_attn_reduce - merge the partials by log-sum-exp (enqueue only).
 *
 * workspace      the workspace the preceding verify_attn_run wrote.
 * out            [sum T_r, H, 512] bf16 (round to nearest even); 16-byte aligned.
 * lse            [sum T_r, H] fp32: natural log of the partition sum of the
 *                scaled scores over the row's visible keys.
 * Rows whose request failed the device checks get NaN in out and lse.
 * Errors: VA_ERR_NULL, VA_ERR_PLAN, VA_ERR_ALIGN, VA_ERR_HIP.
 */
int verify_attn_reduce(const va_plan* plan, const void* workspace, uint16_t* out, float* lse,
                       va_stream_t stream);

/*
 * verify_attn_forward_static - verify_attn_run followed by verify_attn_reduce
 * (the same kernels, enqueued back to back on `stream`) with the partials in
 * a scratch array the library holds on each device for the life of the
 * process, so the call allocates nothing and takes no workspace.  For callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments as verify_attn_run and verify_attn_reduce; out and lse as
 * verify_attn_reduce.  The scratch holds VA_STATIC_SCRATCH_BYTES, enough for
 * VA_STATIC_SCRATCH_WORK work items (any plan with plan->total_work <= 512,
 * e.g. every single-request plan for up to 256 compute units with
 * T*H <= 16,384 rows); a plan whose workspace_bytes exceeds it is refused
 * with VA_ERR_WORKSPACE.
 * The first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress, with the device current); no call allocates.
 * Every call on one device shares its array: calls whose kernels may
 * overlap on one device (different streams without ordering) race and must
 * be serialised by the caller.  The kernels write every scratch word they
 * read in the same call, so nothing needs clearing between calls.  The
 * status words stay in the scratch: rows of a request that failed the
 * device checks come out as NaN in out and lse, as with verify_attn_reduce.
 * Errors: VA_ERR_NULL, VA_ERR_PLAN, VA_ERR_SHAPE, VA_ERR_ALIGN,
 *         VA_ERR_WORKSPACE (plan too large for the scratch), VA_ERR_HIP.
 */
#define VA_STATIC_SCRATCH_WORK 512
/* 512 work items x (65,536 B partials + 512 B lse pairs) + 2,048 B status words */
#define VA_STATIC_SCRATCH_BYTES 33818624
int verify_attn_forward_static(const va_plan* plan, const uint16_t* q, const uint16_t* kv_pool,
                               int64_t num_slots, int32_t kv_row_stride,
                               const int32_t* slot_table, int32_t slot_table_len,
                               const int32_t* slot_indptr, const int32_t* prefix_len,
                               const int32_t* parent, float sm_scale, uint16_t* out, float* lse,
                               va_stream_t stream);

/*
 * verify_attn_read_status - OR of the device status words the last run wrote
 * (VA_STATUS_* bits) into *h_status.  Diagnostic: it copies to the host and
 * synchronises `stream`, so it must not be called under graph capture.
 * Errors: VA_ERR_NULL, VA_ERR_PLAN, VA_ERR_HIP.
 */
int verify_attn_read_status(const va_plan* plan, const void* workspace, va_stream_t stream,
                            uint32_t* h_status);

/*
 * verify_attn_check_tree - host validator for one request's parent array:
 * VA_OK when every parent[i] is in [-1, i-1] and 1 <= T <= VA_MAX_TREE,
 * else VA_ERR_TREE (VA_ERR_NULL for a NULL pointer).
 */
int verify_attn_check_tree(const int32_t* h_parent, int32_t T);

/*
 * verify_attn_gather_rows - diagnostic copy of pool rows through the partial
 * pass's own tile loader (its slot-table ring, 16-byte copy sources and copy
 * instructions into its LDS tile layout, 64 keys per tile), read back out of
 * LDS: dst[k, 0:576] = kv_pool[slot_table[k], 0:576] for k < n.  dst is [n, 576] bf16, 16-byte
 * aligned.  Slots outside [0, num_slots) yield rows of NaN.  Enqueue only.
 * Errors: VA_ERR_NULL, VA_ERR_SHAPE, VA_ERR_ALIGN, VA_ERR_HIP.
 */
int verify_attn_gather_rows(const uint16_t* kv_pool, int64_t num_slots, int32_t kv_row_stride,
                            const int32_t* slot_table, int32_t n, uint16_t* dst,
                            va_stream_t stream);

/*
 * verify_attn_stream_read - measurement helper: reads every 16-byte word of
 * buf once with streaming loads (the device's plain read ceiling, against
 * which the partial pass's effective bandwidth is compared).  Each of its
 * blocks XORs the XOR of the 32-bit words it read into one of the
 * sink_words words of sink, so the XOR of all sink words (which the caller
 * initialises) equals the XOR of buf's words.  Up to 8 blocks per compute
 * unit; with sink_words at least that many no two blocks share a word.
 * buf: `bytes` of device memory, 16-byte aligned, bytes a multiple of 16.
 * sink: sink_words >= 1 device uint32.  Enqueue only; allocates nothing.
 * Errors: VA_ERR_NULL, VA_ERR_SHAPE, VA_ERR_ALIGN, VA_ERR_HIP.
 */
int verify_attn_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t sink_words,
                            va_stream_t stream);

/* Static text for a return code. */
const char* verify_attn_error_string(int code);

/* sizeof(va_plan) as compiled into the library, for bindings to check
 * their mirror of the struct. */
size_t verify_attn_plan_struct_size(void);

/*
 * ---- Tier 1 KV defragmentation: compaction of one request's slots ----
 *
 * "The Execution Phase" (section "Tier 0 KV Defragmentation") names live
 * relocation of a request's fragmented KV slots under a copy budget as the
 * next tier; "The Architecture Detective" (section "Deconstructing the K/V
 * Defrag Hypothesis") describes moving a request's KV entries to contiguous
 * slots.  Policy (the plainest reading): logical position k of the table
 * belongs at slot dst_begin + k of a free run [dst_begin, dst_begin + n)
 * the caller reserved.  Walking k upward, each row not yet at its place is
 * copied there (its 576 columns) and table[k] rewritten,
 * until `budget` rows have been copied; rows already in place are skipped
 * and do not count.
 *
 * kv_pool        [num_slots, kv_row_stride] bf16, device, 16-byte aligned;
 *                the copied rows' first 576 columns are written.
 * slot_table     [n] int32, device: one request's table (prefix then draft
 *                entries, or any other run of logical positions); rewritten.
 *                May be NULL when n = 0 (then copied is set to 0).
 * dst_begin      first slot of the reserved run; dst_begin + n <= num_slots.
 * budget         most rows to copy (>= 0).
 * workspace      device, 256-byte aligned, at least
 *                verify_attn_compact_workspace_bytes(n, budget) bytes.
 * copied         device int32 out: rows copied, or minus the OR of the
 *                VA_COMPACT_* bits when a precondition failed (then nothing
 *                is copied and the table is unchanged).
 * Preconditions checked on the device: every slot inside the pool, and no
 * slot inside the destination run except at its own place (such a row could
 * be overwritten before it is read).  Stream-ordered, asynchronous,
 * graph-capture safe (grids depend on n and budget only).
 * Errors (host): VA_ERR_NULL, VA_ERR_SHAPE (negative sizes, run outside the
 * pool, stride < 576), VA_ERR_ALIGN, VA_ERR_WORKSPACE, VA_ERR_HIP.
 */
#define VA_COMPACT_BAD_SLOT 1u       /* a slot outside [0, num_slots) */
#define VA_COMPACT_RUN_OCCUPIED 2u   /* a slot inside the run but not at its own place */
size_t verify_attn_compact_workspace_bytes(int32_t n, int32_t budget);
int verify_attn_compact(uint16_t* kv_pool, int64_t num_slots, int32_t kv_row_stride,
                        int32_t* slot_table, int32_t n, int32_t dst_begin, int32_t budget,
                        void* workspace, size_t workspace_bytes, int32_t* copied,
                        va_stream_t stream);

/*
 * ---- Draft-tree marshaling on the device ----
 *
 * The pages build the draft tree and its mask on the host ("The Execution
 * Phase", section "The Methodology: Evidence-Driven Engineering": 1.8 ms of
 * tree build and 0.18 ms of mask build per step); this call does it on the
 * device so a whole verify step can live in one HIP graph.
 *
 * For request r of `plan` (its T_r = num_tree[r] and tree_begin layout):
 * raw_parent     [sum T_r] device: request-local parent of raw node j, in
 *                [-1, T_r) (-1: hangs off the prefix), nodes in any order.
 * raw_slot       [sum T_r] device: pool slot holding raw node j's KV row.
 * prefix_len, slot_indptr   as for verify_attn_run (device).
 * slot_table     device, slot_table_len entries: receives, for verify
 *                position i, slot_table[slot_indptr[r] + prefix_len[r] + i]
 *                = raw_slot[perm[i]] (only inside [slot_indptr[r],
 *                slot_indptr[r+1])).
 * perm, parent   [sum T_r] int32 out: verify order = raw nodes sorted by
 *                (depth, raw index), i.e. breadth first, so parent[i] < i;
 *                perm[i] is the raw node at position i, parent[i] its
 *                parent's position or -1 - ready for verify_attn_run.
 * anc            [sum T_r] uint64 out: bit k set iff position k is i or an
 *                ancestor of i (the tree mask; verify_attn_run builds the
 *                same masks itself from `parent`, so it needs no anc input).
 * status         [B] uint32 out: 0, or VA_TREE_* bits for a request whose
 *                raw tree is not a forest or whose draft entries do not all
 *                fall inside its table range (a short range or a negative
 *                device prefix length; entries outside the range are not
 *                written, and its outputs are unspecified; other requests
 *                are not affected).
 * One 64-lane wave per request; stream-ordered, graph-capture safe.
 * Errors (host): VA_ERR_NULL, VA_ERR_PLAN, VA_ERR_SHAPE, VA_ERR_HIP.
 */
#define VA_TREE_BAD_PARENT 1u   /* a parent outside [-1, T_r) or a cycle */
#define VA_TREE_BAD_TABLE 2u    /* a draft entry falls outside the request's table range */
int verify_attn_build_tree(const va_plan* plan, const int32_t* raw_parent, const int32_t* raw_slot,
                           const int32_t* prefix_len, const int32_t* slot_indptr,
                           int32_t* slot_table, int32_t slot_table_len, int32_t* perm,
                           int32_t* parent, uint64_t* anc, uint32_t* status, va_stream_t stream);

/*
 * verify_attn_permute_rows - gather per-node rows from raw node order into
 * verify order (enqueue only): the step between verify_attn_build_tree and
 * verify_attn_run for queries produced in raw node order, so that raw trees
 * in, verify outputs out is a sequence of library calls on one stream.
 *
 * perm       [sum T_r] device: from verify_attn_build_tree (request-local raw
 *            node of each verify position).
 * src        [sum T_r, row_elems] bf16 device: one row per raw node, requests
 *            concatenated as in `plan` (for q: row_elems = H * 576).
 * dst        [sum T_r, row_elems] bf16 device out:
 *            dst[t0 + i] = src[t0 + perm[t0 + i]] for request r starting at
 *            t0 = tree_begin[r].  A perm entry outside [0, T_r) (a request
 *            verify_attn_build_tree flagged) gives a row of zeros.
 * row_elems  elements per row, >= 8 and a multiple of 8 (16-byte pieces).
 * src and dst are 16-byte aligned and must not overlap.
 * Errors (host): VA_ERR_NULL, VA_ERR_PLAN, VA_ERR_SHAPE, VA_ERR_ALIGN, VA_ERR_HIP.
 */
int verify_attn_permute_rows(const va_plan* plan, const int32_t* perm, const uint16_t* src,
                             uint16_t* dst, int64_t row_elems, va_stream_t stream);

/*
 * verify_attn_build_tree_rows - verify_attn_build_tree and
 * verify_attn_permute_rows in one launch (enqueue only), for the same
 * reason: the draft tree and the verify-order rows of one step without a
 * second dependent launch ("The Execution Phase", section "The Methodology:
 * Evidence-Driven Engineering" measures the tree and mask build as host work
 * of every step).
 *
 * Arguments as for verify_attn_build_tree, then src, dst and row_elems as
 * for verify_attn_permute_rows; every output is as those two calls write it
 * for a request whose status is 0.  For a flagged request its outputs are
 * unspecified (dst rows are some source row of the request, or zeros),
 * nothing is written outside its own ranges, and other requests are not
 * affected.  The row gather ranks the request's nodes again in each gather
 * block (the same ranking) rather than reading perm.
 * Errors (host): VA_ERR_NULL, VA_ERR_PLAN, VA_ERR_SHAPE, VA_ERR_ALIGN, VA_ERR_HIP.
 */
int verify_attn_build_tree_rows(const va_plan* plan, const int32_t* raw_parent,
                                const int32_t* raw_slot, const int32_t* prefix_len,
                                const int32_t* slot_indptr, int32_t* slot_table,
                                int32_t slot_table_len, int32_t* perm, int32_t* parent,
                                uint64_t* anc, uint32_t* status, const uint16_t* src,
                                uint16_t* dst, int64_t row_elems, va_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_ATTN_H */
