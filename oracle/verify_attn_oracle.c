/*
 * Plain CPU fp64 oracle for tree-masked, weight-absorbed MLA verify attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * What it computes (the plain definition, no splitting, no online softmax):
 *
 *   "The Execution Phase: From Plan to 3-6x Decode Speedup on Blackwell
 *   Consumer GPUs", section "The Transition: From Planning to Execution"
 *   names the operation as MLA-absorb attention with a custom tree mask.
 *   "The Architecture Detective", section "The Split Verify Design", says the
 *   draft queries attend the whole prefix densely (no mask) and only the
 *   tree block among the draft tokens carries the custom mask.
 *
 * Readings taken where the pages are silent (each one is listed in the
 * design notes of the repository):
 *   - K is the whole 576-wide latent row (512 latent followed by 64 rope
 *     columns); V is its first 512 columns (the absorbed form: one latent
 *     row is shared by every head).
 *   - The score is sm_scale * <q, k> with nothing else multiplied in.
 *   - Node i of a request sees every prefix position 0..L-1, itself and
 *     its ancestors (follow parent[] until -1); never siblings or
 *     descendants.  parent[i] lies in [-1, i-1].
 *   - lse is the natural log of the sum of exp(score) over visible keys.
 *   - Per request the slot table holds L prefix slots in logical order and
 *     then T draft slots in node order.
 *
 * Everything is fp64; bf16 inputs are decoded exactly (bits << 16).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_D_QK 576
#define ORACLE_D_V 512

enum {
  ORACLE_OK = 0,
  ORACLE_ERR_ARG = -1,
  ORACLE_ERR_TREE = -2,
  ORACLE_ERR_SLOT = -3,
  ORACLE_ERR_TABLE = -4,
  ORACLE_ERR_NOMEM = -5
};

int oracle_d_qk(void) { return ORACLE_D_QK; }
int oracle_d_v(void) { return ORACLE_D_V; }

/* Exact bf16 -> double: a bf16 value is the top half of an IEEE float. */
static double bf16_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * Tree visibility.  vis[i*T + j] = 1 when draft node j is node i itself or
 * one of its ancestors (the custom tree mask of "The Split Verify Design"),
 * else 0.  Found by following parent[] from i up to -1.
 * Returns ORACLE_ERR_TREE when some parent[i] is outside [-1, i-1].
 */
int oracle_tree_visibility(const int32_t* parent, int32_t T, uint8_t* vis) {
  if (T < 0 || (T > 0 && (parent == NULL || vis == NULL))) return ORACLE_ERR_ARG;
  for (int32_t i = 0; i < T; ++i)
    if (parent[i] < -1 || parent[i] >= i) return ORACLE_ERR_TREE;
  for (int32_t i = 0; i < T; ++i) {
    for (int32_t j = 0; j < T; ++j) vis[(int64_t)i * T + j] = 0;
    for (int32_t a = i; a != -1; a = parent[a]) vis[(int64_t)i * T + a] = 1;
  }
  return ORACLE_OK;
}

/*
 * Softmax attention of one query over an explicit list of pool slots, no
 * mask: s_k = sm_scale * <q, K[slot_k]> over all 576 columns,
 * lse = log(sum_k exp(s_k)), p_k = exp(s_k - lse),
 * o[c] = sum_k p_k * K[slot_k][c] for c < 512.
 * With n == 0 the result is o = 0, lse = -inf.
 * probs (optional, length n) receives p_k.
 */
int oracle_attend(const double* q, const uint16_t* kv_pool, int64_t num_slots,
                  int32_t kv_row_stride, const int32_t* slots, int64_t n,
                  double sm_scale, double* o, double* lse, double* probs) {
  if (q == NULL || o == NULL || lse == NULL || (n > 0 && (kv_pool == NULL || slots == NULL)))
    return ORACLE_ERR_ARG;
  for (int64_t k = 0; k < n; ++k)
    if (slots[k] < 0 || (int64_t)slots[k] >= num_slots) return ORACLE_ERR_SLOT;
  for (int c = 0; c < ORACLE_D_V; ++c) o[c] = 0.0;
  if (n == 0) {
    *lse = -INFINITY;
    return ORACLE_OK;
  }
  double* s = (double*)malloc((size_t)n * sizeof(double));
  if (s == NULL) return ORACLE_ERR_NOMEM;
  double m = -INFINITY;
  for (int64_t k = 0; k < n; ++k) {
    const uint16_t* row = kv_pool + (int64_t)slots[k] * kv_row_stride;
    double dot = 0.0;
    for (int d = 0; d < ORACLE_D_QK; ++d) dot += q[d] * bf16_to_double(row[d]);
    s[k] = sm_scale * dot;
    if (s[k] > m) m = s[k];
  }
  double z = 0.0;
  for (int64_t k = 0; k < n; ++k) z += exp(s[k] - m);
  const double l = m + log(z);
  for (int64_t k = 0; k < n; ++k) {
    const double p = exp(s[k] - l);
    if (probs != NULL) probs[k] = p;
    const uint16_t* row = kv_pool + (int64_t)slots[k] * kv_row_stride;
    for (int c = 0; c < ORACLE_D_V; ++c) o[c] += p * bf16_to_double(row[c]);
  }
  *lse = l;
  free(s);
  return ORACLE_OK;
}

/*
 * Combine attention results computed over disjoint parts of one key set.
 * Each part j holds its own normalised output o_j (length d) and its
 * log-partition lse_j.  By the definition of softmax over the union:
 *   lse = log(sum_j exp(lse_j)),   o = sum_j exp(lse_j - lse) * o_j.
 * Parts with lse_j = -inf (empty parts) carry no weight.  This is the merge
 * of per-split results named in "The Verify Kernel Breakthrough" (section
 * "The Message in Context", partial+reduce) and "The Architecture
 * Detective" (section "The Split Verify Design", LSE merge).
 */
int oracle_lse_merge(int32_t num_parts, int32_t d, const double* o_parts,
                     const double* lse_parts, double* o, double* lse) {
  if (num_parts < 0 || d < 0 || o == NULL || lse == NULL) return ORACLE_ERR_ARG;
  double m = -INFINITY;
  for (int32_t j = 0; j < num_parts; ++j)
    if (lse_parts[j] > m) m = lse_parts[j];
  for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
  if (m == -INFINITY) {
    *lse = -INFINITY;
    return ORACLE_OK;
  }
  double z = 0.0;
  for (int32_t j = 0; j < num_parts; ++j)
    if (lse_parts[j] != -INFINITY) z += exp(lse_parts[j] - m);
  const double l = m + log(z);
  for (int32_t j = 0; j < num_parts; ++j) {
    if (lse_parts[j] == -INFINITY) continue;
    const double w = exp(lse_parts[j] - l);
    for (int32_t c = 0; c < d; ++c) o[c] += w * o_parts[(int64_t)j * d + c];
  }
  *lse = l;
  return ORACLE_OK;
}

/*
 * Tree-masked verify attention over a batch of requests.
 *
 * Request r has T_r = num_tree[r] draft nodes and L_r = prefix_len[r]
 * prefix tokens.  Its slot table is slot_table[slot_indptr[r] ...], holding
 * L_r + T_r entries (prefix then draft nodes).  Rows are (node, head);
 * q, out and lse are laid out [sum T_r, H, ...] with requests concatenated.
 * For every row the visible keys are the L_r prefix positions and the draft
 * positions L_r + j with j in anc*(i); the row is then plain softmax
 * attention over those keys (oracle_attend).
 *
 * row_select (optional, length sum T_r * H): compute only rows with a
 *   non-zero entry; other rows of out/lse are left untouched.
 * probs (optional): probs[row * probs_stride + k] = p of logical key k of
 *   the row's request (k < L_r + T_r), exactly 0 for keys the mask hides.
 * num_threads <= 0 uses the OpenMP default; 1 runs single-threaded.
 */
int oracle_verify_attn(int32_t num_requests, int32_t num_heads, const int32_t* num_tree,
                       const int32_t* prefix_len, const uint16_t* q, const uint16_t* kv_pool,
                       int64_t num_slots, int32_t kv_row_stride, const int32_t* slot_table,
                       const int32_t* slot_indptr, const int32_t* parent, double sm_scale,
                       double* out, double* lse, const uint8_t* row_select, double* probs,
                       int64_t probs_stride, int32_t num_threads) {
  if (num_requests < 1 || num_heads < 1 || num_tree == NULL || prefix_len == NULL || q == NULL ||
      kv_pool == NULL || slot_table == NULL || slot_indptr == NULL || parent == NULL ||
      out == NULL || lse == NULL || kv_row_stride < ORACLE_D_QK)
    return ORACLE_ERR_ARG;

  /* Row bookkeeping and per-request checks. */
  int64_t total_tree = 0;
  for (int32_t r = 0; r < num_requests; ++r) {
    if (num_tree[r] < 1 || prefix_len[r] < 0) return ORACLE_ERR_ARG;
    const int64_t n = (int64_t)prefix_len[r] + num_tree[r];
    if ((int64_t)slot_indptr[r + 1] - slot_indptr[r] < n) return ORACLE_ERR_TABLE;
    if (probs != NULL && probs_stride < n) return ORACLE_ERR_ARG;
    total_tree += num_tree[r];
  }
  const int64_t total_rows = total_tree * num_heads;
  int64_t* row_req = (int64_t*)malloc((size_t)total_rows * sizeof(int64_t));
  int64_t* row_node = (int64_t*)malloc((size_t)total_rows * sizeof(int64_t));
  int64_t* tree_begin = (int64_t*)malloc((size_t)(num_requests + 1) * sizeof(int64_t));
  if (row_req == NULL || row_node == NULL || tree_begin == NULL) {
    free(row_req); free(row_node); free(tree_begin);
    return ORACLE_ERR_NOMEM;
  }
  tree_begin[0] = 0;
  for (int32_t r = 0; r < num_requests; ++r) {
    tree_begin[r + 1] = tree_begin[r] + num_tree[r];
    for (int64_t i = 0; i < num_tree[r]; ++i)
      for (int32_t h = 0; h < num_heads; ++h) {
        const int64_t row = (tree_begin[r] + i) * num_heads + h;
        row_req[row] = r;
        row_node[row] = i;
      }
  }
  int status = ORACLE_OK;
  for (int32_t r = 0; r < num_requests && status == ORACLE_OK; ++r) {
    uint8_t* vis = (uint8_t*)malloc((size_t)num_tree[r] * num_tree[r]);
    if (vis == NULL) { status = ORACLE_ERR_NOMEM; break; }
    status = oracle_tree_visibility(parent + tree_begin[r], num_tree[r], vis);
    free(vis);
  }
  if (status != ORACLE_OK) {
    free(row_req); free(row_node); free(tree_begin);
    return status;
  }

#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t row = 0; row < total_rows; ++row) {
    if (row_select != NULL && row_select[row] == 0) continue;
    const int64_t r = row_req[row];
    const int64_t i = row_node[row];
    const int32_t T = num_tree[r];
    const int32_t L = prefix_len[r];
    const int32_t* table = slot_table + slot_indptr[r];

    uint8_t* vis = (uint8_t*)malloc((size_t)T * T);
    int32_t* slots = (int32_t*)malloc((size_t)(L + T) * sizeof(int32_t));
    int64_t* keys = (int64_t*)malloc((size_t)(L + T) * sizeof(int64_t));
    double* p = (double*)malloc((size_t)(L + T) * sizeof(double));
    double qd[ORACLE_D_QK];
    int rc = (vis && slots && keys && p) ? ORACLE_OK : ORACLE_ERR_NOMEM;
    if (rc == ORACLE_OK) rc = oracle_tree_visibility(parent + tree_begin[r], T, vis);
    if (rc == ORACLE_OK) {
      /* Visible logical keys: the whole prefix, then anc*(i) in node order. */
      int64_t n = 0;
      for (int64_t k = 0; k < L; ++k) keys[n++] = k;
      for (int32_t j = 0; j < T; ++j)
        if (vis[i * T + j]) keys[n++] = (int64_t)L + j;
      for (int64_t k = 0; k < n; ++k) slots[k] = table[keys[k]];
      const uint16_t* qrow = q + row * ORACLE_D_QK;
      for (int d = 0; d < ORACLE_D_QK; ++d) qd[d] = bf16_to_double(qrow[d]);
      rc = oracle_attend(qd, kv_pool, num_slots, kv_row_stride, slots, n, sm_scale,
                         out + row * ORACLE_D_V, lse + row, p);
      if (rc == ORACLE_OK && probs != NULL) {
        double* prow = probs + row * probs_stride;
        for (int64_t k = 0; k < (int64_t)L + T; ++k) prow[k] = 0.0;
        for (int64_t k = 0; k < n; ++k) prow[keys[k]] = p[k];
      }
    }
    if (rc != ORACLE_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
      status = rc;
    }
    free(vis); free(slots); free(keys); free(p);
  }
  free(row_req); free(row_node); free(tree_begin);
  return status;
}
