/*
 * libseer: gated block-sparse decode attention for AMD Instinct MI355X (gfx950).
 *
 * One decode step of one attention layer: every sequence has one new query
 * token; its query heads attend, in groups of G = Hq / Hkv heads per KV head
 * (grouped-query attention), to a KV cache cut into blocks of S tokens.  For
 * every (sequence, KV head) the blocks are scored against the group's query
 * through a pooled summary of each block's keys, the top-scoring blocks are
 * kept, and exact softmax attention runs over the kept blocks only.
 *
 * Sources: "SeerAttention-R: Sparse Attention Adaptation for Long Reasoning"
 * (Abstract; AI Summary) -- block-level gating on pooled keys with the query
 * not pooled, block sizes 64/128, 90% sparsity or a token budget, a sparse
 * decoding kernel; "Sparse Attention Reasoning" (Step 1: top-k selection from
 * gate scores; Step 4: softmax(QK^T/sqrt(d)) with unselected keys masked).
 * The gate is parameter free: the score of block j for KV head g is
 *     s_j = sum_{h in group g} q_h . P_j / sqrt(d),
 * P_j the fp32-stored mean of the block's valid keys.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Every pointer except `shape`/`kv` structs and host-only helpers is a
 *    device pointer.  The caller allocates and owns all memory; the library
 *    allocates nothing and keeps no state between calls, except the static
 *    scratch array of seer_gated_sparse_decode_no_alloc (one per GPU).
 *  - Work is enqueued on `stream` and is asynchronous; no call synchronises.
 *  - Arguments are validated on the host before anything is enqueued: a bad
 *    argument returns SEER_ERR_INVALID_ARG / SEER_ERR_UNSUPPORTED /
 *    SEER_ERR_WORKSPACE and enqueues nothing.  A failed launch returns
 *    SEER_ERR_HIP.  seer_last_error() describes the last failure of the
 *    calling thread.  Nothing aborts and no exception crosses this interface.
 *  - Values that live on the device (lengths, counts, block ids, page ids)
 *    cannot be checked without a synchronisation.  Their contract is stated
 *    per call; kernels skip out-of-range ids instead of reading out of bounds.
 *  - Calls that share output or scratch buffers on one stream are ordered by
 *    the stream; concurrent calls on different streams must not share them.
 *  - q, k, v, the pooled table and the workspace must be 16-byte aligned
 *    (open_sum 8-byte); a misaligned one returns SEER_ERR_INVALID_ARG
 *    (SEER_ERR_WORKSPACE for the workspace).
 *
 * Supported: head_dim d in {64, 128}; block_size S in {64, 128}; G = Hq/Hkv in
 * 1..8; dtype fp32 or bf16 for q, k, v (one dtype for all three); at most
 * SEER_MAX_UNITS (sequence, KV head) pairs.  Outputs are fp32.
 */
#ifndef SEER_H_
#define SEER_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SEER_MAX_UNITS 8192

typedef enum seer_status {
  SEER_OK = 0,
  SEER_ERR_INVALID_ARG = 1,  /* null pointer, inconsistent sizes, bad rule */
  SEER_ERR_UNSUPPORTED = 2,  /* valid but outside the supported set above */
  SEER_ERR_WORKSPACE = 3,    /* workspace missing or too small */
  SEER_ERR_HIP = 4           /* a HIP runtime call or launch failed */
} seer_status;

typedef enum seer_dtype { SEER_F32 = 0, SEER_BF16 = 1 } seer_dtype;

/* Problem shape, shared by all calls. */
typedef struct seer_shape {
  int32_t batch;        /* B: sequences */
  int32_t num_q_heads;  /* Hq */
  int32_t num_kv_heads; /* Hkv; Hq must be a multiple of Hkv */
  int32_t head_dim;     /* d */
  int32_t block_size;   /* S: tokens per block (= tokens per page when paged) */
  int32_t max_blocks;   /* NB: blocks per sequence that the cache and tables hold */
  int32_t dtype;        /* seer_dtype of q, k and v */
} seer_shape;

/* The KV cache.
 *  page_table == NULL: contiguous, k and v are [B][Hkv][NB*S][d] (the
 *    (batch, heads, key_len, head_dim) layout of "Sparse Attention
 *    Reasoning", Step 4), row t of sequence b / head g at
 *    ((b*Hkv + g)*NB*S + t)*d.
 *  page_table != NULL: [B][NB] int32 page ids; k and v are pools
 *    [num_pages][Hkv][S][d]; block j of sequence b lives in page
 *    page_table[b*NB + j].  Ids outside [0, num_pages) make that block empty. */
typedef struct seer_kv {
  const void* k;
  const void* v;
  const int32_t* page_table;
  int64_t num_pages;
} seer_kv;

/* Pooled-key table layout used by the calls below (fp32, "d-major"):
 *   pooled[((b*Hkv + g)*d + i)*NB + j] = mean over the valid tokens t of block j
 *   of k[b][g][t][i], the sum taken in fp64 in token order, divided by the
 *   block's token count and rounded to fp32 (nearest even).
 * open_sum[(b*Hkv + g)*d + i] = the fp64 sum of the last block's keys.
 * Keys are pooled per block; the query is not ("SeerAttention-R", Abstract). */

/* seer_block_pool_keys -- builds or extends the pooled-key table.
 *
 *  lens_old == NULL: bulk build.  Writes pooled[..][j] for every block
 *    j < ceil(lens_new[b] / S) and open_sum, from the first lens_new[b] tokens.
 *  lens_old != NULL: incremental append of tokens lens_old[b] .. lens_new[b]-1
 *    (their keys must already be in the cache).  The fp64 running sum in
 *    open_sum restarts when a token opens a new block; the pooled column of
 *    every block that gets a token is rewritten.  Bit-identical to a bulk build
 *    over lens_new tokens.  Requires the table to be built up to lens_old.
 *  Device contract: 1 <= lens_new[b] <= NB*S; lens_old[b] <= lens_new[b]
 *  (sequences with lens_old[b] >= lens_new[b] are left unchanged).
 *  pooled: [B][Hkv][d][NB] fp32; open_sum: [B][Hkv][d] fp64 (in/out). */
seer_status seer_block_pool_keys(const seer_shape* shape, const seer_kv* kv,
                                 const int32_t* lens_old, const int32_t* lens_new,
                                 float* pooled, double* open_sum, hipStream_t stream);

/* seer_gate_scores_topk -- gate scores and top-k block selection.
 *
 *  q: [B][Hq][d] (shape->dtype).  pooled: the table above.  lens: [B] tokens
 *  per sequence including the new one (1 <= lens[b] <= NB*S); n_b =
 *  ceil(lens[b] / S).
 *  Kept count k_b ("Sparse Attention Reasoning", Step 1; "SeerAttention-R",
 *  Abstract: 90% sparsity, 4K token budget):
 *    top_k != NULL: k_b = clamp(top_k[b], 1, n_b) (a token budget T is
 *      top_k = T / S), then at most k_max;
 *    top_k == NULL: k_b = max(1, min(n_b, ceil(n_b * keep_num / keep_den)))
 *      in integer arithmetic (90% sparsity: keep_num = 1, keep_den = 10);
 *      requires 1 <= keep_num <= keep_den and that NB blocks keep <= k_max.
 *  Order: score descending, ties to the lower block id, -0.0 == +0.0; scores
 *  must be finite.
 *  scores: [B][Hkv][NB] fp64 out, s_j for j < n_b (the rest untouched).
 *  sel_idx: [B][Hkv][k_max] int32 out: the kept ids in ascending order, then -1.
 *  sel_cnt: [B][Hkv] int32 out: k_b. */
seer_status seer_gate_scores_topk(const seer_shape* shape, const void* q, const float* pooled,
                                  const int32_t* lens, const int32_t* top_k, int32_t keep_num,
                                  int32_t keep_den, int32_t k_max, double* scores,
                                  int32_t* sel_idx, int32_t* sel_cnt, hipStream_t stream);

/* Selection rule of seer_gate_select and seer_gated_sparse_decode.
 *  mode SEER_SELECT_TOPK: k_b as in seer_gate_scores_topk (top_k[b] when
 *    top_k != NULL, else the keep fraction keep_num / keep_den).
 *  mode SEER_SELECT_THRESHOLD: keep the blocks whose score is above
 *    `threshold` -- the hard gate of "Sparse Attention Reasoning" (Step 1:
 *    the selection with a temperature keeps sigmoid(s / T) > 0.5, which is
 *    s > 0 for any T > 0) with a general threshold; at least 1 block (the
 *    best), at most k_max (the best k_max).
 *  force_first / force_last: block 0 (an attention sink) and the newest block
 *    n_b - 1 are kept whatever their score; a top-k count below the number of
 *    forced blocks is raised to it (still at most min(n_b, k_max)).
 *  unified: one selection per sequence, from the scores summed over its KV
 *    heads, s_j = sum_g sum_{h in group g} q_h . P_{g,j} / sqrt(d) (the KV
 *    heads added in order), copied to every KV head of the sequence (the
 *    cross-head selection of the LessIsMore abstract on the author page
 *    "Shijie Cao"); scores[b][g] then holds the summed score for every g.
 *  The order is score descending, ties to the lower block id, as everywhere. */
typedef enum seer_select_mode { SEER_SELECT_TOPK = 0, SEER_SELECT_THRESHOLD = 1 } seer_select_mode;
/* How the gated decode calls run the selection (results are bit-identical
 * either way): AUTO lets the library choose per shape (see
 * seer_gated_sparse_decode), ALWAYS runs it inside the attention kernel
 * whenever the rule allows that (top-k, not unified) and it fits in LDS,
 * NEVER runs the gate kernel first.  Ignored by the gate-only calls. */
typedef enum seer_fuse { SEER_FUSE_AUTO = 0, SEER_FUSE_ALWAYS = 1, SEER_FUSE_NEVER = 2 } seer_fuse;
typedef struct seer_select {
  int32_t mode;            /* seer_select_mode */
  const int32_t* top_k;    /* TOPK: device [B] counts, or NULL for the keep fraction */
  int32_t keep_num;        /* TOPK without top_k: kept fraction keep_num / keep_den */
  int32_t keep_den;
  double threshold;        /* THRESHOLD: keep blocks scoring above it (finite) */
  int32_t force_first;     /* nonzero: keep block 0 */
  int32_t force_last;      /* nonzero: keep block n_b - 1 */
  int32_t unified;         /* nonzero: one selection per sequence over its KV heads */
  int32_t fuse;            /* seer_fuse (0 = SEER_FUSE_AUTO); other values: SEER_ERR_INVALID_ARG */
} seer_select;

/* seer_gate_select -- seer_gate_scores_topk under a general rule (above);
 * same arguments otherwise.  seer_gate_scores_topk(top_k, keep_num, keep_den)
 * is this call with {SEER_SELECT_TOPK, top_k, keep_num, keep_den}.
 * SEER_ERR_UNSUPPORTED when max_blocks needs more LDS than one workgroup has. */
seer_status seer_gate_select(const seer_shape* shape, const void* q, const float* pooled,
                             const int32_t* lens, const seer_select* rule, int32_t k_max,
                             double* scores, int32_t* sel_idx, int32_t* sel_cnt,
                             hipStream_t stream);

/* Weights of the learned gate network, one set per KV head (device memory).
 * hidden must be 256.
 *   w1       int8  [Hkv][256][d]   first layer, row m = hidden unit m
 *   w1_scale float [Hkv][256]      row scales: the weight is w1_scale[m] * w1[m][i]
 *   b1       float [Hkv][256]      first-layer bias
 *   wq       float [Hkv][256][d]   query projection (the second layer's weights)
 * w1 and wq must be 16-byte aligned, w1_scale and b1 4-byte aligned. */
typedef struct seer_gate_weights {
  const int8_t* w1;
  const float* w1_scale;
  const float* b1;
  const float* wq;
  int32_t hidden;
} seer_gate_weights;

/* seer_learned_gate_select -- gate scores from a learned gate network, then
 * the selection rule of seer_gate_select.
 *
 *  The network is the gate of "Sparse Attention Reasoning" (Step 1:
 *  Linear(d, 256), ReLU, Linear(256, 1)) applied to every block's pooled key;
 *  its second layer's weights are a projection of the group's query, so that
 *  the decode query is used unpooled ("SeerAttention-R", Abstract).  For KV
 *  head g of sequence b, block j:
 *    z_jm = w1_scale[m] * (w1[m] . P_j) + b1[m],
 *    s_j  = sum_m u_m * max(z_jm, 0),  u_m = wq[m] . qbar,
 *  qbar the sum of the group's query heads, P_j the stored fp32 pooled key.
 *  Arithmetic and its error bound: the first layer runs on int8 matrix cores
 *  over an image of P_j in five int8 limbs under the block exponent e_j (the
 *  smallest integer with 127 * 2^e_j >= max_i |P_ji|, 0 for a zero block),
 *  which holds every key element to within 2^(e_j - 29); the int32 products
 *  are exact and everything after them is fp64.  So
 *    |s_j - s_j(exact)| <= 2^(e_j - 29) * sum_m |u_m| w1_scale[m] ||w1[m]||_1
 *  plus fp64 rounding, and the selection is that of the exact scores
 *  wherever no two candidates are closer than twice that.
 *  scores (fp64), sel_idx, sel_cnt, lens, k_max and the rule are as in
 *  seer_gate_select; a unified rule is SEER_ERR_UNSUPPORTED, so are
 *  hidden != 256 and tables that need more LDS than one workgroup has.
 *  Missing or misaligned weights: SEER_ERR_INVALID_ARG. */
seer_status seer_learned_gate_select(const seer_shape* shape, const void* q, const float* pooled,
                                     const int32_t* lens, const seer_gate_weights* weights,
                                     const seer_select* rule, int32_t k_max, double* scores,
                                     int32_t* sel_idx, int32_t* sel_cnt, hipStream_t stream);

/* Bytes of workspace seer_sparse_decode needs for this shape on the current
 * device (it depends on the device's compute-unit count). */
seer_status seer_sparse_decode_workspace_size(const seer_shape* shape, size_t* bytes);

/* seer_sparse_decode -- exact softmax attention over the kept blocks.
 *
 *  For every query head h of sequence b, with g = h / G:
 *    T = { valid tokens t < lens[b] of the blocks sel_idx[b][g][0..sel_cnt[b][g]) },
 *    out[b][h] = sum_{t in T} softmax_t(l) v_t,  l_t = scale * (q_h . k_t),
 *    lse[b][h] = log sum_{t in T} exp(l_t)  (natural log),
 *  the attention of "Sparse Attention Reasoning", Step 4, with every key
 *  outside T masked to -inf, computed without touching keys outside T.
 *  sel_idx == NULL: dense decode, T = all lens[b] tokens (sel_cnt unused).
 *  sel_idx/sel_cnt: as written by seer_gate_scores_topk, or any ids in
 *  [0, n_b) (order free, no duplicates); ids outside [0, n_b) and counts
 *  outside [0, k_max] are skipped/clamped.  A head with no token gets out = 0
 *  and lse = -inf.
 *  softmax_scale <= 0 selects 1/sqrt(d).
 *  out: [B][Hq][d] fp32; lse: [B][Hq] fp32 or NULL.
 *  workspace: seer_sparse_decode_workspace_size bytes of device scratch; its
 *  contents need no initialisation and are overwritten. */
seer_status seer_sparse_decode(const seer_shape* shape, const void* q, const seer_kv* kv,
                               const int32_t* lens, const int32_t* sel_idx,
                               const int32_t* sel_cnt, int32_t k_max, float softmax_scale,
                               float* out, float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* The two stages of seer_sparse_decode, for callers that time or overlap them:
 * _partial streams the kept K/V and leaves per-split partial results in the
 * workspace (with the split plan); _combine reads them and merges them by
 * log-sum-exp into out/lse.  _partial followed by _combine on the same
 * workspace and stream is exactly seer_sparse_decode.
 * The merge runs one workgroup per (sequence, KV head), or one per query head
 * when the units are few for the device (at least 8 partial results each on
 * average) and the query heads at least 64.
 * seer_sparse_decode_combine_mode is _combine with that choice made by the
 * caller: SEER_COMBINE_AUTO (the rule above), SEER_COMBINE_PER_UNIT or
 * SEER_COMBINE_PER_HEAD; any other mode is SEER_ERR_INVALID_ARG.  The modes
 * run the same fp32 operations in the same record order and give
 * bit-identical out and lse. */
seer_status seer_sparse_decode_partial(const seer_shape* shape, const void* q, const seer_kv* kv,
                                       const int32_t* lens, const int32_t* sel_idx,
                                       const int32_t* sel_cnt, int32_t k_max,
                                       float softmax_scale, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);
seer_status seer_sparse_decode_combine(const seer_shape* shape, float* out, float* lse,
                                       const void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);
typedef enum seer_combine_mode {
  SEER_COMBINE_AUTO = 0,
  SEER_COMBINE_PER_UNIT = 1,
  SEER_COMBINE_PER_HEAD = 2
} seer_combine_mode;
seer_status seer_sparse_decode_combine_mode(const seer_shape* shape, int32_t mode, float* out,
                                            float* lse, const void* workspace,
                                            size_t workspace_bytes, hipStream_t stream);

/* seer_gated_sparse_decode -- one decode step from the pooled table: gate
 * scores, top-k selection and sparse attention, as seer_gate_scores_topk
 * followed by seer_sparse_decode on its selection, with bit-identical
 * results (scores, sel_idx, sel_cnt, out, lse), in two launches instead of
 * three: every workgroup of the attention kernel selects the blocks of the
 * (sequence, KV head) pairs it streams itself, so the attention does not wait
 * for a separate gate launch ("SeerAttention-R: Sparse Attention Adaptation
 * for Long Reasoning", Abstract: gating on pooled keys with a sparse decoding
 * kernel; "Sparse Attention Reasoning", Step 1 and Step 4).
 *  Arguments: as seer_gate_select (q, pooled, lens, rule, k_max, scores,
 *  sel_idx, sel_cnt, all outputs written) and seer_sparse_decode (kv,
 *  softmax_scale, out, lse, workspace).
 *  The selection is fused for top-k rules (forced blocks included) while
 *  every workgroup gates about one unit in one pass: at most one (sequence,
 *  KV head) unit per workgroup of the attention kernel and at most 256
 *  blocks per unit.  With longer tables (and a top-k rule, at most one unit
 *  per workgroup, rule->fuse left to the library) the gate's score kernel
 *  scores the table first and the attention kernel's workgroups select from
 *  those scores (the selection launch is saved).  For a threshold or unified
 *  rule, more units, or when one workgroup's selections would not fit in its
 *  LDS, the call runs the gate kernel(s) first instead (same results, one
 *  launch more).  seer_gated_decode_is_fused tells which for a shape.
 *  rule->fuse overrides the choice (SEER_FUSE_ALWAYS scores and selects in
 *  the attention kernel whenever the rule allows it and the selections fit
 *  in LDS, SEER_FUSE_NEVER never selects there); the results do not depend
 *  on it.
 * _partial: the first launch(es) alone (gate + partial results in the
 * workspace, selections written); seer_sparse_decode_combine finishes it. */
/* seer_learned_gated_sparse_decode -- one decode step with the learned gate:
 * seer_learned_gate_select followed by seer_sparse_decode on its selection,
 * with bit-identical results (scores, sel_idx, sel_cnt, out, lse) ("Sparse
 * Attention Reasoning", Step 1: the gate network and its top-k; Step 4: the
 * attention over the kept blocks).  Where the learned gate gives each
 * (sequence, KV head) unit several workgroups (few units: its scores go to
 * memory), the rule is a per-unit top-k (forced blocks allowed), every
 * attention workgroup meets at most one unit and rule->fuse is not
 * SEER_FUSE_NEVER, the attention kernel's workgroups select from those
 * scores in place of a selection launch; otherwise the three launches run
 * as the two calls would.
 *  Arguments: as seer_learned_gate_select (q, pooled, lens, weights, rule,
 *  k_max, scores, sel_idx, sel_cnt, all written) and seer_sparse_decode (kv,
 *  softmax_scale, out, lse, workspace); out = NULL stops after the partial
 *  results in the workspace (seer_sparse_decode_combine finishes them).
 *  Errors: those of the two calls, before any launch. */
seer_status seer_learned_gated_sparse_decode(
    const seer_shape* shape, const void* q, const seer_kv* kv, const int32_t* lens,
    const float* pooled, const seer_gate_weights* weights, const seer_select* rule, int32_t k_max,
    float softmax_scale, double* scores, int32_t* sel_idx, int32_t* sel_cnt, float* out,
    float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);
/* seer_gated_decode_is_fused -- *fused = 1 if seer_gated_sparse_decode
 * (tokens = 1) or seer_multi_gated_sparse_decode (tokens > 1) with this shape,
 * rule and k_max scores and selects inside the attention kernel on the
 * current device, 2 if the gate's score kernel scores first and the attention
 * kernel selects (tokens = 1 only), 0 if it runs the gate kernel(s) first (no
 * launch; results are the same either way).  SEER_ERR_INVALID_ARG for NULL pointers, k_max outside [1,
 * max_blocks] or a token count outside [1, 16 / G]. */
seer_status seer_gated_decode_is_fused(const seer_shape* shape, int32_t tokens,
                                       const seer_select* rule, int32_t k_max, int32_t* fused);
seer_status seer_gated_sparse_decode(const seer_shape* shape, const void* q, const seer_kv* kv,
                                     const int32_t* lens, const float* pooled,
                                     const seer_select* rule, int32_t k_max,
                                     float softmax_scale, double* scores, int32_t* sel_idx,
                                     int32_t* sel_cnt, float* out, float* lse, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);
seer_status seer_gated_sparse_decode_partial(const seer_shape* shape, const void* q,
                                             const seer_kv* kv, const int32_t* lens,
                                             const float* pooled, const seer_select* rule,
                                             int32_t k_max, float softmax_scale, double* scores,
                                             int32_t* sel_idx, int32_t* sel_cnt,
                                             void* workspace, size_t workspace_bytes,
                                             hipStream_t stream);

/* seer_gated_sparse_decode_no_alloc -- seer_gated_sparse_decode without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The workspace is a static device array of 16 MiB that the
 * library holds on every GPU it runs on until the process ends; its device
 * address is looked up once per device, on the first call with that device
 * current.  The call allocates nothing (no hipMalloc, no allocating library
 * routine) and writes the same scores, sel_idx, sel_cnt, out and lse as
 * seer_gated_sparse_decode with a workspace.
 *  Arguments: as seer_gated_sparse_decode, less the workspace.
 *  A shape whose workspace (seer_sparse_decode_workspace_size) exceeds 16 MiB
 *  returns SEER_ERR_WORKSPACE and enqueues nothing.
 *  Every call on one GPU shares that GPU's array, and the array keeps the
 *  last call's contents (nothing in it needs to start at zero): calls that
 *  may overlap on one GPU (several streams, several host threads) race on it
 *  and must be serialised by the caller. */
seer_status seer_gated_sparse_decode_no_alloc(const seer_shape* shape, const void* q,
                                              const seer_kv* kv, const int32_t* lens,
                                              const float* pooled, const seer_select* rule,
                                              int32_t k_max, float softmax_scale, double* scores,
                                              int32_t* sel_idx, int32_t* sel_cnt, float* out,
                                              float* lse, hipStream_t stream);

/* seer_gated_sparse_decode_append -- one decode step after new tokens entered
 * the cache: seer_block_pool_keys(kv, lens_old, lens, pooled, open_sum)
 * followed by seer_gated_sparse_decode(lens, pooled, ...), with bit-identical
 * results (pooled, open_sum, scores, sel_idx, sel_cnt, out, lse).  Where the
 * step has a score kernel for per-unit rules, the pooling append runs inside
 * it (the open block's new mean is computed, used and written there), one
 * launch fewer; otherwise it is its own launch first.  The keys of tokens
 * lens_old[b] .. lens[b] - 1 must be in the cache.
 *  Arguments: as seer_block_pool_keys (kv, lens_old, pooled and open_sum in
 *  and out) and seer_gated_sparse_decode (the rest; lens = lens_new).
 *  Errors as those calls'; lens_old NULL is SEER_ERR_INVALID_ARG. */
seer_status seer_gated_sparse_decode_append(const seer_shape* shape, const void* q,
                                            const seer_kv* kv, const int32_t* lens_old,
                                            const int32_t* lens, float* pooled, double* open_sum,
                                            const seer_select* rule, int32_t k_max,
                                            float softmax_scale, double* scores,
                                            int32_t* sel_idx, int32_t* sel_cnt, float* out,
                                            float* lse, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/* Several new query tokens per sequence (speculative or chunked decode).
 *
 *  Sequence b has `tokens` = T new query tokens at positions
 *  lens[b] - T .. lens[b] - 1, their keys and values already in the cache
 *  (lens includes them; lens[b] >= T).  q is [B][T][Hq][d] (the dtype of the
 *  shape).  Token t attends to the kept blocks' tokens at positions
 *  <= lens[b] - T + t ("Sparse Attention Reasoning", Step 4, with query_len =
 *  T and the causal mask of autoregressive decoding); one selection per
 *  (sequence, KV head) serves all T tokens.  Supported: 1 <= T and
 *  G * T <= 16 (SEER_ERR_UNSUPPORTED otherwise).
 *
 * seer_multi_gate_select -- seer_gate_select with the gate's query summed over
 *  the T tokens and the group's heads (token-major, fp64): the query pooling of
 *  SeerAttention, which "-R" removes for single-token decoding
 *  ("SeerAttention-R", Abstract).  Other arguments as seer_gate_select.
 *
 * seer_multi_sparse_decode_workspace_size -- bytes of workspace the decode
 *  below needs for this shape and token count on the current device.
 *
 * seer_multi_sparse_decode -- the attention of the T tokens over the given
 *  selection (sel_idx/sel_cnt/k_max as in seer_sparse_decode; sel_idx NULL
 *  means every block).  out: [B][T][Hq][d] fp32; lse: [B][T][Hq] fp32 natural
 *  log, or NULL.  A token that sees no key gets out = 0 and lse = -inf.
 *  Two launches (partial records, then their merge) on `stream`. */
seer_status seer_multi_gate_select(const seer_shape* shape, int32_t tokens, const void* q,
                                   const float* pooled, const int32_t* lens,
                                   const seer_select* rule, int32_t k_max, double* scores,
                                   int32_t* sel_idx, int32_t* sel_cnt, hipStream_t stream);
seer_status seer_multi_sparse_decode_workspace_size(const seer_shape* shape, int32_t tokens,
                                                    size_t* bytes);
seer_status seer_multi_sparse_decode(const seer_shape* shape, int32_t tokens, const void* q,
                                     const seer_kv* kv, const int32_t* lens,
                                     const int32_t* sel_idx, const int32_t* sel_cnt,
                                     int32_t k_max, float softmax_scale, float* out, float* lse,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* The two stages of seer_multi_sparse_decode, as seer_sparse_decode_partial
 * and seer_sparse_decode_combine are of seer_sparse_decode: _partial leaves
 * 16-row partial results and the split plan in the workspace; _combine merges
 * them into out/lse.  The same shape, token count, workspace and stream must
 * be given to both. */
seer_status seer_multi_sparse_decode_partial(const seer_shape* shape, int32_t tokens,
                                             const void* q, const seer_kv* kv,
                                             const int32_t* lens, const int32_t* sel_idx,
                                             const int32_t* sel_cnt, int32_t k_max,
                                             float softmax_scale, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream);
seer_status seer_multi_sparse_decode_combine(const seer_shape* shape, int32_t tokens, float* out,
                                             float* lse, const void* workspace,
                                             size_t workspace_bytes, hipStream_t stream);

/* seer_multi_gated_sparse_decode -- one decode step of T new query tokens
 * from the pooled table: seer_multi_gate_select followed by
 * seer_multi_sparse_decode on its selection, with bit-identical results
 * (scores, sel_idx, sel_cnt, out, lse), the gate fused into the attention
 * kernel under the same conditions as seer_gated_sparse_decode (each
 * workgroup selects the units it streams; otherwise the gate kernel runs
 * first).  Arguments as those two calls; workspace:
 * seer_multi_sparse_decode_workspace_size bytes.
 * _partial: the selection and the partial results alone;
 * seer_multi_sparse_decode_combine finishes it. */
seer_status seer_multi_gated_sparse_decode(
    const seer_shape* shape, int32_t tokens, const void* q, const seer_kv* kv,
    const int32_t* lens, const float* pooled, const seer_select* rule, int32_t k_max,
    float softmax_scale, double* scores, int32_t* sel_idx, int32_t* sel_cnt, float* out,
    float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);
seer_status seer_multi_gated_sparse_decode_partial(
    const seer_shape* shape, int32_t tokens, const void* q, const seer_kv* kv,
    const int32_t* lens, const float* pooled, const seer_select* rule, int32_t k_max,
    float softmax_scale, double* scores, int32_t* sel_idx, int32_t* sel_cnt, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/* Host helper: max(1, min(n, ceil(n * keep_num / keep_den))), or -1 for bad
 * arguments (n < 1, keep_num < 1, keep_den < keep_num). */
int32_t seer_keep_blocks(int32_t n_blocks, int32_t keep_num, int32_t keep_den);

/* Static name of a status code. */
const char* seer_status_str(int32_t status);

/* Text of the last failure on the calling thread ("" if none). */
const char* seer_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SEER_H_ */
