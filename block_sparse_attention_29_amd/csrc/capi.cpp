// C-ABI of libseer: host-side validation and launch of the gfx950 kernels.
// The public contract of every entry point is documented in include/seer.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "seer.h"
#include "seer_kernels.h"

static_assert(seer::kMaxUnits == SEER_MAX_UNITS, "unit limit mismatch");

namespace {

thread_local char g_err[512] = "";

seer_status fail(seer_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
seer_status fail(seer_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

seer_status ok() {
  g_err[0] = '\0';
  return SEER_OK;
}

seer_status hip_fail(hipError_t e, const char* what) {
  return fail(SEER_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxBlocks = 8192;
constexpr int64_t kMaxTokens = int64_t(1) << 30;

seer_status check_shape(const seer_shape* s) {
  if (!s) return fail(SEER_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->head_dim < 1 ||
      s->block_size < 1 || s->max_blocks < 1)
    return fail(SEER_ERR_INVALID_ARG, "shape fields must be positive");
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(SEER_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                s->num_q_heads, s->num_kv_heads);
  if (s->dtype != SEER_F32 && s->dtype != SEER_BF16)
    return fail(SEER_ERR_INVALID_ARG, "dtype %d is not a seer_dtype", s->dtype);
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G > 8) return fail(SEER_ERR_UNSUPPORTED, "query heads per KV head %d > 8", G);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(SEER_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", s->head_dim);
  if (s->block_size != 64 && s->block_size != 128)
    return fail(SEER_ERR_UNSUPPORTED, "block_size %d not in {64, 128}", s->block_size);
  if ((int64_t)s->batch * s->num_kv_heads > SEER_MAX_UNITS)
    return fail(SEER_ERR_UNSUPPORTED, "batch * num_kv_heads = %lld > %d",
                (long long)s->batch * s->num_kv_heads, SEER_MAX_UNITS);
  if (s->max_blocks > kMaxBlocks)
    return fail(SEER_ERR_UNSUPPORTED, "max_blocks %d > %d", s->max_blocks, kMaxBlocks);
  if ((int64_t)s->max_blocks * s->block_size > kMaxTokens)
    return fail(SEER_ERR_UNSUPPORTED, "max_blocks * block_size exceeds 2^30 tokens");
  return SEER_OK;
}

// The kernels move q, k, v, pooled rows and partial records in 16-byte loads.
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

seer_status check_kv(const seer_kv* kv) {
  if (!kv) return fail(SEER_ERR_INVALID_ARG, "kv is NULL");
  if (!kv->k || !kv->v) return fail(SEER_ERR_INVALID_ARG, "kv.k or kv.v is NULL");
  if (!aligned16(kv->k) || !aligned16(kv->v))
    return fail(SEER_ERR_INVALID_ARG, "kv.k and kv.v must be 16-byte aligned");
  if (kv->page_table && kv->num_pages < 1)
    return fail(SEER_ERR_INVALID_ARG, "paged cache with num_pages < 1");
  return SEER_OK;
}

int wave_cap(const seer_shape* s) {
  return seer::decode_max_waves(s->dtype, s->head_dim, s->num_q_heads / s->num_kv_heads);
}

// Waves of a partial launch: all resident slots, but no more than an upper
// bound of the 16-token tiles (blocks_per_unit blocks per unit), in whole
// workgroups.
int decode_waves(const seer_shape* s, int64_t blocks_per_unit, int wmax) {
  const int64_t tiles_bound =
      (int64_t)s->batch * s->num_kv_heads * blocks_per_unit * (s->block_size / 16);
  int64_t W = tiles_bound < wmax ? tiles_bound : wmax;
  W = (W + seer::kDecodeWavesPerWG - 1) / seer::kDecodeWavesPerWG * seer::kDecodeWavesPerWG;
  return (int)W;
}

// Whether the attention kernel selects its own blocks (one launch fewer) for
// this shape, rule and wave count.  It pays while every workgroup gates about
// one unit in a single pass over its pooled table: at most one unit per
// workgroup (with more, a workgroup gates several units one after another,
// each behind its own load round trip and selection, where the gate kernel
// gates them all in parallel), and at most 256 blocks per unit (the blocks
// one pass of the workgroup's loads covers; a longer table makes every
// workgroup that shares the unit re-score all of it).
// rule->fuse = SEER_FUSE_ALWAYS fuses whenever the rule allows it,
// SEER_FUSE_NEVER never (the results are the same either way).
bool fused_gate_pays(const seer_shape* s, const seer_select* rule, int W) {
  if (rule->mode != SEER_SELECT_TOPK || rule->unified) return false;
  if (rule->fuse == SEER_FUSE_ALWAYS) return true;
  if (rule->fuse == SEER_FUSE_NEVER) return false;
  const int U = s->batch * s->num_kv_heads;
  return U <= W / seer::kDecodeWavesPerWG && s->max_blocks <= 256;
}

// Whether the single-token combine runs one workgroup per query head instead
// of one per unit, when the caller leaves the choice to the library: when the
// units average 8 or more partial records at full width (few, long units: a
// workgroup per unit leaves most CUs idle and gives each thread long chains of
// record loads) and there are at least 64 query heads.  Measured per step: 32
// units x 8 heads at 131K tokens 49.9 -> 49.0 us, 64 units x 4 heads 18.3 ->
// 18.0 us; with 512 units (3-4 records each) the 2560 small workgroups cost
// 2.7 us more, and one unit of 4 heads 3.9 us more.
bool combine_per_head(const seer_shape* s, int wmax) {
  const int64_t U = (int64_t)s->batch * s->num_kv_heads;
  return U * 8 <= wmax && (int64_t)s->batch * s->num_q_heads >= 64;
}

// Validates a decode call and fills the partial kernel's arguments.
seer_status prepare_decode(const seer_shape* shape, const void* q, const seer_kv* kv,
                           const int32_t* lens, const int32_t* sel_idx, const int32_t* sel_cnt,
                           int32_t k_max, float softmax_scale, void* workspace,
                           size_t workspace_bytes, seer::DecodeArgs* out_args) {
  seer_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_kv(kv))) return st;
  if (!q || !lens) return fail(SEER_ERR_INVALID_ARG, "q or lens is NULL");
  if (!aligned16(q)) return fail(SEER_ERR_INVALID_ARG, "q must be 16-byte aligned");
  if (sel_idx) {
    if (!sel_cnt) return fail(SEER_ERR_INVALID_ARG, "sel_idx given without sel_cnt");
    if (k_max < 1 || k_max > shape->max_blocks)
      return fail(SEER_ERR_INVALID_ARG, "k_max %d outside [1, max_blocks=%d]", k_max,
                  shape->max_blocks);
  }
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale))
    return fail(SEER_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (!workspace) return fail(SEER_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(SEER_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const int wmax = wave_cap(shape);
  if (wmax <= 0) return fail(SEER_ERR_HIP, "cannot query the current device");
  const int U = shape->batch * shape->num_kv_heads;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const size_t need = seer::decode_workspace_bytes(shape->batch, shape->num_kv_heads, G,
                                                   shape->head_dim, wmax);
  if (workspace_bytes < need)
    return fail(SEER_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);

  const int W = decode_waves(shape, sel_idx ? k_max : shape->max_blocks, wmax);

  const double scale = softmax_scale > 0.f ? (double)softmax_scale
                                           : 1.0 / sqrt((double)shape->head_dim);
  seer::DecodeArgs& a = *out_args;
  a = seer::DecodeArgs{};
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.page_table = kv->page_table;
  a.num_pages = kv->num_pages;
  a.lens = lens;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.B = shape->batch;
  a.Hq = shape->num_q_heads;
  a.Hkv = shape->num_kv_heads;
  a.D = shape->head_dim;
  a.NB = shape->max_blocks;
  a.S = shape->block_size;
  a.k_max = sel_idx ? k_max : shape->max_blocks;
  a.dtype = shape->dtype;
  a.W = (int32_t)W;
  a.scale_log2 = (float)(scale * 1.4426950408889634074);
  char* ws = (char*)workspace;
  a.hdr = (int32_t*)ws;
  a.prefix = (int32_t*)(ws + 64);
  a.part = (float*)(ws + seer::decode_part_offset(U));
  return SEER_OK;
}

// Validates the gate's arguments.
seer_status check_gate(const seer_shape* shape, const void* q, const float* pooled,
                       const int32_t* lens, const seer_select* rule, int32_t k_max,
                       const double* scores, const int32_t* sel_idx, const int32_t* sel_cnt) {
  seer_status st = check_shape(shape);
  if (st) return st;
  if (!q || !pooled || !lens || !rule || !scores || !sel_idx || !sel_cnt)
    return fail(SEER_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(q) || !aligned16(pooled))
    return fail(SEER_ERR_INVALID_ARG, "q and pooled must be 16-byte aligned");
  if (k_max < 1 || k_max > shape->max_blocks)
    return fail(SEER_ERR_INVALID_ARG, "k_max %d outside [1, max_blocks=%d]", k_max,
                shape->max_blocks);
  if (rule->mode != SEER_SELECT_TOPK && rule->mode != SEER_SELECT_THRESHOLD)
    return fail(SEER_ERR_INVALID_ARG, "selection mode %d is not a seer_select_mode", rule->mode);
  if (rule->fuse != SEER_FUSE_AUTO && rule->fuse != SEER_FUSE_ALWAYS &&
      rule->fuse != SEER_FUSE_NEVER)
    return fail(SEER_ERR_INVALID_ARG, "fuse %d is not a seer_fuse", rule->fuse);
  if (rule->mode == SEER_SELECT_THRESHOLD) {
    if (!(rule->threshold == rule->threshold) || isinf(rule->threshold))
      return fail(SEER_ERR_INVALID_ARG, "threshold is not finite");
  } else if (!rule->top_k) {
    const int32_t kk = seer_keep_blocks(shape->max_blocks, rule->keep_num, rule->keep_den);
    if (kk < 0)
      return fail(SEER_ERR_INVALID_ARG, "keep rule %d/%d invalid (need 1 <= num <= den)",
                  rule->keep_num, rule->keep_den);
    if (kk > k_max)
      return fail(SEER_ERR_INVALID_ARG, "keep rule keeps %d of max_blocks=%d blocks > k_max=%d",
                  kk, shape->max_blocks, k_max);
  }
  return SEER_OK;
}

// Largest dynamic LDS one workgroup may use on the current device.
size_t max_block_smem() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return 0;
  return (size_t)v;
}

// Static LDS of the attention kernel with the gate fused in (tokens > 1: the
// multi-token kernel), or (size_t)-1.
size_t gated_static_smem(const seer_shape* s, int tokens) {
  if (tokens > 1) return seer::gated_decode_multi_static_smem(s->dtype, s->head_dim);
  return seer::gated_decode_static_smem(s->dtype, s->head_dim, s->num_q_heads / s->num_kv_heads);
}

// Whether the call with W waves runs the attention kernel with the gate fused
// in: the rule and shape make it pay, and its LDS (static + ids + keys) fits.
bool fused_gate_runs(const seer_shape* s, const seer_select* rule, int32_t k_max, int W,
                     int tokens) {
  if (!fused_gate_pays(s, rule, W)) return false;
  const int U = s->batch * s->num_kv_heads;
  const size_t st = gated_static_smem(s, tokens);
  if (st == (size_t)-1) return false;
  const size_t dyn = seer::gated_decode_smem_bytes(U, s->max_blocks,
                                                   seer::gated_decode_ids_cap(U, k_max, W));
  return st + dyn <= max_block_smem();
}

// Whether a single-token call with W waves takes the scores from the gate's
// score kernel and selects inside the attention kernel: a per-unit top-k rule
// left to the library, a table of more than one 256-block score chunk (where
// re-scoring it in every workgroup that shares a unit costs more than the
// selection launch it saves), at most one unit per workgroup, and the LDS
// fits.  Each workgroup then selects its units from their scores (the unit's
// selection, bit-identical in every workgroup) in place of a selection launch
// and its round trips.
// Whether the single-token attention kernel with W waves can select from
// given scores for this rule: a per-unit top-k rule, at most one unit per
// workgroup, and its LDS fits.
bool given_scores_fit(const seer_shape* s, const seer_select* rule, int32_t k_max, int W) {
  if (rule->mode != SEER_SELECT_TOPK || rule->unified) return false;
  const int U = s->batch * s->num_kv_heads;
  if (U > W / seer::kDecodeWavesPerWG) return false;
  const size_t st = gated_static_smem(s, 1);
  if (st == (size_t)-1) return false;
  const size_t dyn = seer::gated_decode_smem_bytes(U, s->max_blocks,
                                                   seer::gated_decode_ids_cap(U, k_max, W));
  return st + dyn <= max_block_smem();
}

bool given_scores_runs(const seer_shape* s, const seer_select* rule, int32_t k_max, int W,
                       int tokens) {
  if (tokens != 1 || rule->fuse != SEER_FUSE_AUTO) return false;
  if (s->max_blocks <= seer::kGateScoreChunk) return false;
  return given_scores_fit(s, rule, k_max, W);
}

// How a gated call selects, for this shape, rule and wave count.
enum GatePath {
  kGateKernels = 0,  // the gate kernel(s) first, then the attention kernel
  kGateFused = 1,    // scores and selection inside the attention kernel
  kGateScoresThenFused = 2,  // the score kernel, then selection inside the attention kernel
};

GatePath gate_path(const seer_shape* s, const seer_select* rule, int32_t k_max, int W,
                   int tokens) {
  if (fused_gate_runs(s, rule, k_max, W, tokens)) return kGateFused;
  if (given_scores_runs(s, rule, k_max, W, tokens)) return kGateScoresThenFused;
  return kGateKernels;
}

// Turns the partial kernel's arguments into the fused gate's: the kernel
// selects by the rule and writes scores, ids and counts.
void set_fused_gate(const seer_shape* s, const float* pooled, const seer_select* rule,
                    int32_t k_max, double* scores, int32_t* sel_idx, int32_t* sel_cnt,
                    seer::DecodeArgs& a) {
  const int U = s->batch * s->num_kv_heads;
  a.sel_idx = nullptr;
  a.sel_cnt = nullptr;
  a.pooled = pooled;
  a.top_k = rule->top_k;
  a.keep_num = rule->keep_num;
  a.keep_den = rule->keep_den;
  a.force_first = rule->force_first != 0;
  a.force_last = rule->force_last != 0;
  a.scores = scores;
  a.sel_idx_out = sel_idx;
  a.sel_cnt_out = sel_cnt;
  a.ids_cap = seer::gated_decode_ids_cap(U, k_max, a.W);
}


// The gate kernels' arguments from a validated call.
seer::GateArgs gate_args(const seer_shape* shape, const void* q, const float* pooled,
                         const int32_t* lens, const seer_select* rule, int32_t k_max,
                         double* scores, int32_t* sel_idx, int32_t* sel_cnt) {
  seer::GateArgs a{};
  a.q = q;
  a.pooled = pooled;
  a.lens = lens;
  a.top_k = rule->top_k;
  a.keep_num = rule->keep_num;
  a.keep_den = rule->keep_den;
  a.k_max = k_max;
  a.B = shape->batch;
  a.Hq = shape->num_q_heads;
  a.Hkv = shape->num_kv_heads;
  a.D = shape->head_dim;
  a.NB = shape->max_blocks;
  a.S = shape->block_size;
  a.dtype = shape->dtype;
  a.scores = scores;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.threshold_mode = rule->mode == SEER_SELECT_THRESHOLD;
  a.threshold = rule->threshold;
  a.force_first = rule->force_first != 0;
  a.force_last = rule->force_last != 0;
  a.unified = rule->unified != 0;
  a.tokens = 1;
  return a;
}


// Token count of a multi-token call.
seer_status check_tokens(const seer_shape* shape, int32_t tokens) {
  const int G = shape->num_q_heads / shape->num_kv_heads;
  if (tokens < 1) return fail(SEER_ERR_INVALID_ARG, "tokens %d < 1", tokens);
  if ((int64_t)G * tokens > seer::kMultiRows)
    return fail(SEER_ERR_UNSUPPORTED, "G * tokens = %lld > %d query rows per KV head",
                (long long)G * tokens, seer::kMultiRows);
  return SEER_OK;
}

// Validates a learned gate call and fills the gate kernels' arguments.
seer_status learned_gate_args(const seer_shape* shape, const void* q, const float* pooled,
                              const int32_t* lens, const seer_gate_weights* weights,
                              const seer_select* rule, int32_t k_max, double* scores,
                              int32_t* sel_idx, int32_t* sel_cnt, seer::GateArgs* out) {
  const seer_status st = check_gate(shape, q, pooled, lens, rule, k_max, scores, sel_idx, sel_cnt);
  if (st) return st;
  if (!weights || !weights->w1 || !weights->w1_scale || !weights->b1 || !weights->wq)
    return fail(SEER_ERR_INVALID_ARG, "gate weights missing");
  if (!aligned16(weights->w1) || !aligned16(weights->wq) || ((uintptr_t)weights->w1_scale & 3) ||
      ((uintptr_t)weights->b1 & 3))
    return fail(SEER_ERR_INVALID_ARG,
                "gate weights misaligned (w1 and wq 16-byte aligned, w1_scale and b1 4-byte)");
  if (weights->hidden != seer::kGateHidden)
    return fail(SEER_ERR_UNSUPPORTED, "gate hidden width %d != %d", weights->hidden,
                seer::kGateHidden);
  if (rule->unified)
    return fail(SEER_ERR_UNSUPPORTED, "a unified selection is not supported by the learned gate");
  seer::GateArgs a = gate_args(shape, q, pooled, lens, rule, k_max, scores, sel_idx, sel_cnt);
  a.w1 = weights->w1;
  a.w1_scale = weights->w1_scale;
  a.b1 = weights->b1;
  a.wq = weights->wq;
  if (seer::learned_gate_smem_total(a.D, a.NB) > max_block_smem())
    return fail(SEER_ERR_UNSUPPORTED, "max_blocks %d needs more LDS than a workgroup has", a.NB);
  *out = a;
  return SEER_OK;
}


}  // namespace

extern "C" {

const char* seer_status_str(int32_t st) {
  switch (st) {
    case SEER_OK: return "SEER_OK";
    case SEER_ERR_INVALID_ARG: return "SEER_ERR_INVALID_ARG";
    case SEER_ERR_UNSUPPORTED: return "SEER_ERR_UNSUPPORTED";
    case SEER_ERR_WORKSPACE: return "SEER_ERR_WORKSPACE";
    case SEER_ERR_HIP: return "SEER_ERR_HIP";
  }
  return "SEER_STATUS_UNKNOWN";
}

const char* seer_last_error(void) { return g_err; }

int32_t seer_keep_blocks(int32_t n, int32_t num, int32_t den) {
  if (n < 1 || num < 1 || den < num) return -1;
  const int64_t k = ((int64_t)n * num + den - 1) / den;
  return (int32_t)(k < 1 ? 1 : (k > n ? n : k));
}

seer_status seer_block_pool_keys(const seer_shape* shape, const seer_kv* kv,
                                 const int32_t* lens_old, const int32_t* lens_new,
                                 float* pooled, double* open_sum, hipStream_t stream) {
  seer_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_kv(kv))) return st;
  if (!lens_new) return fail(SEER_ERR_INVALID_ARG, "lens_new is NULL");
  if (!pooled || !open_sum) return fail(SEER_ERR_INVALID_ARG, "pooled or open_sum is NULL");
  if (!aligned16(pooled) || ((uintptr_t)open_sum & 7) != 0)
    return fail(SEER_ERR_INVALID_ARG, "pooled must be 16-byte and open_sum 8-byte aligned");
  seer::PoolArgs a{};
  a.k = kv->k;
  a.page_table = kv->page_table;
  a.num_pages = kv->num_pages;
  a.lens_old = lens_old;
  a.lens_new = lens_new;
  a.B = shape->batch;
  a.Hkv = shape->num_kv_heads;
  a.D = shape->head_dim;
  a.NB = shape->max_blocks;
  a.S = shape->block_size;
  a.dtype = shape->dtype;
  a.pooled = pooled;
  a.open_sum = open_sum;
  const hipError_t e = seer::launch_pool_keys(a, stream);
  if (e != hipSuccess) return hip_fail(e, "pool_keys launch");
  return ok();
}


seer_status seer_gate_select(const seer_shape* shape, const void* q, const float* pooled,
                             const int32_t* lens, const seer_select* rule, int32_t k_max,
                             double* scores, int32_t* sel_idx, int32_t* sel_cnt,
                             hipStream_t stream) {
  const seer_status st = check_gate(shape, q, pooled, lens, rule, k_max, scores, sel_idx, sel_cnt);
  if (st) return st;
  const seer::GateArgs a =
      gate_args(shape, q, pooled, lens, rule, k_max, scores, sel_idx, sel_cnt);
  if (seer::gate_smem_bytes(a.NB, k_max) > max_block_smem())
    return fail(SEER_ERR_UNSUPPORTED, "max_blocks %d needs more LDS than a workgroup has", a.NB);
  const hipError_t e = seer::launch_gate_topk(a, stream);
  if (e != hipSuccess) return hip_fail(e, "gate_topk launch");
  return ok();
}

seer_status seer_learned_gate_select(const seer_shape* shape, const void* q, const float* pooled,
                                     const int32_t* lens, const seer_gate_weights* weights,
                                     const seer_select* rule, int32_t k_max, double* scores,
                                     int32_t* sel_idx, int32_t* sel_cnt, hipStream_t stream) {
  seer::GateArgs a;
  const seer_status st = learned_gate_args(shape, q, pooled, lens, weights, rule, k_max, scores,
                                           sel_idx, sel_cnt, &a);
  if (st) return st;
  const hipError_t e = seer::launch_learned_gate(a, stream);
  if (e != hipSuccess) return hip_fail(e, "learned_gate launch");
  return ok();
}


seer_status seer_gate_scores_topk(const seer_shape* shape, const void* q, const float* pooled,
                                  const int32_t* lens, const int32_t* top_k, int32_t keep_num,
                                  int32_t keep_den, int32_t k_max, double* scores,
                                  int32_t* sel_idx, int32_t* sel_cnt, hipStream_t stream) {
  seer_select rule{};
  rule.mode = SEER_SELECT_TOPK;
  rule.top_k = top_k;
  rule.keep_num = keep_num;
  rule.keep_den = keep_den;
  return seer_gate_select(shape, q, pooled, lens, &rule, k_max, scores, sel_idx, sel_cnt, stream);
}

seer_status seer_sparse_decode_workspace_size(const seer_shape* shape, size_t* bytes) {
  seer_status st = check_shape(shape);
  if (st) return st;
  if (!bytes) return fail(SEER_ERR_INVALID_ARG, "bytes is NULL");
  const int wmax = wave_cap(shape);
  if (wmax <= 0) return fail(SEER_ERR_HIP, "cannot query the current device");
  *bytes = seer::decode_workspace_bytes(shape->batch, shape->num_kv_heads,
                                        shape->num_q_heads / shape->num_kv_heads,
                                        shape->head_dim, wmax);
  return ok();
}

seer_status seer_sparse_decode_partial(const seer_shape* shape, const void* q, const seer_kv* kv,
                                       const int32_t* lens, const int32_t* sel_idx,
                                       const int32_t* sel_cnt, int32_t k_max,
                                       float softmax_scale, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  seer::DecodeArgs a;
  const seer_status st = prepare_decode(shape, q, kv, lens, sel_idx, sel_cnt, k_max,
                                        softmax_scale, workspace, workspace_bytes, &a);
  if (st) return st;
  const hipError_t e = seer::launch_decode_partial(a, stream);
  if (e != hipSuccess) return hip_fail(e, "decode_partial launch");
  return ok();
}

}  // extern "C"

namespace {

// The gated partial step, with the pooling append of tokens lens_old[b] ..
// lens[b] - 1 first when lens_old is given (pooled and open_sum updated as
// seer_block_pool_keys would): the append runs inside the score kernel where
// the gate has one (per-unit rules), else as its own launch.
seer_status gated_partial(const seer_shape* shape, const void* q, const seer_kv* kv,
                          const int32_t* lens_old, const int32_t* lens, float* pooled,
                          double* open_sum, const seer_select* rule, int32_t k_max,
                          float softmax_scale, double* scores, int32_t* sel_idx,
                          int32_t* sel_cnt, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  seer_status st = check_gate(shape, q, pooled, lens, rule, k_max, scores, sel_idx, sel_cnt);
  if (st) return st;
  const bool append = lens_old != nullptr;
  if (append && (!open_sum || ((uintptr_t)open_sum & 7) != 0))
    return fail(SEER_ERR_INVALID_ARG, "open_sum missing or not 8-byte aligned");
  if (append && (st = check_kv(kv))) return st;
  seer::DecodeArgs a;
  if ((st = prepare_decode(shape, q, kv, lens, sel_idx, sel_cnt, k_max, softmax_scale,
                           workspace, workspace_bytes, &a)))
    return st;
  seer::GateArgs ga = gate_args(shape, q, pooled, lens, rule, k_max, scores, sel_idx, sel_cnt);
  if (append) {
    ga.lens_old = lens_old;
    ga.k = kv->k;
    ga.page_table = kv->page_table;
    ga.num_pages = kv->num_pages;
    ga.pooled_out = pooled;
    ga.open_sum = open_sum;
  }
  const GatePath path = gate_path(shape, rule, k_max, a.W, 1);
  // a separate append launch where no score kernel takes it
  const bool own_append = append && (path == kGateFused || !seer::gate_topk_appends(ga));
  if (own_append &&
      (st = seer_block_pool_keys(shape, kv, lens_old, lens, pooled, open_sum, stream)))
    return st;
  ga.append = append && !own_append;
  hipError_t e = hipSuccess;
  switch (path) {
    case kGateFused:
      set_fused_gate(shape, pooled, rule, k_max, scores, sel_idx, sel_cnt, a);
      e = seer::launch_gated_decode_partial(a, stream);
      if (e != hipSuccess) return hip_fail(e, "gated decode_partial launch");
      break;
    case kGateScoresThenFused:
      e = seer::launch_gate_scores(ga, stream);
      if (e != hipSuccess) return hip_fail(e, "gate score launch");
      set_fused_gate(shape, pooled, rule, k_max, scores, sel_idx, sel_cnt, a);
      a.scores_in = scores;
      e = seer::launch_gated_decode_partial(a, stream);
      if (e != hipSuccess) return hip_fail(e, "gated decode_partial launch");
      break;
    default:
      if (seer::gate_smem_bytes(ga.NB, k_max) > max_block_smem())
        return fail(SEER_ERR_UNSUPPORTED, "max_blocks %d needs more LDS than a workgroup has",
                    ga.NB);
      e = seer::launch_gate_topk(ga, stream);
      if (e != hipSuccess) return hip_fail(e, "gate_topk launch");
      e = seer::launch_decode_partial(a, stream);
      if (e != hipSuccess) return hip_fail(e, "decode_partial launch");
  }
  return ok();
}

}  // namespace

extern "C" {

seer_status seer_gated_sparse_decode_partial(const seer_shape* shape, const void* q,
                                             const seer_kv* kv, const int32_t* lens,
                                             const float* pooled, const seer_select* rule,
                                             int32_t k_max, float softmax_scale, double* scores,
                                             int32_t* sel_idx, int32_t* sel_cnt,
                                             void* workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
  return gated_partial(shape, q, kv, nullptr, lens, const_cast<float*>(pooled), nullptr, rule,
                       k_max, softmax_scale, scores, sel_idx, sel_cnt, workspace,
                       workspace_bytes, stream);
}

seer_status seer_gated_sparse_decode_append(const seer_shape* shape, const void* q,
                                            const seer_kv* kv, const int32_t* lens_old,
                                            const int32_t* lens, float* pooled, double* open_sum,
                                            const seer_select* rule, int32_t k_max,
                                            float softmax_scale, double* scores,
                                            int32_t* sel_idx, int32_t* sel_cnt, float* out,
                                            float* lse, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  if (!out) return fail(SEER_ERR_INVALID_ARG, "out is NULL");
  if (!lens_old) return fail(SEER_ERR_INVALID_ARG, "lens_old is NULL");
  const seer_status st = gated_partial(shape, q, kv, lens_old, lens, pooled, open_sum, rule,
                                       k_max, softmax_scale, scores, sel_idx, sel_cnt, workspace,
                                       workspace_bytes, stream);
  if (st) return st;
  return seer_sparse_decode_combine(shape, out, lse, workspace, workspace_bytes, stream);
}

seer_status seer_learned_gated_sparse_decode(
    const seer_shape* shape, const void* q, const seer_kv* kv, const int32_t* lens,
    const float* pooled, const seer_gate_weights* weights, const seer_select* rule, int32_t k_max,
    float softmax_scale, double* scores, int32_t* sel_idx, int32_t* sel_cnt, float* out,
    float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  seer::GateArgs ga;
  seer_status st = learned_gate_args(shape, q, pooled, lens, weights, rule, k_max, scores,
                                     sel_idx, sel_cnt, &ga);
  if (st) return st;
  seer::DecodeArgs a;
  if ((st = prepare_decode(shape, q, kv, lens, sel_idx, sel_cnt, k_max, softmax_scale,
                           workspace, workspace_bytes, &a)))
    return st;
  const int U = shape->batch * shape->num_kv_heads;
  hipError_t e;
  // Where the learned gate splits a unit over several workgroups its scores go
  // to memory anyway: the attention kernel's workgroups then select from them
  // (as the selection launch would, bit for bit) instead of a selection launch.
  if (seer::learned_gate_workgroups_per_unit(U, shape->max_blocks) > 1 &&
      rule->fuse != SEER_FUSE_NEVER && given_scores_fit(shape, rule, k_max, a.W)) {
    if ((e = seer::launch_learned_gate_scores(ga, stream)) != hipSuccess)
      return hip_fail(e, "learned gate score launch");
    set_fused_gate(shape, pooled, rule, k_max, scores, sel_idx, sel_cnt, a);
    a.scores_in = scores;
    if ((e = seer::launch_gated_decode_partial(a, stream)) != hipSuccess)
      return hip_fail(e, "gated decode_partial launch");
  } else {
    if ((e = seer::launch_learned_gate(ga, stream)) != hipSuccess)
      return hip_fail(e, "learned_gate launch");
    if ((e = seer::launch_decode_partial(a, stream)) != hipSuccess)
      return hip_fail(e, "decode_partial launch");
  }
  if (!out) return ok();
  return seer_sparse_decode_combine(shape, out, lse, workspace, workspace_bytes, stream);
}

seer_status seer_gated_decode_is_fused(const seer_shape* shape, int32_t tokens,
                                       const seer_select* rule, int32_t k_max, int32_t* fused) {
  seer_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_tokens(shape, tokens))) return st;
  if (!rule || !fused) return fail(SEER_ERR_INVALID_ARG, "rule or fused is NULL");
  if (rule->fuse != SEER_FUSE_AUTO && rule->fuse != SEER_FUSE_ALWAYS &&
      rule->fuse != SEER_FUSE_NEVER)
    return fail(SEER_ERR_INVALID_ARG, "fuse %d is not a seer_fuse", rule->fuse);
  if (k_max < 1 || k_max > shape->max_blocks)
    return fail(SEER_ERR_INVALID_ARG, "k_max %d outside [1, max_blocks]", k_max);
  const int wmax = wave_cap(shape);
  if (wmax <= 0) return fail(SEER_ERR_HIP, "cannot query the current device");
  // the same wave count and test as the gated decode calls
  *fused = (int32_t)gate_path(shape, rule, k_max, decode_waves(shape, k_max, wmax), tokens);
  return ok();
}

seer_status seer_gated_sparse_decode(const seer_shape* shape, const void* q, const seer_kv* kv,
                                     const int32_t* lens, const float* pooled,
                                     const seer_select* rule, int32_t k_max,
                                     float softmax_scale, double* scores,
                                     int32_t* sel_idx, int32_t* sel_cnt, float* out, float* lse,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  if (!out) return fail(SEER_ERR_INVALID_ARG, "out is NULL");
  const seer_status st = seer_gated_sparse_decode_partial(
      shape, q, kv, lens, pooled, rule, k_max, softmax_scale, scores, sel_idx, sel_cnt,
      workspace, workspace_bytes, stream);
  if (st) return st;
  return seer_sparse_decode_combine(shape, out, lse, workspace, workspace_bytes, stream);
}

seer_status seer_gated_sparse_decode_no_alloc(const seer_shape* shape, const void* q,
                                              const seer_kv* kv, const int32_t* lens,
                                              const float* pooled, const seer_select* rule,
                                              int32_t k_max, float softmax_scale, double* scores,
                                              int32_t* sel_idx, int32_t* sel_cnt, float* out,
                                              float* lse, hipStream_t stream) {
  seer_status st = check_shape(shape);
  if (st) return st;
  const int wmax = wave_cap(shape);
  if (wmax <= 0) return fail(SEER_ERR_HIP, "cannot query the current device");
  const size_t need = seer::decode_workspace_bytes(
      shape->batch, shape->num_kv_heads, shape->num_q_heads / shape->num_kv_heads,
      shape->head_dim, wmax);
  if (need > seer::kStaticScratchBytes)
    return fail(SEER_ERR_WORKSPACE,
                "this shape needs %zu bytes of scratch, more than the %zu bytes of the static "
                "scratch; use seer_gated_sparse_decode with a workspace",
                need, seer::kStaticScratchBytes);
  hipError_t e = hipSuccess;
  void* ws = seer::decode_static_scratch(&e);
  if (!ws) return hip_fail(e, "static scratch address");
  return seer_gated_sparse_decode(shape, q, kv, lens, pooled, rule, k_max, softmax_scale, scores,
                                  sel_idx, sel_cnt, out, lse, ws, seer::kStaticScratchBytes,
                                  stream);
}

seer_status seer_sparse_decode_combine_mode(const seer_shape* shape, int32_t mode, float* out,
                                            float* lse, const void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  seer_status st = check_shape(shape);
  if (st) return st;
  if (mode != SEER_COMBINE_AUTO && mode != SEER_COMBINE_PER_UNIT && mode != SEER_COMBINE_PER_HEAD)
    return fail(SEER_ERR_INVALID_ARG, "combine mode %d is not a seer_combine_mode", mode);
  if (!out) return fail(SEER_ERR_INVALID_ARG, "out is NULL");
  if (!workspace) return fail(SEER_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(SEER_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const int wmax = wave_cap(shape);
  if (wmax <= 0) return fail(SEER_ERR_HIP, "cannot query the current device");
  const int U = shape->batch * shape->num_kv_heads;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const size_t need = seer::decode_workspace_bytes(shape->batch, shape->num_kv_heads, G,
                                                   shape->head_dim, wmax);
  if (workspace_bytes < need)
    return fail(SEER_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  const char* ws = (const char*)workspace;
  seer::CombineArgs c{};
  c.B = shape->batch;
  c.Hq = shape->num_q_heads;
  c.Hkv = shape->num_kv_heads;
  c.D = shape->head_dim;
  c.S = shape->block_size;
  c.hdr = (const int32_t*)ws;
  c.prefix = (const int32_t*)(ws + 64);
  c.part = (const float*)(ws + seer::decode_part_offset(U));
  c.out = out;
  c.lse = lse;
  c.per_head = mode == SEER_COMBINE_PER_HEAD ||
               (mode == SEER_COMBINE_AUTO && combine_per_head(shape, wmax));
  const hipError_t e = seer::launch_decode_combine(c, stream);
  if (e != hipSuccess) return hip_fail(e, "decode_combine launch");
  return ok();
}

seer_status seer_sparse_decode_combine(const seer_shape* shape, float* out, float* lse,
                                       const void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  return seer_sparse_decode_combine_mode(shape, SEER_COMBINE_AUTO, out, lse, workspace,
                                         workspace_bytes, stream);
}

seer_status seer_multi_gate_select(const seer_shape* shape, int32_t tokens, const void* q,
                                   const float* pooled, const int32_t* lens,
                                   const seer_select* rule, int32_t k_max, double* scores,
                                   int32_t* sel_idx, int32_t* sel_cnt, hipStream_t stream) {
  seer_status st = check_gate(shape, q, pooled, lens, rule, k_max, scores, sel_idx, sel_cnt);
  if (st) return st;
  if ((st = check_tokens(shape, tokens))) return st;
  seer::GateArgs a = gate_args(shape, q, pooled, lens, rule, k_max, scores, sel_idx, sel_cnt);
  a.tokens = tokens;
  if (seer::gate_smem_bytes(a.NB, k_max) > max_block_smem())
    return fail(SEER_ERR_UNSUPPORTED, "max_blocks %d needs more LDS than a workgroup has", a.NB);
  const hipError_t e = seer::launch_gate_topk(a, stream);
  if (e != hipSuccess) return hip_fail(e, "gate_topk launch");
  return ok();
}

seer_status seer_multi_sparse_decode_workspace_size(const seer_shape* shape, int32_t tokens,
                                                    size_t* bytes) {
  seer_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_tokens(shape, tokens))) return st;
  if (!bytes) return fail(SEER_ERR_INVALID_ARG, "bytes is NULL");
  const int wmax = wave_cap(shape);
  if (wmax <= 0) return fail(SEER_ERR_HIP, "cannot query the current device");
  *bytes = seer::decode_multi_workspace_bytes(shape->batch, shape->num_kv_heads, shape->head_dim,
                                              wmax);
  return ok();
}

seer_status seer_multi_sparse_decode_partial(const seer_shape* shape, int32_t tokens,
                                             const void* q, const seer_kv* kv,
                                             const int32_t* lens, const int32_t* sel_idx,
                                             const int32_t* sel_cnt, int32_t k_max,
                                             float softmax_scale, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  seer_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_tokens(shape, tokens))) return st;
  seer::DecodeArgs a;
  if ((st = prepare_decode(shape, q, kv, lens, sel_idx, sel_cnt, k_max, softmax_scale, workspace,
                           workspace_bytes, &a)))
    return st;
  const size_t need = seer::decode_multi_workspace_bytes(shape->batch, shape->num_kv_heads,
                                                         shape->head_dim, wave_cap(shape));
  if (workspace_bytes < need)
    return fail(SEER_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  a.tokens = tokens;
  const hipError_t e = seer::launch_decode_multi(a, stream);
  if (e != hipSuccess) return hip_fail(e, "multi decode launch");
  return ok();
}

seer_status seer_multi_sparse_decode_combine(const seer_shape* shape, int32_t tokens, float* out,
                                             float* lse, const void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  seer_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_tokens(shape, tokens))) return st;
  if (!out) return fail(SEER_ERR_INVALID_ARG, "out is NULL");
  if (!workspace) return fail(SEER_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(SEER_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const int wmax = wave_cap(shape);
  if (wmax <= 0) return fail(SEER_ERR_HIP, "cannot query the current device");
  const size_t need = seer::decode_multi_workspace_bytes(shape->batch, shape->num_kv_heads,
                                                         shape->head_dim, wmax);
  if (workspace_bytes < need)
    return fail(SEER_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  const int U = shape->batch * shape->num_kv_heads;
  const char* ws = (const char*)workspace;
  seer::CombineArgs c{};
  c.B = shape->batch;
  c.Hq = shape->num_q_heads;
  c.Hkv = shape->num_kv_heads;
  c.D = shape->head_dim;
  c.S = shape->block_size;
  c.tokens = tokens;
  c.hdr = (const int32_t*)ws;
  c.prefix = (const int32_t*)(ws + 64);
  c.part = (const float*)(ws + seer::decode_part_offset(U));
  c.out = out;
  c.lse = lse;
  const hipError_t e = seer::launch_decode_multi_combine(c, stream);
  if (e != hipSuccess) return hip_fail(e, "multi combine launch");
  return ok();
}

seer_status seer_multi_sparse_decode(const seer_shape* shape, int32_t tokens, const void* q,
                                     const seer_kv* kv, const int32_t* lens,
                                     const int32_t* sel_idx, const int32_t* sel_cnt,
                                     int32_t k_max, float softmax_scale, float* out, float* lse,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  if (!out) return fail(SEER_ERR_INVALID_ARG, "out is NULL");
  const seer_status st = seer_multi_sparse_decode_partial(
      shape, tokens, q, kv, lens, sel_idx, sel_cnt, k_max, softmax_scale, workspace,
      workspace_bytes, stream);
  if (st) return st;
  return seer_multi_sparse_decode_combine(shape, tokens, out, lse, workspace, workspace_bytes,
                                          stream);
}

seer_status seer_multi_gated_sparse_decode_partial(
    const seer_shape* shape, int32_t tokens, const void* q, const seer_kv* kv,
    const int32_t* lens, const float* pooled, const seer_select* rule, int32_t k_max,
    float softmax_scale, double* scores, int32_t* sel_idx, int32_t* sel_cnt, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  seer_status st = check_gate(shape, q, pooled, lens, rule, k_max, scores, sel_idx, sel_cnt);
  if (st) return st;
  if ((st = check_tokens(shape, tokens))) return st;
  seer::DecodeArgs a;
  if ((st = prepare_decode(shape, q, kv, lens, sel_idx, sel_cnt, k_max, softmax_scale,
                           workspace, workspace_bytes, &a)))
    return st;
  const size_t need = seer::decode_multi_workspace_bytes(shape->batch, shape->num_kv_heads,
                                                         shape->head_dim, wave_cap(shape));
  if (workspace_bytes < need)
    return fail(SEER_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  a.tokens = tokens;
  if (fused_gate_runs(shape, rule, k_max, a.W, tokens)) {
    set_fused_gate(shape, pooled, rule, k_max, scores, sel_idx, sel_cnt, a);
    const hipError_t e = seer::launch_gated_decode_multi(a, stream);
    if (e != hipSuccess) return hip_fail(e, "gated multi decode launch");
  } else {
    if ((st = seer_multi_gate_select(shape, tokens, q, pooled, lens, rule, k_max, scores, sel_idx,
                                     sel_cnt, stream)))
      return st;
    const hipError_t e = seer::launch_decode_multi(a, stream);
    if (e != hipSuccess) return hip_fail(e, "multi decode launch");
  }
  return ok();
}

seer_status seer_multi_gated_sparse_decode(
    const seer_shape* shape, int32_t tokens, const void* q, const seer_kv* kv,
    const int32_t* lens, const float* pooled, const seer_select* rule, int32_t k_max,
    float softmax_scale, double* scores, int32_t* sel_idx, int32_t* sel_cnt, float* out,
    float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!out) return fail(SEER_ERR_INVALID_ARG, "out is NULL");
  const seer_status st = seer_multi_gated_sparse_decode_partial(
      shape, tokens, q, kv, lens, pooled, rule, k_max, softmax_scale, scores, sel_idx, sel_cnt,
      workspace, workspace_bytes, stream);
  if (st) return st;
  return seer_multi_sparse_decode_combine(shape, tokens, out, lse, workspace, workspace_bytes,
                                          stream);
}

seer_status seer_sparse_decode(const seer_shape* shape, const void* q, const seer_kv* kv,
                               const int32_t* lens, const int32_t* sel_idx,
                               const int32_t* sel_cnt, int32_t k_max, float softmax_scale,
                               float* out, float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  if (!out) return fail(SEER_ERR_INVALID_ARG, "out is NULL");
  seer_status st = seer_sparse_decode_partial(shape, q, kv, lens, sel_idx, sel_cnt, k_max,
                                              softmax_scale, workspace, workspace_bytes, stream);
  if (st) return st;
  return seer_sparse_decode_combine(shape, out, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"
