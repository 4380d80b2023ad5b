// Internal launch interface between the C-ABI layer (capi.cpp) and the
// kernels.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace seer {

// ---------------------------------------------------------------- decode

// Waves per workgroup of the partial-decode kernel: one wave per SIMD, and one
// workgroup per CU.  A second wave on a SIMD (or a second workgroup on a CU)
// is younger, and the hardware's oldest-first arbitration serves its loads
// last: it starts later and streams slower than its older neighbour, which
// leaves a long tail of half-occupied CUs.
constexpr int kDecodeWavesPerWG = 4;

// Largest number of (sequence, KV head) units a call may have.
constexpr int kMaxUnits = 8192;
// Most waves one partial launch uses (the equal tile split does its
// arithmetic in 32 bits up to 46340 waves).
constexpr int kMaxWaves = 32768;

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* page_table;
  int64_t num_pages;
  const int32_t* lens;
  const int32_t* sel_idx;  // nullptr: dense
  const int32_t* sel_cnt;
  int32_t B, Hq, Hkv, D, NB, S, k_max;
  int32_t dtype;          // 0 fp32, 1 bf16
  int32_t W;              // waves of the partial kernel (multiple of kDecodeWavesPerWG)
  float scale_log2;       // softmax scale * log2(e)
  int32_t* hdr;           // workspace header: [0] = W
  int32_t* prefix;        // [U + 1] block prefix over units
  float* part;            // [(U + Wmax)][G*D + 16] partial records
  // Fused gate (gated kernel only): each workgroup selects the blocks of the
  // units it streams.  sel_idx/sel_cnt above are unused then.
  const float* pooled;    // [B][Hkv][D][NB]
  const int32_t* top_k;   // [B] or nullptr (then keep_num / keep_den)
  int32_t keep_num, keep_den;
  double* scores;         // [B][Hkv][NB] out
  int32_t* sel_idx_out;   // [B][Hkv][k_max] out
  int32_t* sel_cnt_out;   // [B][Hkv] out
  int32_t ids_cap;        // kept ids one workgroup holds in LDS
  int32_t force_first, force_last;  // forced blocks of the fused gate's top-k
  int32_t tokens;         // new query tokens per sequence (multi-token kernel; q [B][tokens][Hq][D])
  // Single-token gated kernel only: the units' scores [B][Hkv][NB], already
  // written by the gate's score kernel; the kernel selects from them instead
  // of scoring the pooled table (and leaves `scores` as it is).  nullptr: score.
  const double* scores_in;
};

struct CombineArgs {
  int32_t B, Hq, Hkv, D, S;
  int32_t tokens;  // multi-token combine: query tokens per sequence
  int32_t per_head;  // single-token combine: one workgroup per query head (else per unit)
  const int32_t* hdr;
  const int32_t* prefix;
  const float* part;
  float* out;
  float* lse;
};

// Workspace layout: [hdr: 64 bytes][prefix: (U+1) int32, padded to 256][part].
size_t decode_workspace_bytes(int B, int Hkv, int G, int D, int wmax);
size_t decode_part_offset(int U);

// The allocation-free decode call's workspace: a static device array of
// kStaticScratchBytes per GPU.  Returns its address on the current device
// (looked up once per device), or nullptr with *err set.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
void* decode_static_scratch(hipError_t* err);

// Number of resident waves of the partial kernel on the current device for
// this instantiation (0 if the instantiation does not exist).
int decode_max_waves(int dtype, int D, int G);

hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream);
// The same kernel with the gate and top-k fused in (a.pooled set).
hipError_t launch_gated_decode_partial(const DecodeArgs& a, hipStream_t stream);
// Dynamic LDS bytes the gated kernels need (single- and multi-token: the same
// layout), the ids one workgroup must hold, and the gated kernels' static LDS.
size_t gated_decode_smem_bytes(int U, int NB, int ids_cap);
size_t gated_decode_static_smem(int dtype, int D, int G);
size_t gated_decode_multi_static_smem(int dtype, int D);
int gated_decode_ids_cap(int U, int k_max, int W);
hipError_t launch_decode_combine(const CombineArgs& a, hipStream_t stream);

// Several new query tokens per sequence: G * tokens <= 16 query rows per unit,
// partial records of 16 rows.  Selection given (or dense).
constexpr int kMultiRows = 16;
size_t decode_multi_workspace_bytes(int B, int Hkv, int D, int wmax);
hipError_t launch_decode_multi(const DecodeArgs& a, hipStream_t stream);
// The same with the gate fused in (a.pooled set, as launch_gated_decode_partial).
hipError_t launch_gated_decode_multi(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_multi_combine(const CombineArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- gate

struct GateArgs {
  const void* q;
  const float* pooled;
  const int32_t* lens;
  const int32_t* top_k;  // nullptr: keep rule
  int32_t keep_num, keep_den, k_max;
  int32_t B, Hq, Hkv, D, NB, S, dtype;
  double* scores;
  int32_t* sel_idx;
  int32_t* sel_cnt;
  int32_t threshold_mode;  // keep the blocks scoring above `threshold` (else top-k)
  double threshold;
  int32_t force_first;     // keep block 0 whatever its score
  int32_t force_last;      // keep the newest block whatever its score
  int32_t unified;         // one selection per sequence from the KV heads' summed scores
  int32_t tokens;          // query tokens per sequence, summed into the gate's query (q [B][tokens][Hq][D])
  // Learned gate (launch_learned_gate only): per KV head, w1 int8 [Hkv][256][D]
  // with row scales w1_scale [Hkv][256], b1 [Hkv][256], wq [Hkv][256][D].
  const int8_t* w1;
  const float* w1_scale;
  const float* b1;
  const float* wq;
  // Pooling append fused into the per-unit score kernels (append set): tokens
  // lens_old[b] .. lens[b] - 1 of the cache k (page_table as in PoolArgs) are
  // added to the open block's fp64 sum exactly as launch_pool_keys appends
  // them; the touched blocks' pooled columns (pooled_out, the same table as
  // pooled) and open_sum are rewritten and the scores use the new means.
  int32_t append;
  const int32_t* lens_old;
  const void* k;
  const int32_t* page_table;
  int64_t num_pages;
  float* pooled_out;
  double* open_sum;
};

hipError_t launch_gate_topk(const GateArgs& a, hipStream_t stream);
// The per-chunk score kernel of launch_gate_topk alone (with a.append as
// there), for a table of more than one 256-block chunk and a per-unit rule:
// the scores go to a.scores and the selection is left to the caller.
hipError_t launch_gate_scores(const GateArgs& a, hipStream_t stream);
// Blocks per workgroup of that score kernel.
constexpr int kGateScoreChunk = 256;
// Whether launch_gate_topk can take a.append (per-unit rules; not unified).
bool gate_topk_appends(const GateArgs& a);
// Dynamic LDS of the gate kernel.
size_t gate_smem_bytes(int NB, int k_max);
// The learned gate network's scores, then the same selection rule (not unified).
constexpr int kGateHidden = 256;
hipError_t launch_learned_gate(const GateArgs& a, hipStream_t stream);
// Workgroups the learned gate gives each unit (more than one: the scores go to
// a.scores and a separate selection follows), and that split score launch
// alone (hipErrorInvalidValue when a unit has one workgroup).
int learned_gate_workgroups_per_unit(int U, int NB);
hipError_t launch_learned_gate_scores(const GateArgs& a, hipStream_t stream);
// All LDS (static and dynamic) the learned gate kernel needs, and its dynamic part.
size_t learned_gate_smem_total(int D, int NB);
size_t learned_gate_smem_dynamic(int NB);

// ---------------------------------------------------------------- pooling

struct PoolArgs {
  const void* k;
  const int32_t* page_table;
  int64_t num_pages;
  const int32_t* lens_old;  // nullptr: bulk
  const int32_t* lens_new;
  int32_t B, Hkv, D, NB, S, dtype;
  float* pooled;
  double* open_sum;
};

hipError_t launch_pool_keys(const PoolArgs& a, hipStream_t stream);

}  // namespace seer
