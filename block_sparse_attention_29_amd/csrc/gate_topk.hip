// Gate scores and top-k block selection for gfx950.
//
// For every (sequence b, KV head g) -- one "unit" -- and every block j < n_b:
//   s_j = (sum_{h in group g} q_h) . P_j / sqrt(d)           (fp64)
// where P is the fp32 pooled-key table (block means; keys pooled, query not:
// "SeerAttention-R: Sparse Attention Adaptation for Long Reasoning", Abstract).
// Then the k_b highest-scoring blocks are kept ("Sparse Attention Reasoning",
// Step 1: top-k over the gate's scores), ties to the lower block id, and
// written in ascending id order.
//
// One kernel, one 1024-thread workgroup per unit: the scores (the pooled table
// is d-major, so the 64 lanes of a wave read 64 consecutive blocks' entries
// of one dimension per load, 256 contiguous bytes), then an exact radix select
// of the kept set in LDS, compacted in id order with block-wide scans.
// Deterministic; no sorting network needed.
#include "seer_device.h"
#include "seer_kernels.h"
#include "select_device.h"

namespace seer {
namespace {

constexpr int kTopkThreads = 1024;

template <typename T>
__device__ __forceinline__ double load_as_double(const T* p, int64_t i);

template <>
__device__ __forceinline__ double load_as_double<uint16_t>(const uint16_t* p, int64_t i) {
  return (double)__uint_as_float((uint32_t)p[i] << 16);
}

template <>
__device__ __forceinline__ double load_as_double<float>(const float* p, int64_t i) {
  return (double)p[i];
}

// One workgroup per unit: scores for all blocks, then the selection.
//
// Scores (all 16 waves): block j's dot product is split over 4 thread
// quarters of D/4 dimensions each (each a sequential fp64 FMA chain whose
// loads are all issued up front), and the 4 partial sums are added in a fixed
// order, so equal blocks get bit-identical scores.  The pooled loads of the
// first 256 blocks are issued before the query loads, so the two round trips
// overlap.
//
// Selection: block_topk_ids (an exact radix select by the whole workgroup).
template <typename T, int D>
__global__ __launch_bounds__(kTopkThreads) void gate_topk_kernel(GateArgs a) {
  constexpr int DQ = D / 4;  // dimensions per quarter
  extern __shared__ uint64_t s_key[];  // [NB]
  __shared__ double s_q[D];
  __shared__ double s_part[4][256];
  __shared__ int s_hist[2][256];
  __shared__ int s_pick[3];
  __shared__ int s_scan[kTopkThreads / 64 + 1];

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int n = seq_blocks(a.lens[b], a.S, a.NB);
  const int G = a.Hq / a.Hkv;
  int32_t* out = a.sel_idx + (int64_t)u * a.k_max;

  // ---- pooled loads of the first 256 blocks (clamped ids, always in bounds) ----
  const float* pu = a.pooled + (int64_t)u * D * a.NB;
  const int jl = tid & 255, qd = tid >> 8;
  float pv[DQ];
  auto load_pooled = [&](int j) {
    // Unsigned 32-bit offsets from the unit's (uniform) base; every load is
    // issued before anything waits on the first one.
    uint32_t off = (uint32_t)(qd * DQ * a.NB + (n > 0 ? min(j, n - 1) : 0));
#pragma unroll
    for (int i = 0; i < DQ; ++i, off += (uint32_t)a.NB) pv[i] = pu[off];
  };
  load_pooled(jl);  // unconditional (in bounds even when n == 0)

  // ---- group-summed query, fp64, head order ----
  const T* q = (const T*)a.q + ((int64_t)b * a.Hq + (int64_t)g * G) * D;
  for (int i = tid; i < D; i += kTopkThreads) {
    // All 8 possible heads are loaded (clamped to the group) before summing the
    // first G in head order, so the loads are in flight together.
    double x[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) x[h] = load_as_double<T>(q, (int64_t)min(h, G - 1) * D + i);
    double s = x[0];
#pragma unroll
    for (int h = 1; h < 8; ++h) s = h < G ? s + x[h] : s;
    s_q[i] = s;
  }
  __syncthreads();

  // ---- scores, 256 blocks at a time ----
  const double inv = 1.0 / sqrt((double)D);
  auto score_chunk = [&](int j0) {
    const int j = j0 + jl;
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < DQ; ++i) s = fma(s_q[qd * DQ + i], (double)pv[i], s);
    s_part[qd][jl] = s;
    __syncthreads();
    if (qd == 0 && j < n) {
      const double sc = ((s_part[0][jl] + s_part[1][jl]) + s_part[2][jl]) + s_part[3][jl];
      s_key[j] = order_key(sc * inv);
    }
    __syncthreads();
  };
  if (n > 0) score_chunk(0);
  for (int j0 = 256; j0 < n; j0 += 256) {
    load_pooled(j0 + jl);
    __builtin_amdgcn_sched_barrier(0);
    score_chunk(j0);
  }

  const int k = kept_count(n, a.top_k, b, a.keep_num, a.keep_den, a.k_max);
  // The scores go out last (rebuilt from the order keys): a pending store
  // would hold its data registers and stall the selection behind it.
  auto write_scores = [&](int j0, int stride) {
    double* sc = a.scores + (int64_t)u * a.NB;
    for (int j = j0; j < n; j += stride) sc[j] = key_score(s_key[j]);
  };
  if (k >= n) {  // every block kept (or none when n == 0)
    for (int j = tid; j < a.k_max; j += kTopkThreads) out[j] = j < n ? j : -1;
    if (tid == 0) a.sel_cnt[u] = n;
    write_scores(tid, kTopkThreads);
    return;
  }

  block_topk_ids<kTopkThreads>(s_key, n, k, &s_hist[0][0], s_pick, s_scan, out);
  for (int j = k + tid; j < a.k_max; j += kTopkThreads) out[j] = -1;
  if (tid == 0) a.sel_cnt[u] = k;
  write_scores(tid, kTopkThreads);
}

}  // namespace

hipError_t launch_gate_topk(const GateArgs& a, hipStream_t stream) {
  const int U = a.B * a.Hkv;
  GateArgs args = a;
  void* params[] = {&args};
  const void* fn = nullptr;
  if (a.dtype == 1) fn = a.D == 64 ? (const void*)&gate_topk_kernel<uint16_t, 64>
                                   : (const void*)&gate_topk_kernel<uint16_t, 128>;
  else fn = a.D == 64 ? (const void*)&gate_topk_kernel<float, 64>
                      : (const void*)&gate_topk_kernel<float, 128>;
  return hipLaunchKernel(fn, dim3(U), dim3(kTopkThreads), params,
                         (size_t)a.NB * sizeof(uint64_t), stream);
}

}  // namespace seer
