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

// One workgroup per selection -- a unit (sequence b, KV head g), or a whole
// sequence when the selection is unified over its KV heads: scores for all
// blocks, then the selection.
//
// Scores (all 16 waves): block j's dot product with the group-summed query is
// split over 4 thread quarters of D/4 dimensions each (each a sequential fp64
// FMA chain whose loads are all issued up front), and the 4 partial sums are
// added in a fixed order, so equal blocks get bit-identical scores.  The
// pooled loads of the first 256 blocks are issued before the query loads, so
// the two round trips overlap.  Unified: the KV heads' dot products are added
// in head order (fp64) before the 1/sqrt(D) scaling.
//
// Selection (the rule of select_device.h): forced blocks get a key above every
// score; the count is the top-k count (raised to the forced blocks), or the
// number of keys above the threshold's key; then block_topk_ids (an exact radix
// select by the whole workgroup).  The scores written out are the blocks' own.
template <typename T, int D, bool UNIFIED>
__global__ __launch_bounds__(kTopkThreads) void gate_topk_kernel(GateArgs a) {
  constexpr int DQ = D / 4;  // dimensions per quarter
  extern __shared__ uint64_t s_key[];  // [NB] keys (unified: fp64 sums first), then [k_max] ids
  __shared__ double s_q[D];
  __shared__ double s_part[4][256];
  __shared__ int s_hist[3][256];
  __shared__ int s_scan[kTopkThreads / 64 + 1];

  const int tid = threadIdx.x;
  const int b = UNIFIED ? (int)blockIdx.x : (int)blockIdx.x / a.Hkv;
  const int g_lo = UNIFIED ? 0 : (int)blockIdx.x - b * a.Hkv;
  const int g_hi = UNIFIED ? a.Hkv : g_lo + 1;
  const int n = seq_blocks(a.lens[b], a.S, a.NB);
  const int G = a.Hq / a.Hkv;
  const int jl = tid & 255, qd = tid >> 8;
  int32_t* s_ids = (int32_t*)(s_key + a.NB);
  double* s_acc = (double*)s_key;  // unified: running fp64 sums over the KV heads
  const double inv = 1.0 / sqrt((double)D);

  for (int g = g_lo; g < g_hi; ++g) {
    const int u = b * a.Hkv + g;
    // ---- pooled loads of the first 256 blocks (clamped ids, always in bounds) ----
    const float* pu = a.pooled + (int64_t)u * D * a.NB;
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
      double sq = x[0];
#pragma unroll
      for (int h = 1; h < 8; ++h) sq = h < G ? sq + x[h] : sq;
      s_q[i] = sq;
    }
    __syncthreads();

    // ---- dot products, 256 blocks at a time ----
    auto score_chunk = [&](int j0) {
      const int j = j0 + jl;
      double sp = 0.0;
#pragma unroll
      for (int i = 0; i < DQ; ++i) sp = fma(s_q[qd * DQ + i], (double)pv[i], sp);
      s_part[qd][jl] = sp;
      __syncthreads();
      if (qd == 0 && j < n) {
        const double dot = ((s_part[0][jl] + s_part[1][jl]) + s_part[2][jl]) + s_part[3][jl];
        if constexpr (UNIFIED) s_acc[j] = g == 0 ? dot : s_acc[j] + dot;
        else s_key[j] = order_key(dot * inv);
      }
      __syncthreads();
    };
    if (n > 0) score_chunk(0);
    for (int j0 = 256; j0 < n; j0 += 256) {
      load_pooled(j0 + jl);
      __builtin_amdgcn_sched_barrier(0);
      score_chunk(j0);
    }
  }
  if constexpr (UNIFIED) {
    for (int j = tid; j < n; j += kTopkThreads) s_key[j] = order_key(s_acc[j] * inv);
    __syncthreads();
  }

  // ---- forced blocks and the kept count ----
  const int nf = forced_count(n, a.force_first, a.force_last);
  uint64_t key_first = 0, key_last = 0;
  if (nf > 0) {
    key_first = s_key[0];
    key_last = s_key[n - 1];
    __syncthreads();
    if (tid == 0) {
      if (a.force_first) s_key[0] = kForcedKey;
      if (a.force_last) s_key[n - 1] = kForcedKey;
    }
    __syncthreads();
  }
  int k;
  if (a.threshold_mode) {
    const uint64_t kt = order_key(a.threshold);
    int c = 0;
    for (int j = tid; j < n; j += kTopkThreads) c += s_key[j] > kt;
    int total;
    block_excl_scan<kTopkThreads>(c, s_scan, &total);
    const int cap = n < a.k_max ? n : a.k_max;
    k = n > 0 ? max(1, min(total, cap)) : 0;
  } else {
    k = kept_count_forced(n, a.top_k, b, a.keep_num, a.keep_den, a.k_max, nf);
  }

  // ---- selection: into the unit's row, or into LDS and then every row of
  // the sequence when unified ----
  int32_t* row0 = a.sel_idx + (int64_t)(b * a.Hkv + g_lo) * a.k_max;
  int32_t* dst = UNIFIED ? s_ids : row0;
  if (k >= n) {
    for (int j = tid; j < n; j += kTopkThreads) dst[j] = j;
  } else {
    block_topk_ids<kTopkThreads>(s_key, n, k, &s_hist[0][0], s_scan, dst);
  }
  if (nf > 0 || UNIFIED) __syncthreads();
  if (nf > 0) {
    if (tid == 0) {  // the forced blocks' own scores go out
      s_key[0] = key_first;
      s_key[n - 1] = key_last;
    }
    __syncthreads();
  }

  // ---- outputs (the scores last: a pending store holds its data registers,
  // so nothing waits behind it) ----
  for (int g = g_lo; g < g_hi; ++g) {
    const int u = b * a.Hkv + g;
    int32_t* out = a.sel_idx + (int64_t)u * a.k_max;
    if constexpr (UNIFIED) {
      for (int j = tid; j < a.k_max; j += kTopkThreads) out[j] = j < k ? s_ids[j] : -1;
    } else {
      for (int j = k + tid; j < a.k_max; j += kTopkThreads) out[j] = -1;
    }
    if (tid == 0) a.sel_cnt[u] = k;
  }
  for (int g = g_lo; g < g_hi; ++g) {
    double* sc = a.scores + (int64_t)(b * a.Hkv + g) * a.NB;
    for (int j = tid; j < n; j += kTopkThreads) sc[j] = key_score(s_key[j]);
  }
}

}  // namespace

size_t gate_smem_bytes(int NB, int k_max) {
  return (size_t)NB * sizeof(uint64_t) + (size_t)k_max * sizeof(int32_t);
}

hipError_t launch_gate_topk(const GateArgs& a, hipStream_t stream) {
  const int U = a.B * a.Hkv;
  GateArgs args = a;
  void* params[] = {&args};
  const void* fn = nullptr;
  if (a.unified) {
    if (a.dtype == 1) fn = a.D == 64 ? (const void*)&gate_topk_kernel<uint16_t, 64, true>
                                     : (const void*)&gate_topk_kernel<uint16_t, 128, true>;
    else fn = a.D == 64 ? (const void*)&gate_topk_kernel<float, 64, true>
                        : (const void*)&gate_topk_kernel<float, 128, true>;
  } else {
    if (a.dtype == 1) fn = a.D == 64 ? (const void*)&gate_topk_kernel<uint16_t, 64, false>
                                     : (const void*)&gate_topk_kernel<uint16_t, 128, false>;
    else fn = a.D == 64 ? (const void*)&gate_topk_kernel<float, 64, false>
                        : (const void*)&gate_topk_kernel<float, 128, false>;
  }
  const int grid = a.unified ? a.B : U;
  return hipLaunchKernel(fn, dim3(grid), dim3(kTopkThreads), params,
                         gate_smem_bytes(a.NB, a.k_max), stream);
}

}  // namespace seer
