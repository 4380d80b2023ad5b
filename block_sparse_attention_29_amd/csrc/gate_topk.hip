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
// Two kernels:
//  * gate_scores_kernel: one thread per block, grid (block chunks, units).  The
//    pooled table is d-major, so the 64 lanes of a wave read 64 consecutive
//    blocks' entries for one dimension per load (256 contiguous bytes).
//  * topk_kernel: one workgroup per unit.  Exact radix select of the k-th
//    largest order key (8 passes of 8 bits, LDS histogram), then the kept set
//    is {key > tau} plus the lowest-indexed keys equal to tau, compacted in id
//    order with block-wide scans.  Deterministic; no sorting network needed.
#include "seer_device.h"
#include "seer_kernels.h"

namespace seer {
namespace {

constexpr int kGateThreads = 256;

__device__ __forceinline__ int unit_nblocks(int L, int S, int NB) {
  if (L <= 0) return 0;
  const int n = (int)(((int64_t)L + S - 1) / S);
  return n > NB ? NB : n;
}

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

template <typename T, int D>
__global__ __launch_bounds__(kGateThreads) void gate_scores_kernel(GateArgs a) {
  __shared__ double s_q[D];
  const int u = blockIdx.y;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int n = unit_nblocks(a.lens[b], a.S, a.NB);
  const int j0 = blockIdx.x * kGateThreads;
  if (j0 >= n) return;
  const int G = a.Hq / a.Hkv;
  const T* q = (const T*)a.q + ((int64_t)b * a.Hq + (int64_t)g * G) * D;
  for (int i = threadIdx.x; i < D; i += kGateThreads) {
    double s = load_as_double<T>(q, i);
    for (int h = 1; h < G; ++h) s += load_as_double<T>(q, (int64_t)h * D + i);
    s_q[i] = s;
  }
  __syncthreads();
  const int j = j0 + threadIdx.x;
  if (j >= n) return;
  const float* p = a.pooled + (int64_t)u * D * a.NB + j;
  double s = 0.0;
#pragma unroll 16
  for (int i = 0; i < D; ++i) s = fma(s_q[i], (double)p[(int64_t)i * a.NB], s);
  a.scores[(int64_t)u * a.NB + j] = s / sqrt((double)D);
}

__global__ __launch_bounds__(kGateThreads) void topk_kernel(GateArgs a) {
  extern __shared__ uint64_t s_key[];  // [NB]
  __shared__ int s_hist[256];
  __shared__ int s_scan[kGateThreads / 64 + 1];
  __shared__ int s_pick[2];

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int b = u / a.Hkv;
  const int n = unit_nblocks(a.lens[b], a.S, a.NB);
  int32_t* out = a.sel_idx + (int64_t)u * a.k_max;

  int k = 0;
  if (n > 0) {
    if (a.top_k) {
      k = a.top_k[b];
    } else {
      k = (int)(((int64_t)n * a.keep_num + a.keep_den - 1) / a.keep_den);
    }
    k = k < 1 ? 1 : (k > n ? n : k);
    k = k > a.k_max ? a.k_max : k;
  }
  if (k >= n) {  // every block kept (or none when n == 0)
    for (int j = tid; j < a.k_max; j += kGateThreads) out[j] = j < n ? j : -1;
    if (tid == 0) a.sel_cnt[u] = n;
    return;
  }

  const double* sc = a.scores + (int64_t)u * a.NB;
  for (int j = tid; j < n; j += kGateThreads) s_key[j] = order_key(sc[j]);
  __syncthreads();

  // Radix select of tau, the k-th largest key.  Invariant: krem of the keys
  // that match `prefix` on the bits in `mask` belong to the top k.
  uint64_t prefix = 0, mask = 0;
  int krem = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    s_hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += kGateThreads) {
      const uint64_t key = s_key[j];
      if ((key & mask) == prefix) atomicAdd(&s_hist[(int)((key >> shift) & 255)], 1);
    }
    __syncthreads();
    // Digit dv with (#keys of larger digit) < krem <= (#keys of digit >= dv).
    const int digit = 255 - tid;
    const int c = s_hist[digit];
    int tot;
    const int larger = block_excl_scan<kGateThreads>(c, s_scan, &tot);
    if (larger < krem && krem <= larger + c) {
      s_pick[0] = digit;
      s_pick[1] = krem - larger;
    }
    __syncthreads();
    prefix |= (uint64_t)s_pick[0] << shift;
    mask |= (uint64_t)255 << shift;
    krem = s_pick[1];
    __syncthreads();
  }
  const uint64_t tau = prefix;

  // Keep every key > tau and the first krem keys == tau in id order; emit ids
  // in ascending order.  Thread t owns the contiguous ids [lo, hi).
  const int per = (n + kGateThreads - 1) / kGateThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int eq = 0;
  for (int j = lo; j < hi; ++j) eq += s_key[j] == tau;
  int tot;
  const int eq_base = block_excl_scan<kGateThreads>(eq, s_scan, &tot);
  int kept = 0;
  {
    int er = eq_base;
    for (int j = lo; j < hi; ++j) {
      const uint64_t key = s_key[j];
      const bool is_eq = key == tau;
      kept += (key > tau) || (is_eq && er < krem);
      er += is_eq;
    }
  }
  int pos = block_excl_scan<kGateThreads>(kept, s_scan, &tot);
  {
    int er = eq_base;
    for (int j = lo; j < hi; ++j) {
      const uint64_t key = s_key[j];
      const bool is_eq = key == tau;
      if ((key > tau) || (is_eq && er < krem)) out[pos++] = j;
      er += is_eq;
    }
  }
  for (int j = k + tid; j < a.k_max; j += kGateThreads) out[j] = -1;
  if (tid == 0) a.sel_cnt[u] = k;
}

}  // namespace

hipError_t launch_gate_topk(const GateArgs& a, hipStream_t stream) {
  const int U = a.B * a.Hkv;
  GateArgs args = a;
  void* params[] = {&args};
  const void* fn = nullptr;
  if (a.dtype == 1) fn = a.D == 64 ? (const void*)&gate_scores_kernel<uint16_t, 64>
                                   : (const void*)&gate_scores_kernel<uint16_t, 128>;
  else fn = a.D == 64 ? (const void*)&gate_scores_kernel<float, 64>
                      : (const void*)&gate_scores_kernel<float, 128>;
  const dim3 grid1((a.NB + kGateThreads - 1) / kGateThreads, U);
  hipError_t e = hipLaunchKernel(fn, grid1, dim3(kGateThreads), params, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)&topk_kernel, dim3(U), dim3(kGateThreads), params,
                         (size_t)a.NB * sizeof(uint64_t), stream);
}

}  // namespace seer
