// Block-mean key pooling for gfx950, bulk and incremental.
//
// Keys are summarised per block and the query is not pooled ("SeerAttention-R:
// Sparse Attention Adaptation for Long Reasoning", Abstract and AI Summary).
// The summary of block j is the mean of its valid keys: an fp64 sum in token
// order (the first key, then one add per further key), divided by the token
// count (IEEE fp64 division) and rounded to fp32 (nearest even).  The fp64
// running sum of the last block (open_sum) lets a decode step append one
// token at a time with the same adds in the same order, so the incremental
// table is bit-identical to a rebuild.
//
// Layouts: pooled[((b*Hkv + g)*d + i)*NB + j] (fp32, d-major so the gate can
// read 64 blocks per wave load); open_sum[(b*Hkv + g)*d + i] (fp64).  One
// thread per dimension i; consecutive threads read consecutive elements of a
// key row.
#include "seer_device.h"
#include "seer_kernels.h"

namespace seer {
namespace {

template <typename T>
__device__ __forceinline__ double elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ double elem<uint16_t>(const uint16_t* p, int64_t i) {
  return (double)__uint_as_float((uint32_t)p[i] << 16);
}
template <>
__device__ __forceinline__ double elem<float>(const float* p, int64_t i) {
  return (double)p[i];
}

// Element offset of block j's first row for (b, g), or -1 if the block has no
// page.
__device__ __forceinline__ int64_t block_row0(const PoolArgs& a, int b, int g, int j, int D) {
  if (a.page_table) {
    const int pg = a.page_table[(int64_t)b * a.NB + j];
    if (pg < 0 || pg >= a.num_pages) return -1;
    return ((int64_t)pg * a.Hkv + g) * a.S * D;
  }
  return (((int64_t)b * a.Hkv + g) * a.NB + j) * (int64_t)a.S * D;
}

// grid (NB, U), block D: one workgroup per (unit, block).
template <typename T, int D>
__global__ __launch_bounds__(D) void pool_bulk_kernel(PoolArgs a) {
  const int j = blockIdx.x, u = blockIdx.y, i = threadIdx.x;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int L = a.lens_new[b];
  if (L <= 0) return;
  const int64_t cap = (int64_t)a.NB * a.S;
  const int Lc = (int)(L > cap ? cap : L);
  const int n = (Lc + a.S - 1) / a.S;
  if (j >= n) return;
  const int nv = min(a.S, Lc - j * a.S);
  const int64_t r0 = block_row0(a, b, g, j, D);
  if (r0 < 0) return;
  const T* kp = (const T*)a.k + r0 + i;
  double acc = elem<T>(kp, 0);
  for (int t = 1; t < nv; ++t) acc += elem<T>(kp, (int64_t)t * D);
  a.pooled[((int64_t)u * D + i) * a.NB + j] = (float)(acc / (double)nv);
  if (j == n - 1) a.open_sum[(int64_t)u * D + i] = acc;
}

// grid (U), block D: appends tokens lens_old[b] .. lens_new[b]-1 in order.
template <typename T, int D>
__global__ __launch_bounds__(D) void pool_append_kernel(PoolArgs a) {
  const int u = blockIdx.x, i = threadIdx.x;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int64_t cap = (int64_t)a.NB * a.S;
  // the open sum is requested with the lengths (one round trip for both; the
  // empty asm keeps the compiler from sinking the load past the early return)
  double acc = a.open_sum[(int64_t)u * D + i];
  __asm__ volatile("" ::: "memory");
  const int lo = a.lens_old[b];
  int hi = a.lens_new[b];
  if (hi > cap) hi = (int)cap;
  if (lo < 0 || lo >= hi) return;
  for (int t = lo; t < hi; ++t) {
    const int j = t / a.S, pos = t - j * a.S;
    const int64_t r0 = block_row0(a, b, g, j, D);
    if (r0 < 0) continue;
    const double x = elem<T>((const T*)a.k, r0 + (int64_t)pos * D + i);
    acc = pos == 0 ? x : acc + x;
    if (pos == a.S - 1 || t == hi - 1)
      a.pooled[((int64_t)u * D + i) * a.NB + j] = (float)(acc / (double)(pos + 1));
  }
  a.open_sum[(int64_t)u * D + i] = acc;
}

template <typename T, int D>
hipError_t launch_typed(const PoolArgs& a, hipStream_t stream) {
  PoolArgs args = a;
  void* params[] = {&args};
  const int U = a.B * a.Hkv;
  if (a.lens_old == nullptr)
    return hipLaunchKernel((const void*)&pool_bulk_kernel<T, D>, dim3(a.NB, U), dim3(D), params,
                           0, stream);
  return hipLaunchKernel((const void*)&pool_append_kernel<T, D>, dim3(U), dim3(D), params, 0,
                         stream);
}

}  // namespace

hipError_t launch_pool_keys(const PoolArgs& a, hipStream_t stream) {
  if (a.dtype == 1) return a.D == 64 ? launch_typed<uint16_t, 64>(a, stream)
                                     : launch_typed<uint16_t, 128>(a, stream);
  return a.D == 64 ? launch_typed<float, 64>(a, stream) : launch_typed<float, 128>(a, stream);
}

}  // namespace seer
