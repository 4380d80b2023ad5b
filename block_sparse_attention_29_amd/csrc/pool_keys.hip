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
#include <type_traits>

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

// Bulk pooling, grid (ceil(NB / BPW), U), 256 threads: workgroup (c, u)
// pools blocks c*BPW .. c*BPW + BPW - 1 of unit u.  LPR lanes cover one key
// row with 16-byte loads (EPL dimensions each), so the workgroup's threads
// split into BPW groups, one block each.  A lane keeps EPL independent fp64
// sums and walks its block's tokens in order, kUnroll rows of loads in flight
// at a time; every sum is still the first key plus one add per further key in
// token order, the arithmetic pool_append_kernel repeats.  The means are
// transposed through LDS so that each dimension's row of the table is written
// as BPW consecutive floats.
constexpr int kPoolThreads = 256;
constexpr int kUnroll = 16;

template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_bulk_kernel(PoolArgs a) {
  constexpr int EPL = 16 / (int)sizeof(T);  // dimensions per lane
  constexpr int LPR = D / EPL;              // lanes per key row
  constexpr int BPW = kPoolThreads / LPR;   // blocks per workgroup
  __shared__ float s_mean[D][BPW + 1];
  __shared__ int s_ok[BPW];  // the block has a page and tokens: its means are written

  const int u = blockIdx.y, tid = threadIdx.x;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int jb = tid / LPR, l = tid - jb * LPR;  // block of the group, lane in the row
  const int j0 = (int)blockIdx.x * BPW, j = j0 + jb;
  const int L = a.lens_new[b];
  const int64_t cap = (int64_t)a.NB * a.S;
  const int Lc = L <= 0 ? 0 : (int)(L > cap ? cap : L);
  const int n = (Lc + a.S - 1) / a.S;  // blocks of the sequence
  if (j0 >= n) return;                 // the whole workgroup
  const int nv = j < n ? min(a.S, Lc - j * a.S) : 0;
  const int64_t r0 = nv > 0 ? block_row0(a, b, g, j, D) : -1;

  double acc[EPL];
  if (r0 >= 0) {
    const char* kp = (const char*)((const T*)a.k + r0) + l * 16;
    // rows t0 .. t0 + kUnroll - 1, those past nv re-reading the last (in
    // bounds, unused), all in flight before the first add
    auto group = [&](int t0, auto tail_tag) {
      constexpr bool TAIL = decltype(tail_tag)::value;
      uint4 raw[kUnroll];
#pragma unroll
      for (int r = 0; r < kUnroll; ++r)
        raw[r] = *(const uint4*)(kp + (int64_t)(TAIL ? min(t0 + r, nv - 1) : t0 + r) * D *
                                          sizeof(T));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < kUnroll; ++r)
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const double x = (double)chunk_elem<T>(raw[r], e);
          const double y = t0 + r == 0 ? x : acc[e] + x;
          acc[e] = (!TAIL || t0 + r < nv) ? y : acc[e];
        }
    };
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0;  // replaced by the first key
    int t0 = 0;
    for (; t0 + kUnroll <= nv; t0 += kUnroll) group(t0, std::bool_constant<false>{});
    if (t0 < nv) group(t0, std::bool_constant<true>{});
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_mean[l * EPL + e][jb] = (float)(acc[e] / (double)nv);
    if (j == n - 1) {
      double* os = a.open_sum + (int64_t)u * D + l * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) os[e] = acc[e];
    }
  }
  if (l == 0) s_ok[jb] = r0 >= 0;
  __syncthreads();
  // each dimension's BPW consecutive entries (a block past the sequence or
  // without a page keeps its table entries)
  for (int x = tid; x < D * BPW; x += kPoolThreads) {
    const int i = x / BPW, jj = x - i * BPW;
    if (s_ok[jj]) a.pooled[((int64_t)u * D + i) * a.NB + j0 + jj] = s_mean[i][jj];
  }
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
  if (a.lens_old == nullptr) {
    constexpr int BPW = kPoolThreads / (D * (int)sizeof(T) / 16);
    return hipLaunchKernel((const void*)&pool_bulk_kernel<T, D>, dim3((a.NB + BPW - 1) / BPW, U),
                           dim3(kPoolThreads), params, 0, stream);
  }
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
