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

namespace seer {
namespace {

constexpr int kTopkThreads = 1024;

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

// One workgroup per unit: scores for all blocks, then the selection.
//
// Scores (all 16 waves): block j's dot product is split over 4 thread
// quarters of D/4 dimensions each (each a sequential fp64 FMA chain whose
// loads are all issued up front), and the 4 partial sums are added in a fixed
// order, so equal blocks get bit-identical scores.  The pooled loads of the
// first 256 blocks are issued before the query loads, so the two round trips
// overlap.
//
// Selection: exact radix select over 64-bit order keys (-0 folded into +0),
// 8 bits per pass from the top, by the whole workgroup with an LDS histogram.
// After a pass only the keys matching the chosen prefix remain candidates;
// once all of them are needed (or all 64 bits are used) the kept set is every
// key with a larger prefix plus the first `krem` matching keys in id order,
// which is the top k by (score desc, id asc).  Random scores usually settle
// after 3 passes.
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
  const int tid = threadIdx.x, lane = tid & 63;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int n = unit_nblocks(a.lens[b], a.S, a.NB);
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

  // ---- kept count ----
  int k = 0;
  if (n > 0) {
    k = a.top_k ? a.top_k[b] : (int)(((int64_t)n * a.keep_num + a.keep_den - 1) / a.keep_den);
    k = k < 1 ? 1 : (k > n ? n : k);
    k = k > a.k_max ? a.k_max : k;
  }
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

  // ---- block radix select ----
  // Thread t owns the contiguous ids [t*m, t*m + m).  Each pass histograms
  // the next 8 bits of the candidates' keys (double-buffered LDS histogram,
  // the next one cleared during the current pass), wave 0 scans the 256 bins
  // from the top and publishes the digit that holds the krem-th largest key.
  const int m = (n + kTopkThreads - 1) / kTopkThreads;
  const int lo = min(n, tid * m), hi = min(n, lo + m);
  uint64_t prefix = 0, mask = 0;
  int krem = k;
  if (tid < 256) s_hist[0][tid] = 0;
  __syncthreads();
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    int* hist = s_hist[pass & 1];
    for (int j = lo; j < hi; ++j) {
      const uint64_t key = s_key[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(int)((key >> shift) & 255)], 1);
    }
    if (tid < 256) s_hist[(pass & 1) ^ 1][tid] = 0;
    __syncthreads();
    if (tid < 64) {
      // lane l holds digits 255-4l .. 252-4l (descending)
      int c[4], sum = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) { c[r] = hist[255 - 4 * lane - r]; sum += c[r]; }
      int larger = wave_incl_scan(sum) - sum;  // keys with a larger digit than this lane's first
      int pick = -1, nk = 0, pc = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (larger < krem && krem <= larger + c[r]) {
          pick = 255 - 4 * lane - r;
          nk = krem - larger;
          pc = c[r];
        }
        larger += c[r];
      }
      // exactly one lane picked: it publishes its digit, new krem and count
      if (pick >= 0) {
        s_pick[0] = pick;
        s_pick[1] = nk;
        s_pick[2] = pc;
      }
    }
    __syncthreads();
    const int dv = s_pick[0], cnt = s_pick[2];
    krem = s_pick[1];
    prefix |= (uint64_t)dv << shift;
    mask |= (uint64_t)255 << shift;
    if (cnt == krem) break;  // every remaining candidate is kept
  }

  // ---- kept ids in id order: every key above the prefix, then the first
  // krem keys equal to it.  One block scan of packed (above, equal) counts
  // gives each thread the counts before its first id. ----
  int gt = 0, eq = 0;
  for (int j = lo; j < hi; ++j) {
    const uint64_t mk = s_key[j] & mask;
    gt += mk > prefix;
    eq += mk == prefix;
  }
  int total;
  const int packed = block_excl_scan<kTopkThreads>(gt | (eq << 16), s_scan, &total);
  int gb = packed & 0xFFFF, eb = packed >> 16;
  for (int j = lo; j < hi; ++j) {
    const uint64_t mk = s_key[j] & mask;
    // (positions are < k by construction; the checks keep every store inside
    // this unit's row whatever the keys hold)
    if (mk > prefix) {
      const int pos = gb + min(eb, krem);
      if (pos < k) out[pos] = j;
      ++gb;
    } else if (mk == prefix) {
      if (eb < krem && gb + eb < k) out[gb + eb] = j;
      ++eb;
    }
  }
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
