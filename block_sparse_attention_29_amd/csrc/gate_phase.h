// The gate phase of the decode kernels with the gate fused in: each
// workgroup scores and selects the blocks of the units it streams itself
// (included by sparse_decode.hip and multi_decode.hip; the arithmetic is the
// gate kernel's, so the selections are bit-identical to it).
#pragma once

#include "decode_common.h"
#include "select_device.h"

namespace seer {
namespace {

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// The value a unit's block count needs besides its length: the explicit kept
// count top_k[b] (fused gate) or the given selection's count sel_cnt[u].
template <bool GATED>
__device__ __forceinline__ int unit_aux(const DecodeArgs& a, int u) {
  if constexpr (GATED) return a.top_k ? a.top_k[u / a.Hkv] : 0;
  return a.sel_idx ? a.sel_cnt[u] : 0;
}

// Blocks a unit contributes: its kept count (given, or from the keep rule when
// the gate is fused in), or all its blocks when dense.
// L: the unit's sequence length; aux: unit_aux of the unit.
template <bool GATED>
__device__ __forceinline__ int unit_blocks(const DecodeArgs& a, int L, int aux) {
  if constexpr (GATED) {
    const int n = seq_blocks(L, a.S, a.NB);
    return kept_count_forced_of(n, a.top_k != nullptr, aux, a.keep_num, a.keep_den, a.k_max,
                                forced_count(n, a.force_first, a.force_last));
  }
  if (a.sel_idx) return aux < 0 ? 0 : (aux > a.k_max ? a.k_max : aux);
  return seq_blocks(L, a.S, a.NB);
}

// The query rows the gate sums for unit (b, g): the G heads of its group, or
// with several new tokens (MULTI: G and the token count T read at run time,
// QR = 16 rows at most) the G heads of each token, row r = t * G + h.  Rows
// past the unit's count are clamped to its last row (in bounds, unused).
template <int QR, bool MULTI>
__device__ __forceinline__ int gate_rows(const DecodeArgs& a) {
  if constexpr (MULTI) return (a.Hq / a.Hkv) * a.tokens;
  return QR;
}

template <typename T, int D, int QR, bool MULTI>
__device__ __forceinline__ const T* gate_q_row(const DecodeArgs& a, int b, int g, int r) {
  if constexpr (!MULTI) return (const T*)a.q + ((int64_t)b * a.Hq + (int64_t)g * QR + r) * D;
  const int G = a.Hq / a.Hkv, R = G * a.tokens;
  const int rr = min(r, R - 1), t = rr / G, h = rr - t * G;
  return (const T*)a.q + (((int64_t)b * a.tokens + t) * a.Hq + (int64_t)g * G + h) * D;
}

// The first gate pass's pooled-table and query loads of one unit, issued at
// kernel entry, before the plan says which unit the workgroup gates: u is the
// unit it gates first when every unit keeps as many blocks as any other (the
// plan then confirms it; otherwise the values go unused).  Lane (qd, jq) holds
// dimensions qd*D/4 .. of blocks 4jq .. 4jq+3, as fused_scores loads them.
template <typename T, int D, int QR>
struct GatePreload {
  int u;
  float pv[D / 4][4];
  T qr[QR];
  // With scores given (a.scores_in): unit u's scores tid + 256 e instead
  // (sx_ok says they were loaded).
  double sx[8];
  bool sx_ok;
};

// The first unit's given scores, requested at kernel entry (scores_in set;
// u as in issue_gate_preload).  Ids past the table are clamped into the unit's
// row (read, unused).
__device__ __forceinline__ void issue_score_preload_into(const DecodeArgs& a, int u, int& pu,
                                                         double (&sx)[8], bool& ok) {
  const double* sc = a.scores_in + (int64_t)u * a.NB;
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < 8; ++e) sx[e] = sc[min(tid + e * kThreads, a.NB - 1)];
  pu = u;
  ok = true;
}

template <typename T, int D, int QR, bool MULTI, bool GIVEN = false>
__device__ __forceinline__ void issue_gate_preload(const DecodeArgs& a, int u,
                                                   GatePreload<T, D, QR>& pre) {
  pre.sx_ok = false;
  if constexpr (GIVEN) {  // the scores are given (a.scores_in): load those instead
    issue_score_preload_into(a, u, pre.u, pre.sx, pre.sx_ok);
    return;
  }
  constexpr int DQ = D / 4;
  const int tid = threadIdx.x, qd = tid >> 6, jq = tid & 63;
  const int NB = a.NB;
  pre.u = u;
  // Aligned 16-byte loads need NB % 4 == 0; otherwise every lane re-reads the
  // table's first 16 bytes (in bounds, unused) and the gate loads for itself.
  const bool vec4 = NB % 4 == 0;
  const float* row = vec4 ? a.pooled + ((int64_t)u * D + qd * DQ) * NB + min(4 * jq, NB - 4)
                          : a.pooled;
  const int64_t step = vec4 ? NB : 0;
#pragma unroll
  for (int i = 0; i < DQ; ++i) {
    const float4 v = *(const float4*)(row + i * step);
    pre.pv[i][0] = v.x; pre.pv[i][1] = v.y; pre.pv[i][2] = v.z; pre.pv[i][3] = v.w;
  }
  const int b = u / a.Hkv, g = u - b * a.Hkv;
#pragma unroll
  for (int r = 0; r < QR; ++r) pre.qr[r] = gate_q_row<T, D, QR, MULTI>(a, b, g, r)[min(tid, D - 1)];
}

// VEC consecutive pooled values of one dimension row (one 4*VEC-byte load).
template <int VEC>
__device__ __forceinline__ void load_pooled_vec(const float* p, float (&x)[VEC]) {
  if constexpr (VEC == 4) {
    const float4 v = *(const float4*)p;
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else if constexpr (VEC == 2) {
    const float2 v = *(const float2*)p;
    x[0] = v.x; x[1] = v.y;
  } else {
    x[0] = *p;
  }
}

// Scores of unit (b, g)'s n blocks into s_key (order keys), VEC blocks per
// lane per load: wave qd of the workgroup sums the dimensions qd*D/4 ..
// qd*D/4 + D/4 - 1 of 64*VEC blocks per pass (one sequential fp64 FMA chain
// per block), and the four partial sums of a block are added in quarter order
// through LDS:
//   s_j = (((c0 + c1) + c2) + c3) / sqrt(D),  c_q = sum_i qbar_i P_ij over quarter q,
// qbar = sum of the unit's query rows in row order (fp64; the group's heads,
// token-major with several tokens): the same arithmetic as the gate kernel.  The first pass's pooled loads go out before
// the query's, so both round trips overlap.  VEC consecutive blocks are one
// aligned load when NB is a multiple of VEC (no load crosses the table's end).
// With PRE and use_pre the first pass takes its pooled and query values from
// `pre` (VEC = 4 only), loaded at kernel entry.
template <typename T, int D, int QR, bool MULTI, int VEC, bool PRE>
__device__ __forceinline__ void fused_scores(const DecodeArgs& a, int b, int g, const float* pu,
                                             int n, double* s_q, double* s_part,
                                             uint64_t* s_key, int* s_hist,
                                             const GatePreload<T, D, QR>& pre, bool use_pre) {
  constexpr int DQ = D / 4, PASS = 64 * VEC;
  const int NB = a.NB;
  const int tid = threadIdx.x, qd = tid >> 6, jq = tid & 63;
  const double inv = 1.0 / sqrt((double)D);
  // the fold of the keys this thread writes, for the selection
  KeyFold kf;
  // One pass over blocks j0 .. j0 + PASS - 1; the first (FIRST) also sums the
  // query and may take the entry loads (peeled, so that they are dead after).
  auto pass = [&](int j0, auto first_tag) {
    constexpr bool FIRST = decltype(first_tag)::value;
    // block ids past n are clamped to a valid, aligned group (read, unused)
    const int jg = min(j0 + VEC * jq, ((n - 1) / VEC) * VEC);
    float pv[DQ][VEC];
    const float* row = pu + (int64_t)qd * DQ * NB + jg;
    bool from_pre = false;
    if constexpr (FIRST && PRE && VEC == 4) from_pre = use_pre;
    if (from_pre) {
#pragma unroll
      for (int i = 0; i < DQ; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) pv[i][e] = pre.pv[i][e & 3];
    } else {
#pragma unroll
      for (int i = 0; i < DQ; ++i) load_pooled_vec<VEC>(row + (int64_t)i * NB, pv[i]);
    }
    if constexpr (FIRST) {
      if (tid < D) {
        const int R = gate_rows<QR, MULTI>(a);
        double x[QR];
#pragma unroll
        for (int r = 0; r < QR; ++r) {
          T qv;
          if constexpr (PRE) qv = use_pre ? pre.qr[r] : gate_q_row<T, D, QR, MULTI>(a, b, g, r)[tid];
          else qv = gate_q_row<T, D, QR, MULTI>(a, b, g, r)[tid];
          if constexpr (sizeof(T) == 2) x[r] = (double)__uint_as_float((uint32_t)qv << 16);
          else x[r] = (double)qv;
        }
        double sq = x[0];
#pragma unroll
        for (int r = 1; r < QR; ++r) sq = r < R ? sq + x[r] : sq;
        s_q[tid] = sq;
      }
      __syncthreads();
    }
    // every load is in flight before the chains; values widen only where used
    __builtin_amdgcn_sched_barrier(0);
    double c[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) c[e] = 0.0;
#pragma unroll
    for (int i = 0; i < DQ; ++i)
#pragma unroll
      for (int e = 0; e < VEC; ++e) c[e] = fma(s_q[qd * DQ + i], (double)pv[i][e], c[e]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) s_part[qd * PASS + VEC * jq + e] = c[e];
    __syncthreads();
    for (int t = tid; t < PASS; t += kThreads) {
      const int j = j0 + t;
      if (j < n) {
        const double sc = ((s_part[t] + s_part[PASS + t]) + s_part[2 * PASS + t]) +
                          s_part[3 * PASS + t];
        const uint64_t key = order_key(sc * inv);
        s_key[j] = key;
        kf.add(key);
      }
    }
    // the last pass hands the keys' fold to the selection (behind this
    // barrier; topk_keys_collect reads it)
    if (j0 + PASS >= n) topk_keys_publish<kThreads>(kf, s_hist);
    __syncthreads();
  };
  pass(0, BoolTag<true>{});  // n >= 1
  for (int j0 = PASS; j0 < n; j0 += PASS) pass(j0, BoolTag<false>{});
}

// The order keys of unit u's n given scores (a.scores_in, as the gate's score
// kernel wrote them) into s_key, their fold published for the selection
// like fused_scores does; ends with a barrier.  The first 8 * kThreads come
// from the entry loads when those are this unit's.
template <typename T, int D, int QR, bool PRE>
__device__ __forceinline__ void given_score_keys(const DecodeArgs& a, int u, int n,
                                                 uint64_t* s_key, int* s_hist,
                                                 const GatePreload<T, D, QR>& pre, bool use_pre) {
  const int tid = threadIdx.x;
  const double* sc = a.scores_in + (int64_t)u * a.NB;
  double x[8];
  bool from_pre = false;
  if constexpr (PRE) from_pre = use_pre;  // (peeled: the entry loads are dead after)
  if (from_pre) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = pre.sx[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sc[min(tid + e * kThreads, n - 1)];
  }
  KeyFold kf;
  auto put = [&](int j, double v) {
    const uint64_t key = order_key(v);
    s_key[j] = key;
    kf.add(key);
  };
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (tid + e * kThreads < n) put(tid + e * kThreads, x[e]);
  for (int j0 = tid + 8 * kThreads; j0 < n; j0 += 8 * kThreads) {  // longer tables
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sc[min(j0 + e * kThreads, n - 1)];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (j0 + e * kThreads < n) put(j0 + e * kThreads, x[e]);
  }
  topk_keys_publish<kThreads>(kf, s_hist);
  __syncthreads();
}

// The selection outputs of unit u from LDS: its k kept ids (dst, then -1 up to
// k_max), its count and (unless GIVEN: they came from a.scores_in) the scores
// of its n blocks (s_key).  Thread-strided, no barrier: the LDS values must
// have been final before a barrier every thread has passed.
template <bool GIVEN = false>
__device__ __forceinline__ void fused_gate_write(const DecodeArgs& a, int u, int n, int k,
                                                 const int32_t* dst, const uint64_t* s_key) {
  const int tid = threadIdx.x;
  int32_t* ids = a.sel_idx_out + (int64_t)u * a.k_max;
  for (int i = tid; i < a.k_max; i += kThreads) ids[i] = i < k ? dst[i] : -1;
  if (tid == 0) a.sel_cnt_out[u] = k;
  if constexpr (GIVEN) return;  // the given scores are already the output
  double* sc = a.scores + (int64_t)u * a.NB;
  for (int j = tid; j < n; j += kThreads) sc[j] = key_score(s_key[j]);
}

// Gate of unit u inside a decode workgroup (the fused mode): the fp64 scores
// of its n blocks (fused_scores), then its k kept ids, ascending, into dst
// (LDS).  With `owner` the workgroup also writes the scores, ids and count out
// (fused_gate_write); a caller may instead write them later from the same LDS.
template <typename T, int D, int QR, bool MULTI, bool PRE, bool GIVEN = false>
__device__ __forceinline__ void fused_gate_unit(const DecodeArgs& a, int u, int n, int k,
                                                int32_t* dst,
                                                bool owner, uint64_t* s_key, double* s_q,
                                                double* s_part, int* s_hist,
                                                int* s_scan, const GatePreload<T, D, QR>& pre) {
  const int tid = threadIdx.x;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int NB = a.NB;
  const float* pu = a.pooled + (int64_t)u * D * NB;
  const bool use_pre = u == pre.u;  // the entry loads are this unit's (uniform)
  if constexpr (GIVEN)  // scores given by the gate's score kernel
    given_score_keys<T, D, QR, PRE>(a, u, n, s_key, s_hist, pre, use_pre && pre.sx_ok);
  else if (NB % 4 == 0)
    fused_scores<T, D, QR, MULTI, 4, PRE>(a, b, g, pu, n, s_q, s_part, s_key, s_hist, pre,
                                            use_pre);
  else if (NB % 2 == 0)
    fused_scores<T, D, QR, MULTI, 2, PRE>(a, b, g, pu, n, s_q, s_part, s_key, s_hist, pre,
                                            use_pre);
  else
    fused_scores<T, D, QR, MULTI, 1, PRE>(a, b, g, pu, n, s_q, s_part, s_key, s_hist, pre,
                                            use_pre);
  // forced blocks rank above every score while the selection runs
  const bool forced = a.force_first || a.force_last;  // uniform
  uint64_t key_first = 0, key_last = 0;
  if (forced) {
    key_first = s_key[0];
    key_last = s_key[n - 1];
    __syncthreads();
    if (tid == 0) {
      if (a.force_first) s_key[0] = kForcedKey;
      if (a.force_last) s_key[n - 1] = kForcedKey;
    }
    __syncthreads();
  }
  if (k >= n) {
    for (int i = tid; i < n; i += kThreads) dst[i] = i;
  } else if (!forced) {  // the keys' fold came with the scores
    block_topk_ids_from<kThreads>(s_key, n, k, topk_keys_collect<kThreads>(s_hist), s_hist,
                                  s_scan, dst);
  } else {
    block_topk_ids<kThreads>(s_key, n, k, s_hist, s_scan, dst);
  }
  __syncthreads();
  if (forced) {
    if (tid == 0) {  // the forced blocks' own scores go out
      s_key[0] = key_first;
      s_key[n - 1] = key_last;
    }
    __syncthreads();
  }
  if (owner) fused_gate_write<GIVEN>(a, u, n, k, dst, s_key);
  __syncthreads();  // s_key, s_q and s_part are reused by the next unit
}

}  // namespace
}  // namespace seer
