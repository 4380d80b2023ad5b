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
// Per-unit selections: the scores by 256-thread workgroups over chunks of 256
// blocks (the pooled table is d-major, so a wave's lanes read consecutive
// blocks of one dimension row), then an exact radix select of the kept set in
// LDS, compacted in id order with block-wide scans -- in one launch, one
// workgroup per unit, when a table is one chunk, else a score launch over
// (unit, chunk) and a select launch per unit.  A selection unified over a sequence's KV heads takes one
// 1024-thread workgroup per sequence for both.  Deterministic; no sorting
// network needed.
#include "seer_device.h"
#include "seer_kernels.h"
#include "select_device.h"

namespace seer {
namespace {

constexpr int kTopkThreads = 1024;

// Largest n that wave_topk_ids takes (16 keys per lane).
constexpr int kWaveSelectMax = 1024;

// LDS operations of one wave complete in issue order; this keeps the compiler
// from moving them across the point (no workgroup barrier involved).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// AND (AND_ = true) or OR of a 32-bit value over the 64 lanes, in every lane.
template <bool AND_>
__device__ __forceinline__ uint32_t wave_bits(uint32_t x) {
  auto op = [](uint32_t p, uint32_t q) { return AND_ ? (p & q) : (p | q); };
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppQuadXor1, 0xF, 0xF, true));
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppQuadXor2, 0xF, 0xF, true));
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowHalfMirror, 0xF, 0xF, true));
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowMirror, 0xF, 0xF, true));
  return op(op((uint32_t)readlane_i((int)x, 0), (uint32_t)readlane_i((int)x, 16)),
            op((uint32_t)readlane_i((int)x, 32), (uint32_t)readlane_i((int)x, 48)));
}

// The selection of block_topk_ids (select_device.h) by one wave, for n <= kWaveSelectMax:
// the ids of the k largest keys of s_key[0..n) (ties to the lower id),
// ascending, to out[0..k).  Requires 0 < k < n.  Called by the 64 lanes of
// one wave only -- no workgroup barrier, so the other waves of the workgroup
// need not take part; s_hist: 256 ints of LDS this wave alone uses.  Lane l
// owns the contiguous ids [l*m, l*m + m); each 8-bit pass histograms the
// digit of the keys still matching the chosen prefix with LDS atomics, and a
// wave scan of the bins from the top finds the digit holding the krem-th
// largest key.  The kept set and its order are unique, so the output is the
// workgroup version's bit for bit.
__device__ void wave_topk_ids(const uint64_t* s_key, int n, int k, int* s_hist, int32_t* out) {
  const int lane = threadIdx.x & 63;
  const int m = (n + 63) / 64;
  const int lo = min(n, lane * m), hi = min(n, lo + m);

  uint64_t kand = ~0ull, kor = 0;
  for (int j = lo; j < hi; ++j) {
    const uint64_t key = s_key[j];
    kand &= key;
    kor |= key;
  }
  kand = ((uint64_t)wave_bits<true>((uint32_t)(kand >> 32)) << 32) | wave_bits<true>((uint32_t)kand);
  kor = ((uint64_t)wave_bits<false>((uint32_t)(kor >> 32)) << 32) | wave_bits<false>((uint32_t)kor);
  const uint64_t diff = kand ^ kor;

  int top = diff ? 63 - __builtin_clzll(diff) : -1;  // highest bit where keys differ
  uint64_t mask = top >= 63 ? 0ull : (~0ull << (top + 1));
  uint64_t prefix = kand & mask;
  int krem = k;
  while (top >= 0) {
    const int shift = top > 7 ? top - 7 : 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) s_hist[4 * lane + r] = 0;
    wave_lds_sync();
    for (int j = lo; j < hi; ++j) {
      const uint64_t key = s_key[j];
      if ((key & mask) == prefix) atomicAdd(&s_hist[(int)((key >> shift) & 255)], 1);
    }
    wave_lds_sync();
    // lane l holds digits 255-4l .. 252-4l (descending)
    int c[4], sum = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) { c[r] = s_hist[255 - 4 * lane - r]; sum += c[r]; }
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
    const int src = __builtin_ctzll(__ballot(pick >= 0));  // exactly one lane picked
    const int dv = readlane_i(pick, src), cnt = readlane_i(pc, src);
    krem = readlane_i(nk, src);
    prefix |= (uint64_t)dv << shift;
    mask |= (uint64_t)255 << shift;
    if (cnt == krem) break;  // every remaining candidate is kept
    top = shift - 1;
    wave_lds_sync();  // every lane has read the bins before the next pass clears them
  }

  int gt = 0, eq = 0;
  for (int j = lo; j < hi; ++j) {
    const uint64_t mk = s_key[j] & mask;
    gt += mk > prefix;
    eq += mk == prefix;
  }
  const int packed = gt | (eq << 16);  // n <= 1024: the fields do not overflow
  const int excl = wave_incl_scan(packed) - packed;
  int gb = excl & 0xFFFF, eb = excl >> 16;
  for (int j = lo; j < hi; ++j) {
    const uint64_t mk = s_key[j] & mask;
    // (positions are < k by construction; the checks keep every store inside
    // the k slots whatever the keys hold)
    if (mk > prefix) {
      const int pos = gb + min(eb, krem);
      if (pos < k) out[pos] = j;
      ++gb;
    } else if (mk == prefix) {
      if (eb < krem && gb + eb < k) out[gb + eb] = j;
      ++eb;
    }
  }
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

// The selection rule and the outputs of one selection, once s_key[0..n) holds
// the scores' order keys: forced blocks get a key above every score; the count
// is the top-k count (raised to the forced blocks), or the number of keys
// above the threshold's key; then block_topk_ids (an exact radix select by the
// whole workgroup); the ids go to the rows of KV heads g_lo .. g_hi - 1 (from
// LDS when UNIFIED), the scores written out are the blocks' own.
// ANDOR: the keys' fold (AND and OR, also of the keys >= 0, and their count)
// was published (topk_keys_publish) before the barrier that preceded the
// call; the selection takes it from there unless forced blocks change the
// keys.
template <int NT, bool UNIFIED, bool SCORES = true, bool ANDOR = false>
__device__ __forceinline__ void gate_finish(const GateArgs& a, int b, int g_lo, int g_hi, int n,
                                            uint64_t* s_key, int32_t* s_ids, int* s_hist,
                                            int* s_scan) {
  const int tid = threadIdx.x;
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
    for (int j = tid; j < n; j += NT) c += s_key[j] > kt;
    int total;
    block_excl_scan<NT>(c, s_scan, &total);
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
    for (int j = tid; j < n; j += NT) dst[j] = j;
  } else if (NT >= 1024 && n <= kWaveSelectMax) {
    // one wave selects: with 16 waves a workgroup barrier costs more than the
    // one wave's extra work (with 4 waves the workgroup select is faster)
    if (tid < kWave) wave_topk_ids(s_key, n, k, s_hist, dst);
  } else if (ANDOR && nf == 0) {
    block_topk_ids_from<NT>(s_key, n, k, topk_keys_collect<NT>(s_hist), s_hist, s_scan, dst);
  } else {
    block_topk_ids<NT>(s_key, n, k, s_hist, s_scan, dst);
  }
  if ((nf > 0 && SCORES) || UNIFIED) __syncthreads();
  if (nf > 0 && SCORES) {
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
      for (int j = tid; j < a.k_max; j += NT) out[j] = j < k ? s_ids[j] : -1;
    } else {
      for (int j = k + tid; j < a.k_max; j += NT) out[j] = -1;
    }
    if (tid == 0) a.sel_cnt[u] = k;
  }
  if constexpr (SCORES) {
    for (int g = g_lo; g < g_hi; ++g) {
      double* sc = a.scores + (int64_t)(b * a.Hkv + g) * a.NB;
      for (int j = tid; j < n; j += NT) sc[j] = key_score(s_key[j]);
    }
  }
}

// One workgroup per selection -- a whole sequence when the selection is
// unified over its KV heads (the only use; a per-unit selection is the same
// code with one KV head): scores for all blocks, then the selection.
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

    // ---- group-summed query, fp64, token-major then head order ----
    const int TQ = a.tokens;
    const T* q0 = (const T*)a.q + ((int64_t)b * TQ * a.Hq + (int64_t)g * G) * D;
    for (int i = tid; i < D; i += kTopkThreads) {
      double sq = 0.0;
      for (int t = 0; t < TQ; ++t) {
        const T* q = q0 + (int64_t)t * a.Hq * D;
        // All 8 possible heads are loaded (clamped to the group) before summing
        // the first G in head order, so the loads are in flight together.
        double x[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) x[h] = load_as_double<T>(q, (int64_t)min(h, G - 1) * D + i);
        sq = t == 0 ? x[0] : sq + x[0];
#pragma unroll
        for (int h = 1; h < 8; ++h) sq = h < G ? sq + x[h] : sq;
      }
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

  gate_finish<kTopkThreads, UNIFIED>(a, b, g_lo, g_hi, n, s_key, s_ids, &s_hist[0][0], s_scan);
}

// ---------------------------------------------------------------- split gate
//
// The per-unit gate in two launches, so that the scoring of long tables and
// of many units spreads over the whole chip (one workgroup per unit leaves
// most CUs idle when units are few and long, and takes several rounds when
// they are many):
//  gate_score_kernel: one 256-thread workgroup per (unit, chunk of 256
//   blocks).  Wave w owns dimensions w*D/4 .. (w+1)*D/4 - 1; each lane four
//   blocks of the chunk (16-byte loads of 4 consecutive blocks when the
//   table's rows allow, else blocks l, l+64, l+128, l+192).  Per block the
//   arithmetic is the one-kernel gate's: 4 fp64 FMA chains over the quarters
//   of d, added in quarter order, times 1/sqrt(d); the score goes to `scores`
//   (-0 written as +0, as the one-kernel gate does).
//  gate_select_kernel: one 256-thread workgroup per unit reads the scores
//   back as order keys and applies the selection rule (gate_finish).
// A table of at most 256 blocks is one chunk: gate_unit_kernel scores it into
// LDS and selects in the same workgroup, one launch.
// Unified selections keep the one-kernel gate (their scores sum the KV heads
// before the scaling).

constexpr int kScoreThreads = 256;
constexpr int kScoreChunk = 256;  // blocks per workgroup of the score kernel
constexpr int kSelectThreads = 256;

// The append of tokens lens_old[b] .. lens[b] - 1 to the blocks of one score
// chunk [j0, j0 + 256), with pool_append_kernel's arithmetic: thread i < D
// owns dimension i; the open block continues its fp64 sum from open_sum, a
// block the append opens starts from its first token, tokens are added in
// order, and each touched block's new mean is written to the pooled table and
// handed to the scoring lanes (through LDS for the chunk's first kStash
// touched blocks, else read back at device scope after the barrier).  Only
// the workgroup holding block lens_old / S reads and writes open_sum (the new
// value is the last touched block's sum, from its first token when that is a
// later block), so no two workgroups race on it.  issue() runs right after the
// pooled loads (the open sum and first key row of the chunk's first touched
// block, so a one-token append waits on no round trip of its own), apply()
// after the query loads, patch() after the barrier.  Tokens of a block
// without a valid page are skipped.
constexpr int kStash = 4;

template <typename T, int D>
struct ChunkAppend {
  int lo, hi, jlo, jhi, ja, jb;  // the append's tokens and blocks, the chunk's touched range
  double os0;                    // thread i: open sum of block ja, dim i
  T xr;                          // and its first appended key, dim i (raw)
  bool xok;                      // that key has a page

  __device__ __forceinline__ int64_t row_of(const GateArgs& a, int b, int g, int t) const {
    const int S = a.S, j = t / S, pos = t - j * S;
    if (a.page_table) {
      const int pg = a.page_table[(int64_t)b * a.NB + j];
      if (pg < 0 || pg >= a.num_pages) return -1;
      return (((int64_t)pg * a.Hkv + g) * S + pos) * D;
    }
    return (((int64_t)b * a.Hkv + g) * ((int64_t)a.NB * S) + t) * D;
  }

  __device__ __forceinline__ void issue(const GateArgs& a, int u, int b, int g, int n, int j0,
                                        int lens_old) {
    const int S = a.S;
    const int64_t cap = (int64_t)a.NB * S;
    const int tid = threadIdx.x;
    lo = lens_old;
    hi = a.lens[b];
    if (hi > cap) hi = (int)cap;
    const bool any = lo >= 0 && lo < hi;  // (uniform)
    jlo = any ? lo / S : 0;
    jhi = any ? (hi - 1) / S : -1;
    ja = any ? max(jlo, j0) : 0;
    jb = any ? min(min(jhi, j0 + kScoreChunk - 1), n - 1) : -1;
    const bool act = ja <= jb;
    const int t0 = ja * S > lo ? ja * S : lo;
    // the open sum only where the chunk continues the open block (uniform)
    os0 = (act && ja == jlo && lo % S != 0 && tid < D) ? a.open_sum[(int64_t)u * D + tid] : 0.0;
    // The first appended key of block ja: loaded outside any branch and left
    // unconverted, so nothing waits on it before apply() (an inactive chunk
    // or a block without a page reads row 0 instead: in bounds, unused).
    const int64_t r = act ? row_of(a, b, g, t0) : -1;
    xok = r >= 0;
    xr = ((const T*)a.k)[(xok ? r : 0) + (tid < D ? tid : 0)];
  }


  __device__ __forceinline__ void apply(const GateArgs& a, int u, int b, int g,
                                        float (*s_new)[D]) {
    const int tid = threadIdx.x;
    if (ja > jb || tid >= D) return;
    const int S = a.S, NB = a.NB;
    const T* kc = (const T*)a.k;
    auto block_sum = [&](int j, int t0, int t1, double& acc) {
      for (int t = t0; t < t1; ++t) {
        const int64_t r = row_of(a, b, g, t);
        if (r < 0) continue;
        const double x = load_as_double<T>(kc, r + tid);
        acc = t == j * S ? x : acc + x;
      }
    };
    for (int j = ja; j <= jb; ++j) {
      const int t0 = j * S > lo ? j * S : lo;
      const int t1 = j * S + S < hi ? j * S + S : hi;
      double acc;
      if (j == ja) {  // the prefetched open sum and first token
        const double x0 = load_as_double<T>(&xr, 0);
        acc = !xok ? os0 : (t0 == j * S ? x0 : os0 + x0);
        block_sum(j, t0 + 1, t1, acc);
      } else {
        acc = 0.0;
        block_sum(j, t0, t1, acc);
      }
      const float m = (float)(acc / (double)(t1 - j * S));
      a.pooled_out[((int64_t)u * D + tid) * NB + j] = m;
      if (j - ja < kStash) s_new[j - ja][tid] = m;
      if (j == jlo) {
        if (jhi != jlo) {
          acc = 0.0;
          block_sum(jhi, jhi * S, hi, acc);
        }
        a.open_sum[(int64_t)u * D + tid] = acc;
      }
    }
  }

  // the lane's pooled values of the touched blocks it holds
  template <int DQ, typename Blk>
  __device__ __forceinline__ void patch(const GateArgs& a, int u, int qd, Blk blk,
                                        const float (*s_new)[D], float (&pv)[DQ][4]) const {
    if (ja > jb) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = blk(e);
      if (j < ja || j > jb) continue;
      if (j - ja < kStash) {
#pragma unroll
        for (int i = 0; i < DQ; ++i) pv[i][e] = s_new[j - ja][qd * DQ + i];
      } else {
        float* col = a.pooled_out + ((int64_t)u * D + qd * DQ) * a.NB + j;
#pragma unroll
        for (int i = 0; i < DQ; ++i)
          pv[i][e] = __hip_atomic_load(col + (int64_t)i * a.NB, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
};

// Scores of blocks j0 .. j0 + 255 of unit u by a 256-thread workgroup;
// n_of() gives the blocks of its sequence, and emit(j, score) is called once
// for every j < n of the chunk, by thread j - j0.  Returns at once, for the
// whole workgroup, when j0 >= n.  EARLY: the pooled loads go out before the
// length is known, block ids clamped into the table's row (for chunks of long
// tables, which the sequence mostly fills); otherwise after it, clamped into
// the sequence's blocks (for one-chunk tables of varied lengths, where the
// row's unused tail would otherwise be read).  s_q: [D], s_part: [4][256]
// doubles of LDS.
template <typename T, int D, bool VEC4, bool APPEND, bool EARLY, typename NOf, typename Emit>
__device__ __forceinline__ void score_chunk(const GateArgs& a, int u, int b, int g, NOf n_of,
                                            int j0, double* s_q, double (*s_part)[kScoreChunk],
                                            Emit emit, int lens_old = 0) {
  constexpr int DQ = D / 4;
  const int tid = threadIdx.x, qd = tid >> 6, lane = tid & 63;
  const int NB = a.NB;
  const int G = a.Hq / a.Hkv;

  // ---- pooled loads first (EARLY: before the length is known).  Block ids
  // are clamped into [0, lim) -- the table's row (EARLY) or the sequence's
  // blocks -- so every load is in bounds; blocks at or past n are scored from
  // whatever the table holds there and never emitted ----
  int n = 0;
  if constexpr (!EARLY) {
    n = n_of();
    if (j0 >= n) return;  // the whole workgroup: nothing of this chunk is in the sequence
  }
  const int lim = EARLY ? NB : n;
  const float* pu = a.pooled + ((int64_t)u * D + (int64_t)qd * DQ) * NB;
  auto blk = [&](int e) { return VEC4 ? j0 + 4 * lane + e : j0 + lane + 64 * e; };
  float pv[DQ][4];
  if constexpr (VEC4) {
    // an aligned group of 4 (NB % 4 == 0, so it stays inside the row)
    const uint32_t jg = (uint32_t)min(j0 + 4 * lane, ((lim - 1) >> 2) << 2);
#pragma unroll
    for (int i = 0; i < DQ; ++i) {
      const float4 v = *(const float4*)(pu + (uint32_t)(i * NB) + jg);
      pv[i][0] = v.x; pv[i][1] = v.y; pv[i][2] = v.z; pv[i][3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < DQ; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[i][e] = pu[(uint32_t)(i * NB + min(blk(e), lim - 1))];
  }
  if constexpr (EARLY) {
    n = n_of();           // the length's round trip overlaps the loads
    if (j0 >= n) return;  // the whole workgroup: nothing of this chunk is in the sequence
  }
  ChunkAppend<T, D> ap;
  __shared__ float s_new[APPEND ? kStash : 1][D];
  if constexpr (APPEND) ap.issue(a, u, b, g, n, j0, lens_old);

  // ---- group-summed query, fp64, token-major then head order ----
  if (tid < D) {
    const int TQ = a.tokens;
    const T* q0 = (const T*)a.q + ((int64_t)b * TQ * a.Hq + (int64_t)g * G) * D;
    double sq = 0.0;
    for (int t = 0; t < TQ; ++t) {
      const T* q = q0 + (int64_t)t * a.Hq * D;
      double x[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) x[h] = load_as_double<T>(q, (int64_t)min(h, G - 1) * D + tid);
      sq = t == 0 ? x[0] : sq + x[0];
#pragma unroll
      for (int h = 1; h < 8; ++h) sq = h < G ? sq + x[h] : sq;
    }
    s_q[tid] = sq;
  }
  if constexpr (APPEND) ap.apply(a, u, b, g, s_new);
  __syncthreads();
  if constexpr (APPEND) ap.template patch<DQ>(a, u, qd, blk, s_new, pv);

  // ---- quarter dot products, then the blocks' sums in quarter order ----
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    double sp = 0.0;
#pragma unroll
    for (int i = 0; i < DQ; ++i) sp = fma(s_q[qd * DQ + i], (double)pv[i][e], sp);
    s_part[qd][blk(e) - j0] = sp;
  }
  __syncthreads();
  const int j = j0 + tid;
  if (j < n) {
    const double dot = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
    emit(j, dot * (1.0 / sqrt((double)D)));
  }
}

template <typename T, int D, bool VEC4, bool APPEND>
__global__ __launch_bounds__(kScoreThreads) void gate_score_kernel(GateArgs a) {
  __shared__ double s_q[D];
  __shared__ double s_part[4][kScoreChunk];
  const int nchunk = (a.NB + kScoreChunk - 1) / kScoreChunk;
  const int u = (int)blockIdx.x / nchunk, c = (int)blockIdx.x - u * nchunk;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int lens_old = APPEND ? a.lens_old[b] : 0;  // requested with the length
  double* out = a.scores + (int64_t)u * a.NB;
  score_chunk<T, D, VEC4, APPEND, true>(
      a, u, b, g, [&] { return seq_blocks(a.lens[b], a.S, a.NB); }, c * kScoreChunk, s_q, s_part,
      [&](int j, double sc) { out[j] = key_score(order_key(sc)); }, lens_old);
}

// Tables of at most 256 blocks: one workgroup per unit scores its chunk into
// LDS keys and selects, in one launch.
template <typename T, int D, bool VEC4, bool APPEND>
__global__ __launch_bounds__(kScoreThreads) void gate_unit_kernel(GateArgs a) {
  extern __shared__ uint64_t s_key[];  // [NB] order keys of the unit's scores
  __shared__ double s_q[D];
  __shared__ double s_part[4][kScoreChunk];
  __shared__ int s_hist[3 * 256];
  __shared__ int s_scan[kScoreThreads / 64 + 1];
  const int u = blockIdx.x, b = u / a.Hkv, g = u - b * a.Hkv;
  const int lens_old = APPEND ? a.lens_old[b] : 0;  // requested with the length
  KeyFold kf;  // of the keys this thread writes
  score_chunk<T, D, VEC4, APPEND, false>(
      a, u, b, g, [&] { return seq_blocks(a.lens[b], a.S, a.NB); }, 0, s_q, s_part,
      [&](int j, double sc) {
        const uint64_t key = order_key(sc);
        s_key[j] = key;
        kf.add(key);
      },
      lens_old);
  const int n = seq_blocks(a.lens[b], a.S, a.NB);
  topk_keys_publish<kScoreThreads>(kf, s_hist);
  __syncthreads();
  gate_finish<kScoreThreads, false, true, true>(a, b, g, g + 1, n, s_key, nullptr, s_hist, s_scan);
}

__global__ __launch_bounds__(kSelectThreads) void gate_select_kernel(GateArgs a) {
  constexpr int NT = kSelectThreads;
  extern __shared__ uint64_t s_key[];  // [NB] order keys of the unit's scores
  __shared__ int s_hist[3 * 256];
  __shared__ int s_scan[NT / 64 + 1];
  const int tid = threadIdx.x;
  const int u = blockIdx.x, b = u / a.Hkv, g = u - b * a.Hkv;
  const double* sc = a.scores + (int64_t)u * a.NB;
  // The first 8 * NT scores are requested with the length (ids clamped into
  // the unit's row of NB; those past n are never used): one round trip.
  double x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = sc[min(tid + e * NT, a.NB - 1)];
  const int n = seq_blocks(a.lens[b], a.S, a.NB);
  KeyFold kf;  // of the keys this thread writes
  auto put = [&](int j, double v) {
    const uint64_t key = order_key(v);
    s_key[j] = key;
    kf.add(key);
  };
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (tid + e * NT < n) put(tid + e * NT, x[e]);
  for (int j0 = tid + 8 * NT; j0 < n; j0 += 8 * NT) {  // longer tables: eight at a time
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sc[min(j0 + e * NT, n - 1)];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (j0 + e * NT < n) put(j0 + e * NT, x[e]);
  }
  topk_keys_publish<NT>(kf, s_hist);
  __syncthreads();
  gate_finish<NT, false, false, true>(a, b, g, g + 1, n, s_key, nullptr, s_hist, s_scan);
}

// ---------------------------------------------------------------- learned gate
//
// The gate network of "Sparse Attention Reasoning" (Step 1: Linear(hidden,
// 256), ReLU, Linear(256, 1)) on each block's pooled key, with the second
// layer's weights a projection of the group's query so that the decode query
// stays unpooled ("SeerAttention-R", Abstract):
//   z_jm = beta_m * (W1_m . P_j) + b1_m,  s_j = sum_m u_m relu(z_jm),
//   u_m = Wq_m . qbar (fp64),
// W1 int8 with fp32 row scales beta, P the stored fp32 pooled keys.
//
// The first layer runs on int8 MFMA (v_mfma_i32_16x16x64_i8) over an image
// of P in five int8 limbs.  Block j gets the shared exponent e_j, the
// smallest integer with 127 * 2^e_j >= max_i |P_ji| (0 for a zero block);
// x = P_ji * 2^-e_j (exact, |x| <= 127) is split as
//   x = l0 + l1 2^-7 + l2 2^-14 + l3 2^-21 + l4 2^-28 + r,
//   l0 = rint(x) in [-127, 127], then each next limb rint(128 * remainder)
//   in [-64, 64], every remainder exact in fp32 and |r| <= 2^-29,
// so the limbs hold P_ji to within 2^(e_j - 29).  Each limb's product with a
// W1 row is an exact int32 (|sum| < 2^21); the five are recombined in fp64
// exactly (multiples of 2^-28 below 2^21), scaled by 2^e_j, and the epilogue
// z = (2^e_j beta_m) D + b1 (one rounding), relu, u_m * h runs in fp64.
// Hence |s_j - s_j(exact)| <= 2^(e_j - 29) sum_m |u_m| beta_m ||W1_m||_1 plus
// fp64 rounding.  A and B carry the same lane -> k assignment, so the dot
// products do not depend on the hardware's k order.
//
// One 1024-thread workgroup per unit: wave w owns hidden units 16w .. 16w+15
// (its W1 rows come straight from memory in the A operand's layout) and every
// block tile of a chunk of 64 blocks; wave w also cuts dimensions
// w*D/16 .. of the chunk's blocks into limbs.  A score is summed over the
// wave's units, then over the 16 waves in order.  The next chunk's pooled
// loads fly while a chunk is scored.  The selection rule and outputs are the
// gate kernel's.
//
// SPLIT: with fewer units than CUs, S = gridDim.x / units workgroups share a
// unit, workgroup s taking a contiguous range of its 64-block chunks (the
// same arithmetic per block); the scores go to memory and gate_select_kernel
// selects afterwards.

constexpr int kLgThreads = 1024;  // 16 waves x 16 hidden units = 256
constexpr int kLgChunk = 64;      // blocks cut into limbs and scored per pass
constexpr int kLgLimbs = 5;       // int8 limbs per key element
constexpr int kLgPad = 16;        // bytes added to every LDS row of int8 data (bank spread)
typedef int i32x4 __attribute__((ext_vector_type(4)));

template <typename T, int D, bool SPLIT>
__global__ __launch_bounds__(kLgThreads) void learned_gate_kernel(GateArgs a) {
  constexpr int H = kGateHidden, JC = kLgChunk, NW = kLgThreads / 64, NL = kLgLimbs;
  constexpr int KS = D / 64;                 // MFMA k-steps
  constexpr int PD = D + kLgPad;             // LDS row pitch of int8 rows
  constexpr int DQ = D / NW;                 // dimensions a thread cuts (wave = dimension slice)
  constexpr int WPL = D / 16;                // Wq floats per lane (16 lanes, one DPP row, per row)
  constexpr int RPP = 4;                     // Wq rows per pass of a wave
  static_assert(H == 16 * NW, "one wave per 16 hidden units");
  static_assert(JC == 64, "one chunk block per lane");
  static_assert(DQ == 4 || DQ == 8, "4 or 8 int8 per thread and limb");
  extern __shared__ uint64_t s_key[];                 // [NB] order keys of the scores
  __shared__ __align__(16) int8_t s_pq[NL][JC * PD];  // limbs of the chunk's blocks: row j
  __shared__ double s_red[NW][JC];                    // per-wave sums of the chunk's scores
  __shared__ double s_u[H];
  __shared__ double s_q[D];
  __shared__ float s_amx[NW][JC];
  __shared__ int s_exp[JC];
  __shared__ int s_hist[3 * 256];
  __shared__ int s_scan[NW + 1];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane >> 4, n16 = lane & 15;
  const int NB = a.NB;
  // SPLIT: workgroup s of the unit's S takes chunks [s cpw, (s + 1) cpw) of
  // the table (a split by the table's width, so no load waits on the length)
  const int S = SPLIT ? (int)gridDim.x / (a.B * a.Hkv) : 1;
  const int u = (int)blockIdx.x / S, b = u / a.Hkv, g = u - b * a.Hkv;
  const int cpw = ((NB + JC - 1) / JC + S - 1) / S;
  const int jbeg = ((int)blockIdx.x - u * S) * cpw * JC;
  const int G = a.Hq / a.Hkv;
  const int jl = lane, part = wv;  // limbs: block jl of a chunk, dims part*DQ ..

  // ---- loads that wait on nothing: the first chunk's pooled columns (clamped
  // to the table, masked once the length is known), W1 rows in the A
  // operand's layout, Wq rows, row scales, biases, query ----
  const float* pcol = a.pooled + ((int64_t)u * D + part * DQ) * NB;
  float x[DQ];
  auto load_chunk = [&](int j0) {
    const float* c = pcol + min(j0 + jl, NB - 1);
#pragma unroll
    for (int i = 0; i < DQ; ++i) x[i] = c[(int64_t)i * NB];
  };
  load_chunk(jbeg);
  // A operand: W1 row 16 wv + n16, bytes 64 s + 16 r16 .. + 15 of k-step s.
  i32x4 wa[KS];
  {
    const int8_t* wrow = a.w1 + ((int64_t)g * H + wv * 16 + n16) * D + r16 * 16;
#pragma unroll
    for (int st = 0; st < KS; ++st) wa[st] = *(const i32x4*)(wrow + st * 64);
  }
  float4 wq4[16 / RPP][WPL / 4];
  const int lr = lane & 15, rp = lane >> 4;
#pragma unroll
  for (int r = 0; r < 16 / RPP; ++r)
#pragma unroll
    for (int c = 0; c < WPL / 4; ++c)
      wq4[r][c] = *(const float4*)(a.wq + ((int64_t)g * H + wv * 16 + r * RPP + rp) * D +
                                   WPL * lr + 4 * c);
  // This lane's hidden units in the MFMA result: m = 16 wv + 4 r16 + i.
  double bm[4], betam[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = wv * 16 + 4 * r16 + i;
    bm[i] = (double)a.b1[(int64_t)g * H + m];
    betam[i] = (double)a.w1_scale[(int64_t)g * H + m];
  }
  const int n = seq_blocks(a.lens[b], a.S, a.NB);
  const int jend = SPLIT ? min(n, jbeg + cpw * JC) : n;
  if (tid < D) {  // the group-summed query, fp64, head order
    const T* q = (const T*)a.q + ((int64_t)b * a.Hq + (int64_t)g * G) * D;
    double sq = load_as_double<T>(q, tid);
    for (int h = 1; h < G; ++h) sq = sq + load_as_double<T>(q, (int64_t)h * D + tid);
    s_q[tid] = sq;
  }
  __syncthreads();

  // ---- u = Wq qbar: one 16-lane row per Wq row, D/16 dimensions per lane
  // (an fp64 chain), then a DPP sum over the row ----
#pragma unroll
  for (int r = 0; r < 16 / RPP; ++r) {
    double c = 0.0;
#pragma unroll
    for (int cc = 0; cc < WPL / 4; ++cc) {
      const float4 w4 = wq4[r][cc];
      const double* qv = s_q + WPL * lr + 4 * cc;
      c = fma((double)w4.x, qv[0], c);
      c = fma((double)w4.y, qv[1], c);
      c = fma((double)w4.z, qv[2], c);
      c = fma((double)w4.w, qv[3], c);
    }
    c = row_sum16_f64(c);
    if (lr == 0) s_u[wv * 16 + r * RPP + rp] = c;
  }
  __syncthreads();
  double um[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) um[i] = s_u[wv * 16 + 4 * r16 + i];

  for (int j0 = jbeg; j0 < jend; j0 += JC) {
    // ---- limbs of blocks j0 .. j0 + JC - 1 ----
    {
      const bool live = j0 + jl < n;
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
        x[i] = live ? x[i] : 0.f;
        mx = fmaxf(mx, fabsf(x[i]));
      }
      s_amx[part][jl] = mx;
      __syncthreads();
      float amax = 0.f;
#pragma unroll
      for (int p = 0; p < NW; ++p) amax = fmaxf(amax, s_amx[p][jl]);
      int k2;
      const float f = frexpf(amax, &k2);  // amax = f * 2^k2, 0.5 <= f < 1
      const int e = amax > 0.f ? (f <= 127.f / 128.f ? k2 - 7 : k2 - 6) : 0;
      uint32_t w[NL][DQ / 4];
#pragma unroll
      for (int i = 0; i < DQ / 4; ++i) {
        uint32_t word[NL];
#pragma unroll
        for (int l = 0; l < NL; ++l) word[l] = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float r = ldexpf(x[4 * i + c], -e);  // exact, |r| <= 127
#pragma unroll
          for (int l = 0; l < NL; ++l) {
            const float li = rintf(r);         // l0 in [-127, 127], later limbs in [-64, 64]
            r = (r - li) * 128.f;              // exact: the remainder has fewer bits than r
            word[l] |= (uint32_t)((int)li & 0xFF) << (8 * c);
          }
        }
#pragma unroll
        for (int l = 0; l < NL; ++l) w[l][i] = word[l];
      }
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        int8_t* dst = &s_pq[l][jl * PD + part * DQ];
        if constexpr (DQ == 8) *(uint2*)dst = make_uint2(w[l][0], w[l][1]);
        else *(uint32_t*)dst = w[l][0];
      }
      if (part == 0) s_exp[jl] = e;
    }
    if (j0 + JC < jend) load_chunk(j0 + JC);  // the next chunk's loads fly while this one is scored
    __syncthreads();

    // ---- first layer on MFMA, limb by limb; the rest in fp64 ----
#pragma unroll 1
    for (int jt = 0; jt < JC / 16; ++jt) {
      i32x4 acc[NL];
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        acc[l] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          const i32x4 pb = *(const i32x4*)(&s_pq[l][(jt * 16 + n16) * PD + st * 64 + r16 * 16]);
          acc[l] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[st], pb, acc[l], 0, 0, 0);
        }
      }
      // lane (r16, n16) holds the products of units 16 wv + 4 r16 + i with
      // block jt*16 + n16, one int32 per limb
      const int e = s_exp[jt * 16 + n16];
      double sc = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // W1_m . (limb image) / 2^e, exact: multiples of 2^-28 below 2^21
        double dsum = (double)acc[NL - 1][i];
#pragma unroll
        for (int l = NL - 2; l >= 0; --l) dsum = fma(dsum, 0x1p-7, (double)acc[l][i]);
        const double z = fma(ldexp(betam[i], e), dsum, bm[i]);
        sc = fma(um[i], fmax(z, 0.0), sc);
      }
      sc = cross_row_sum_f64(sc);  // the four row groups: units 16 wv .. 16 wv + 15
      if (r16 == 0) s_red[wv][jt * 16 + n16] = sc;
    }
    __syncthreads();

    // ---- scores: the 16 waves' sums in order ----
    if (tid < JC && j0 + tid < n) {
      double sj = s_red[0][tid];
#pragma unroll
      for (int w = 1; w < NW; ++w) sj = sj + s_red[w][tid];
      if constexpr (SPLIT) a.scores[(int64_t)u * NB + j0 + tid] = key_score(order_key(sj));
      else s_key[j0 + tid] = order_key(sj);
    }
    // (the next chunk rewrites s_red and s_amx only after its barriers)
  }
  if constexpr (!SPLIT) {
    __syncthreads();
    gate_finish<kLgThreads, false>(a, b, g, g + 1, n, s_key, nullptr, s_hist, s_scan);
  }
}

template <typename T, int D>
const void* learned_fn(bool split) {
  return split ? (const void*)&learned_gate_kernel<T, D, true>
               : (const void*)&learned_gate_kernel<T, D, false>;
}

const void* learned_kernel(int dtype, int D, bool split = false) {
  if (dtype == 1) return D == 64 ? learned_fn<uint16_t, 64>(split) : learned_fn<uint16_t, 128>(split);
  return D == 64 ? learned_fn<float, 64>(split) : learned_fn<float, 128>(split);
}

// Workgroups per unit of the learned gate: enough to give the chip's 256 CUs
// about one each when units are fewer, at most one per 64-block chunk.
int learned_gate_split(int U, int NB) {
  constexpr int kCus = 256;
  const int chunks = (NB + kLgChunk - 1) / kLgChunk;
  if (U >= kCus || chunks < 2) return 1;
  const int s = kCus / U;
  return s < chunks ? s : chunks;
}

}  // namespace

size_t gate_smem_bytes(int NB, int k_max) {
  return (size_t)NB * sizeof(uint64_t) + (size_t)k_max * sizeof(int32_t);
}

template <typename T, int D, bool APPEND>
const void* score_fn_a(bool vec4, bool one_chunk) {
  if (one_chunk)
    return vec4 ? (const void*)&gate_unit_kernel<T, D, true, APPEND>
                : (const void*)&gate_unit_kernel<T, D, false, APPEND>;
  return vec4 ? (const void*)&gate_score_kernel<T, D, true, APPEND>
              : (const void*)&gate_score_kernel<T, D, false, APPEND>;
}

template <typename T, int D>
const void* score_fn(bool vec4, bool one_chunk, bool append) {
  return append ? score_fn_a<T, D, true>(vec4, one_chunk) : score_fn_a<T, D, false>(vec4, one_chunk);
}

const void* pick_score_fn(const GateArgs& a, bool one_chunk) {
  const bool vec4 = a.NB % 4 == 0, ap = a.append != 0;
  if (a.dtype == 1)
    return a.D == 64 ? score_fn<uint16_t, 64>(vec4, one_chunk, ap)
                     : score_fn<uint16_t, 128>(vec4, one_chunk, ap);
  return a.D == 64 ? score_fn<float, 64>(vec4, one_chunk, ap)
                   : score_fn<float, 128>(vec4, one_chunk, ap);
}

bool gate_topk_appends(const GateArgs& a) { return !a.unified; }

hipError_t launch_gate_scores(const GateArgs& a, hipStream_t stream) {
  static_assert(kGateScoreChunk == kScoreChunk, "score chunk");
  const int U = a.B * a.Hkv;
  const int nchunk = (a.NB + kScoreChunk - 1) / kScoreChunk;
  if (a.unified || nchunk < 2) return hipErrorInvalidValue;
  GateArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(pick_score_fn(a, false), dim3(U * nchunk), dim3(kScoreThreads), params,
                         0, stream);
}

hipError_t launch_gate_topk(const GateArgs& a, hipStream_t stream) {
  const int U = a.B * a.Hkv;
  GateArgs args = a;
  void* params[] = {&args};
  if (a.unified) {
    if (a.append) return hipErrorInvalidValue;  // the caller appends first
    const void* fn;
    if (a.dtype == 1) fn = a.D == 64 ? (const void*)&gate_topk_kernel<uint16_t, 64, true>
                                     : (const void*)&gate_topk_kernel<uint16_t, 128, true>;
    else fn = a.D == 64 ? (const void*)&gate_topk_kernel<float, 64, true>
                        : (const void*)&gate_topk_kernel<float, 128, true>;
    return hipLaunchKernel(fn, dim3(a.B), dim3(kTopkThreads), params,
                           gate_smem_bytes(a.NB, a.k_max), stream);
  }
  const int nchunk = (a.NB + kScoreChunk - 1) / kScoreChunk;
  const bool one = nchunk == 1;
  const void* sfn = pick_score_fn(a, one);
  if (one)  // scores and selection in one launch
    return hipLaunchKernel(sfn, dim3(U), dim3(kScoreThreads), params,
                           (size_t)a.NB * sizeof(uint64_t), stream);
  hipError_t e = hipLaunchKernel(sfn, dim3(U * nchunk), dim3(kScoreThreads), params, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)&gate_select_kernel, dim3(U), dim3(kSelectThreads), params,
                         (size_t)a.NB * sizeof(uint64_t), stream);
}

}  // namespace seer

namespace seer {

size_t learned_gate_smem_dynamic(int NB) { return (size_t)NB * sizeof(uint64_t); }

size_t learned_gate_smem_total(int D, int NB) {
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, learned_kernel(1, D)) != hipSuccess) return (size_t)-1;
  return attr.sharedSizeBytes + learned_gate_smem_dynamic(NB);
}

int learned_gate_workgroups_per_unit(int U, int NB) { return learned_gate_split(U, NB); }

hipError_t launch_learned_gate_scores(const GateArgs& a, hipStream_t stream) {
  const int U = a.B * a.Hkv;
  const int S = learned_gate_split(U, a.NB);
  if (S < 2) return hipErrorInvalidValue;  // one workgroup per unit selects itself
  GateArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(learned_kernel(a.dtype, a.D, true), dim3(U * S), dim3(kLgThreads), params,
                         0, stream);
}

hipError_t launch_learned_gate(const GateArgs& a, hipStream_t stream) {
  GateArgs args = a;
  void* params[] = {&args};
  const int U = a.B * a.Hkv;
  const int S = learned_gate_split(U, a.NB);
  if (S == 1)
    return hipLaunchKernel(learned_kernel(a.dtype, a.D), dim3(U), dim3(kLgThreads), params,
                           learned_gate_smem_dynamic(a.NB), stream);
  // scores by S workgroups per unit, then the selection
  hipError_t e = hipLaunchKernel(learned_kernel(a.dtype, a.D, true), dim3(U * S), dim3(kLgThreads),
                                 params, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)&gate_select_kernel, dim3(U), dim3(kSelectThreads), params,
                         (size_t)a.NB * sizeof(uint64_t), stream);
}

}  // namespace seer
