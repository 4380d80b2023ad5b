// Exact top-k block selection by one workgroup, shared by the gate kernel and
// the fused gate + decode kernel.
//
// The kept count follows "Sparse Attention Reasoning" (Step 1: top-k over the
// gate's scores, k from the sparsity) and "SeerAttention-R: Sparse Attention
// Adaptation for Long Reasoning" (Abstract: 90% sparsity or a token budget):
// either an explicit count per sequence (a token budget T is T / S blocks),
// clamped to [1, n], or the smallest count that covers the kept fraction
// keep_num / keep_den of the n blocks, in integer arithmetic.
//
// Order: score descending, ties to the lower block id (the scores enter as
// 64-bit order keys, which also make -0.0 equal to +0.0); the kept ids are
// written in ascending order.
#pragma once

#include "seer_device.h"

namespace seer {

// Blocks a sequence of L tokens occupies, at most NB.
__device__ __forceinline__ int seq_blocks(int L, int S, int NB) {
  if (L <= 0) return 0;
  const int n = (L - 1) / S + 1;
  return n > NB ? NB : n;
}

// Kept blocks of a unit with n blocks (0 when n == 0), at most k_max: the
// explicit count kval when `explicit_k`, else the keep rule.
// (n < 2^14 and keep_num <= keep_den < 2^31, so the product is below 2^52.)
__device__ __forceinline__ int kept_count_of(int n, bool explicit_k, int kval, int keep_num,
                                             int keep_den, int k_max) {
  if (n <= 0) return 0;
  int k = explicit_k ? kval : (int)div_floor((int64_t)n * keep_num + keep_den - 1, keep_den);
  k = k < 1 ? 1 : (k > n ? n : k);
  return k > k_max ? k_max : k;
}

__device__ __forceinline__ int kept_count(int n, const int32_t* top_k, int b, int keep_num,
                                          int keep_den, int k_max) {
  return kept_count_of(n, top_k != nullptr, top_k ? top_k[b] : 0, keep_num, keep_den, k_max);
}

// Blocks kept whatever their score: block 0 and/or the newest block n-1.
__device__ __forceinline__ int forced_count(int n, int force_first, int force_last) {
  if (n <= 0) return 0;
  return (force_first ? 1 : 0) + ((force_last && !(force_first && n == 1)) ? 1 : 0);
}

// Top-k count of a unit with n blocks once nf forced blocks are counted in:
// at least nf, at most min(n, k_max), at least 1 (0 when n == 0).
__device__ __forceinline__ int kept_count_forced_of(int n, bool explicit_k, int kval,
                                                    int keep_num, int keep_den, int k_max,
                                                    int nf) {
  if (n <= 0) return 0;
  int k = kept_count_of(n, explicit_k, kval, keep_num, keep_den, k_max);
  k = k < nf ? nf : k;
  const int cap = n < k_max ? n : k_max;
  return k > cap ? cap : k;
}

__device__ __forceinline__ int kept_count_forced(int n, const int32_t* top_k, int b, int keep_num,
                                                 int keep_den, int k_max, int nf) {
  return kept_count_forced_of(n, top_k != nullptr, top_k ? top_k[b] : 0, keep_num, keep_den,
                              k_max, nf);
}

// Key that ranks a forced block above every score.
constexpr uint64_t kForcedKey = ~0ull;

// What the radix select starts from, folded over the order keys: the AND and
// OR of all keys, and the AND, OR and number of the keys with the top bit set
// (the scores >= 0).  The bits every key of a set shares are bits the select
// need not histogram; when at least k keys are >= 0, the kept keys are among
// those, and their shared bits usually reach much further down (the sign and
// most of the exponent), which saves a pass.  Each thread folds the keys it
// holds (add); topk_keys_publish, called by every thread before a workgroup
// barrier, reduces the folds per wave (DPP within rows, lane reads across
// them) into s_hist[512 .. 512 + 9 NT/64) and clears the first histogram
// s_hist[0 .. 256); after the barrier topk_keys_collect gives every thread
// the block's fold.  A caller that writes the keys can fold them as it
// writes and publish before the barrier that follows the writes, saving the
// select a pass over the keys and a barrier.
struct KeyFold {
  uint64_t kand = ~0ull, kor = 0;  // all keys
  uint64_t pand = ~0ull, por = 0;  // keys >= 2^63 (scores >= 0)
  int np = 0;                      // how many of those
  __device__ __forceinline__ void add(uint64_t key) {
    kand &= key;
    kor |= key;
    const bool p = (key >> 63) != 0;
    pand = p ? (pand & key) : pand;
    por = p ? (por | key) : por;
    np += p ? 1 : 0;
  }
};

constexpr int kFoldWords = 9;  // per wave in s_hist[512 ..]: 4 ANDs, 4 ORs, the count

template <int NT>
__device__ __forceinline__ void topk_keys_publish(const KeyFold& f, int* s_hist) {
  static_assert(512 + kFoldWords * (NT / 64) <= 3 * 256, "fold words fit the third histogram");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t r[kFoldWords] = {(uint32_t)f.kand, (uint32_t)(f.kand >> 32),
                            (uint32_t)f.pand, (uint32_t)(f.pand >> 32),
                            (uint32_t)f.kor,  (uint32_t)(f.kor >> 32),
                            (uint32_t)f.por,  (uint32_t)(f.por >> 32), (uint32_t)f.np};
#pragma unroll
  for (int i = 0; i < kFoldWords; ++i) {
    // words 0-3 fold by AND, 4-7 by OR, 8 by addition
    auto op = [&](uint32_t x, uint32_t y) { return i < 4 ? (x & y) : i < 8 ? (x | y) : x + y; };
    uint32_t x = r[i];
    x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppQuadXor1, 0xF, 0xF, true));
    x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppQuadXor2, 0xF, 0xF, true));
    x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowHalfMirror, 0xF, 0xF, true));
    x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kDppRowMirror, 0xF, 0xF, true));
    const uint32_t a0 = (uint32_t)readlane_i((int)x, 0), a1 = (uint32_t)readlane_i((int)x, 16);
    const uint32_t a2 = (uint32_t)readlane_i((int)x, 32), a3 = (uint32_t)readlane_i((int)x, 48);
    r[i] = op(op(a0, a1), op(a2, a3));
  }
  int* s_red = s_hist + 2 * 256;
  if (lane < kFoldWords) {
    uint32_t v = r[0];
#pragma unroll
    for (int i = 1; i < kFoldWords; ++i) v = lane == i ? r[i] : v;
    s_red[wv * kFoldWords + lane] = (int)v;
  }
  if (tid < 256) s_hist[tid] = 0;
}

template <int NT>
__device__ __forceinline__ KeyFold topk_keys_collect(const int* s_hist) {
  constexpr int NW = NT / 64;
  const int* s_red = s_hist + 2 * 256;
  uint32_t t[kFoldWords] = {~0u, ~0u, ~0u, ~0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int w = 0; w < NW; ++w) {
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] &= (uint32_t)s_red[w * kFoldWords + i];
#pragma unroll
    for (int i = 4; i < 8; ++i) t[i] |= (uint32_t)s_red[w * kFoldWords + i];
    t[8] += (uint32_t)s_red[w * kFoldWords + 8];
  }
  KeyFold f;
  f.kand = ((uint64_t)t[1] << 32) | t[0];
  f.pand = ((uint64_t)t[3] << 32) | t[2];
  f.kor = ((uint64_t)t[5] << 32) | t[4];
  f.por = ((uint64_t)t[7] << 32) | t[6];
  f.np = (int)t[8];
  return f;
}

// Writes the ids of the k largest keys of s_key[0..n) (ties to the lower id),
// ascending, to out[0..k), given the keys' block-wide fold (see
// topk_keys_publish, whose barrier must have passed: it also clears the
// first histogram).  Requires 0 < k < n and NT >= 256; every thread of the
// workgroup calls it (it contains __syncthreads()).  Scratch in LDS: s_hist
// [3 * 256], s_scan [NT / 64 + 1].
//
// Exact radix select over the 64-bit keys.  Thread t owns the contiguous ids
// [t*m, t*m + m).  The first digit is the 8 bits from the highest bit where
// the candidates differ (the keys >= 2^63 when at least k of them exist, else
// all keys), each later digit the next 8 bits down.  Each pass histograms
// the digit of the keys still matching the chosen prefix, and every wave
// scans the 256 bins from the top (DPP) to find the digit that holds the
// krem-th largest key, so one barrier per pass suffices: the histograms
// rotate over three buffers, the one cleared during a pass last read two
// passes before.  Once every remaining candidate is needed (or all bits are
// used) the kept set is every key with a larger prefix plus the first krem
// keys equal to it in id order.  One block scan of packed (above, equal)
// counts then gives every thread the output slots of its ids.
template <int NT>
__device__ void block_topk_ids_from(const uint64_t* s_key, int n, int k, const KeyFold& f,
                                    int* s_hist, int* s_scan, int32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int m = (n + NT - 1) / NT;
  const int lo = min(n, tid * m), hi = min(n, lo + m);
  // When at least k keys are >= 2^63 (and some are not), every kept key is
  // one of them: start from the bits those share (bit 63 among them, so no
  // smaller key matches the prefix and none exceeds it); else from the bits
  // all keys share.
  const bool upper = f.np >= k && f.np < n;
  const uint64_t cand = upper ? f.pand : f.kand, cor = upper ? f.por : f.kor;
  const uint64_t diff = cand ^ cor;

  int top = diff ? 63 - __builtin_clzll(diff) : -1;  // highest bit where candidates differ
  uint64_t mask = top >= 63 ? 0ull : (~0ull << (top + 1));
  uint64_t prefix = cand & mask;
  int krem = k;
  int slot = 0, nxt = 1;
  while (top >= 0) {
    const int shift = top > 7 ? top - 7 : 0;
    int* hist = s_hist + slot * 256;
    for (int j = lo; j < hi; ++j) {
      const uint64_t key = s_key[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(int)((key >> shift) & 255)], 1);
    }
    if (tid < 256) s_hist[nxt * 256 + tid] = 0;
    __syncthreads();
    // every wave: lane l holds digits 255-4l .. 252-4l (descending)
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
    // exactly one lane picked
    const int src = __builtin_ctzll(__ballot(pick >= 0));
    const int dv = readlane_i(pick, src), cnt = readlane_i(pc, src);
    krem = readlane_i(nk, src);
    prefix |= (uint64_t)dv << shift;
    mask |= (uint64_t)255 << shift;
    if (cnt == krem) break;  // every remaining candidate is kept
    top = shift - 1;
    slot = nxt;
    nxt = nxt == 2 ? 0 : nxt + 1;
  }

  int gt = 0, eq = 0;
  for (int j = lo; j < hi; ++j) {
    const uint64_t mk = s_key[j] & mask;
    gt += mk > prefix;
    eq += mk == prefix;
  }
  int total;
  const int packed = block_excl_scan<NT>(gt | (eq << 16), s_scan, &total);
  int gb = packed & 0xFFFF, eb = packed >> 16;
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

// block_topk_ids_from with the fold taken here: a pass over the keys
// and a barrier.  Same requirements and scratch.
template <int NT>
__device__ void block_topk_ids(const uint64_t* s_key, int n, int k, int* s_hist, int* s_scan,
                               int32_t* out) {
  const int tid = threadIdx.x;
  const int m = (n + NT - 1) / NT;
  const int lo = min(n, tid * m), hi = min(n, lo + m);
  KeyFold f;
  for (int j = lo; j < hi; ++j) f.add(s_key[j]);
  topk_keys_publish<NT>(f, s_hist);
  __syncthreads();
  block_topk_ids_from<NT>(s_key, n, k, topk_keys_collect<NT>(s_hist), s_hist, s_scan, out);
}

}  // namespace seer
