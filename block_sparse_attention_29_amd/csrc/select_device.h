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
  const int n = (int)(((int64_t)L + S - 1) / S);
  return n > NB ? NB : n;
}

// Kept blocks of a unit with n blocks (0 when n == 0), at most k_max.
__device__ __forceinline__ int kept_count(int n, const int32_t* top_k, int b, int keep_num,
                                          int keep_den, int k_max) {
  if (n <= 0) return 0;
  int k = top_k ? top_k[b] : (int)(((int64_t)n * keep_num + keep_den - 1) / keep_den);
  k = k < 1 ? 1 : (k > n ? n : k);
  return k > k_max ? k_max : k;
}

// Blocks kept whatever their score: block 0 and/or the newest block n-1.
__device__ __forceinline__ int forced_count(int n, int force_first, int force_last) {
  if (n <= 0) return 0;
  return (force_first ? 1 : 0) + ((force_last && !(force_first && n == 1)) ? 1 : 0);
}

// Top-k count of a unit with n blocks once nf forced blocks are counted in:
// at least nf, at most min(n, k_max), at least 1 (0 when n == 0).
__device__ __forceinline__ int kept_count_forced(int n, const int32_t* top_k, int b, int keep_num,
                                                 int keep_den, int k_max, int nf) {
  if (n <= 0) return 0;
  int k = kept_count(n, top_k, b, keep_num, keep_den, k_max);
  k = k < nf ? nf : k;
  const int cap = n < k_max ? n : k_max;
  return k > cap ? cap : k;
}

// Key that ranks a forced block above every score.
constexpr uint64_t kForcedKey = ~0ull;

// Writes the ids of the k largest keys of s_key[0..n) (ties to the lower id),
// ascending, to out[0..k).  Requires 0 < k < n and NT >= 256; every thread of
// the workgroup calls it (it contains __syncthreads()).  Scratch in LDS:
// s_hist [2 * 256], s_pick [3], s_scan [NT / 64 + 1].
//
// Exact radix select over the 64-bit keys, 8 bits per pass from the top.
// Thread t owns the contiguous ids [t*m, t*m + m).  Each pass histograms the
// next 8 bits of the candidates' keys (double-buffered histogram, the next one
// cleared during the current pass); wave 0 scans the 256 bins from the top
// with DPP and publishes the digit that holds the krem-th largest key.  After
// a pass only the keys matching the chosen prefix remain candidates; once all
// of them are needed (or all 64 bits are used) the kept set is every key with a
// larger prefix plus the first krem keys equal to it in id order.  Random
// scores usually settle after 3 passes.  One block scan of packed (above,
// equal) counts then gives every thread the output slots of its ids.
template <int NT>
__device__ void block_topk_ids(const uint64_t* s_key, int n, int k, int* s_hist, int* s_pick,
                               int* s_scan, int32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int m = (n + NT - 1) / NT;
  const int lo = min(n, tid * m), hi = min(n, lo + m);
  uint64_t prefix = 0, mask = 0;
  int krem = k;
  if (tid < 256) s_hist[tid] = 0;
  __syncthreads();
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    int* hist = s_hist + (pass & 1) * 256;
    for (int j = lo; j < hi; ++j) {
      const uint64_t key = s_key[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(int)((key >> shift) & 255)], 1);
    }
    if (tid < 256) s_hist[((pass & 1) ^ 1) * 256 + tid] = 0;
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

}  // namespace seer
