// Definitions shared by the decode kernels (sparse_decode.hip, multi_decode.hip):
// the tile geometry, the equal split of the tiles over the waves, and lane
// helpers.
#pragma once

#include "seer_device.h"
#include "seer_kernels.h"

namespace seer {
namespace {

constexpr int kTile = 32;          // tokens per tile (two 16-wide MFMA columns)
constexpr int kXcds = 8;           // XCDs (each with its own L2) of an MI355X
constexpr int kCols = kTile / 16;  // 16-token MFMA columns per tile
constexpr int kWavesPerWG = kDecodeWavesPerWG;
constexpr int kThreads = kWavesPerWG * kWave;
constexpr float kNegInf = -__builtin_huge_valf();

template <typename T, int D>
struct Geo {
  static constexpr int EB = sizeof(T);
  static constexpr int ROWB = D * EB;      // bytes per token row
  static constexpr int E = 16 / EB;        // elements per 16-byte chunk
  static constexpr int NKL = ROWB / 64;    // K chunks per lane per 16-token column
  static constexpr int LPR = ROWB / 16;    // lanes per V row
  static constexpr int RPI = kWave / LPR;  // V rows per load instruction
  static constexpr int NVL = kTile / RPI;  // V chunks per lane per tile
};

__device__ __forceinline__ int64_t readlane64(int64_t x, int lane) {
  const int lo = readlane_i((int)(uint32_t)(uint64_t)x, lane);
  const int hi = readlane_i((int)(uint32_t)((uint64_t)x >> 32), lane);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// ---- P V of one 32-token tile on bf16 matrix cores (bf16 caches, d = 128) ----
//
// The probabilities of a 16-row tile (row 4 r16 + i, tokens 2 n16 and
// 2 n16 + 1 in lane (r16, n16), register i of x[0] and x[1]) are split into
// two bf16 parts, p = hi + lo with lo = bf16(p - hi) (p - hi is exact in fp32,
// so hi + lo holds p to 16 significant bits), and stored in the wave's 2 KiB
// LDS buffer as [part][row][token] words of two tokens.
__device__ __forceinline__ void store_p_split(uint32_t* pb, const float (&x)[kCols][4], int r16,
                                              int n16) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t hi = pack_bf16_rne(x[0][i], x[1][i]);
    const float r0 = x[0][i] - bf16_lo(hi), r1 = x[1][i] - bf16_hi(hi);
    const int at = (4 * r16 + i) * (kTile / 2) + n16;
    pb[at] = hi;
    pb[16 * (kTile / 2) + at] = pack_bf16_rne(r0, r1);
  }
}

// O += P V as v_mfma_f32_16x16x32_bf16 with k = the tile's 32 tokens, lane
// (r16, n16) holding k = 8 r16 .. 8 r16 + 7: A = P (row n16, hi and lo parts
// from LDS), B for dimension step e = V[k][8 n16 + e], the e-th bf16 of the
// lane's chunks vr[j] (token 8 r16 + j, dimensions 8 n16 .. 8 n16 + 7)
// packed in pairs.  oacc[e] holds O[row 4 r16 + i][8 n16 + e] in register i.
// The products are exact and summed in fp32.  Tokens at or past tv are
// zeroed (their rows may hold anything, even NaN).
__device__ __forceinline__ void pv_bf16(const uint32_t* pb, const uint4 (&vr)[8], int tv,
                                        f32x4 (&oacc)[8], int r16, int n16) {
  const uint4 ah = *(const uint4*)(pb + n16 * (kTile / 2) + 4 * r16);
  const uint4 al = *(const uint4*)(pb + 16 * (kTile / 2) + n16 * (kTile / 2) + 4 * r16);
  uint4 vv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) vv[j] = vr[j];
  if (tv < kTile) {  // uniform
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool live = 8 * r16 + j < tv;
      vv[j].x = live ? vv[j].x : 0u;
      vv[j].y = live ? vv[j].y : 0u;
      vv[j].z = live ? vv[j].z : 0u;
      vv[j].w = live ? vv[j].w : 0u;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // bf16 e of a chunk: the low (e even) or high (e odd) half of word e / 2
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    const int q = e >> 1;
    uint32_t wd[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint4& c0 = vv[2 * jj];
      const uint4& c1 = vv[2 * jj + 1];
      const uint32_t a0 = q == 0 ? c0.x : q == 1 ? c0.y : q == 2 ? c0.z : c0.w;
      const uint32_t a1 = q == 0 ? c1.x : q == 1 ? c1.y : q == 2 ? c1.z : c1.w;
      wd[jj] = __builtin_amdgcn_perm(a1, a0, sel);
    }
    const bf16x8 bv = __builtin_bit_cast(bf16x8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
    oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah), bv, oacc[e],
                                                      0, 0, 0);
    oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, al), bv, oacc[e],
                                                      0, 0, 0);
  }
}

// Wave owning tile y when Tot tiles are split over W waves in equal ranges:
// the largest w with floor(w Tot / W) <= y.
__device__ __forceinline__ int tile_owner(int64_t y, int W, int64_t Tot) {
  return (int)div_floor((y + 1) * W - 1, Tot);
}

// Whether wave w owns no tile under the equal split.
__device__ __forceinline__ bool wave_empty(const EqualSplit& sp, int w) {
  return sp.start(w) == sp.start(w + 1);
}

}  // namespace
}  // namespace seer
