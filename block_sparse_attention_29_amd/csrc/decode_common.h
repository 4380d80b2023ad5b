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
