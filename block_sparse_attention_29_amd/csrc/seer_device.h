// Device-side helpers shared by the gfx950 kernels of libseer.
//
// Wavefronts are 64 lanes wide.  A "row" is a group of 16 consecutive lanes,
// the unit that gfx9 DPP row operations work on and the unit in which a
// 16x16 MFMA result is laid out.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seer {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats rounded to bf16 (nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Element e of a 16-byte chunk holding bf16 (T = uint16_t) or fp32 (T = float).
template <typename T>
__device__ __forceinline__ float chunk_elem(const uint4& c, int e);

template <>
__device__ __forceinline__ float chunk_elem<uint16_t>(const uint4& c, int e) {
  const uint32_t w = (e >> 1) == 0 ? c.x : (e >> 1) == 1 ? c.y : (e >> 1) == 2 ? c.z : c.w;
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

template <>
__device__ __forceinline__ float chunk_elem<float>(const uint4& c, int e) {
  const uint32_t w = e == 0 ? c.x : e == 1 ? c.y : e == 2 ? c.z : c.w;
  return __uint_as_float(w);
}

// ---------------------------------------------------------------- DPP

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Every control used here names an in-row source lane for every lane, so the
// plain move form (no "old" operand) is exact.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Max / sum over the 16 lanes of a row; every lane of the row gets the result.
// IEEE max and + are commutative, so every lane computes the same value.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return x;
}

__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  x += dpp_f32<kDppRowHalfMirror>(x);
  x += dpp_f32<kDppRowMirror>(x);
  return x;
}

// fp64 through two 32-bit DPP moves.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// Sum over the 16 lanes of a row, pairs first (lanes i, i^1), then quads,
// eights and the row; IEEE addition commutes, so every lane gets the same bits.
__device__ __forceinline__ double row_sum16_f64(double x) {
  x = x + dpp_f64<kDppQuadXor1>(x);
  x = x + dpp_f64<kDppQuadXor2>(x);
  x = x + dpp_f64<kDppRowHalfMirror>(x);
  return x + dpp_f64<kDppRowMirror>(x);
}

// Sum over the four rows of the wave, (r0 + r1) + (r2 + r3), in every lane:
// v_permlane16_swap with both operands x leaves rows (0,0,2,2) in the first
// result and (1,1,3,3) in the second; v_permlane32_swap then pairs the halves.
__device__ __forceinline__ double cross_row_sum_f64(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  const auto l16 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  auto mk = [](uint32_t l, uint32_t h) {
    return __longlong_as_double((long long)(((uint64_t)h << 32) | l));
  };
  const double y = mk(l16[0], h16[0]) + mk(l16[1], h16[1]);
  const uint64_t c = (uint64_t)__double_as_longlong(y);
  const uint32_t clo = (uint32_t)c, chi = (uint32_t)(c >> 32);
  const auto l32 = __builtin_amdgcn_permlane32_swap(clo, clo, false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap(chi, chi, false, false);
  return mk(l32[0], h32[0]) + mk(l32[1], h32[1]);
}

// The same over fp32: (r0 + r1) + (r2 + r3) of the four rows, in every lane.
__device__ __forceinline__ float cross_row_sum_f32(float x) {
  const uint32_t b = __float_as_uint(x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const float y = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  const uint32_t c = __float_as_uint(y);
  const auto p32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

// x + x of the lane 32 apart (lower half + upper half), in every lane.
__device__ __forceinline__ float cross_half_sum_f32(float x) {
  const uint32_t b = __float_as_uint(x);
  const auto p32 = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

constexpr int kDppRowRor8 = 0x128;  // row_ror:8, lane i of a row reads lane i ^ 8

__device__ __forceinline__ int readlane_i(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }
__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// ---------------------------------------------------------------- scans

// Adds the DPP-moved value of x; lanes without a source lane add 0 (the
// "old" operand), since bound_ctrl is off and every row/bank is enabled.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP: shifts by 1, 2, 4,
// 8 within each 16-lane row, then row 0's and row 2's totals (lane 15, 47) are
// broadcast into rows 1 and 3, then lane 31's total into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x = dpp_add<0x111, 0xF>(x);  // row_shr:1
  x = dpp_add<0x112, 0xF>(x);  // row_shr:2
  x = dpp_add<0x114, 0xF>(x);  // row_shr:4
  x = dpp_add<0x118, 0xF>(x);  // row_shr:8
  x = dpp_add<0x142, 0xA>(x);  // row_bcast:15 into rows 1, 3
  x = dpp_add<0x143, 0xC>(x);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64, at most
// 1024).  `scratch` holds NT/64 + 1 ints of shared memory.  Returns the
// exclusive prefix; *total gets the block total.  Contains __syncthreads().
template <int NT>
__device__ __forceinline__ int block_excl_scan(int x, int* scratch, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int inc = wave_incl_scan(x);
  if (lane == 63) scratch[wv] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int s = scratch[i];
    base += (i < wv) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - x;
}

// ---------------------------------------------------------------- division

// floor(x / d) for 0 <= x < 2^52 and 0 < d < 2^31.  The fp64 quotient is off
// by less than one there, so one integer step either way makes it exact; far
// shorter than the generic 64-bit integer division.
__device__ __forceinline__ int64_t div_floor(int64_t x, int64_t d) {
  int64_t q = (int64_t)((double)x / (double)d);
  const int64_t r = x - q * d;
  q += (r < 0) ? -1 : (r >= d ? 1 : 0);
  return q;
}

// Equal split of `total` items over `parts` parts: part w starts at
// floor(w * total / parts).  With total = q * parts + r that is
// w * q + floor(w * r / parts), in 32-bit arithmetic for parts < 46341.
struct EqualSplit {
  int q, r, parts;
  __device__ __forceinline__ EqualSplit(int total, int parts_)
      : q(total / parts_), r(total - (total / parts_) * parts_), parts(parts_) {}
  __device__ __forceinline__ int start(int w) const {
    return w * q + (int)((uint32_t)(w * r) / (uint32_t)parts);
  }
};

// ---------------------------------------------------------------- fp64 order key

// Order-preserving map of a finite double to uint64 (larger value -> larger
// key), with -0.0 and +0.0 mapped to the same key.
__device__ __forceinline__ uint64_t order_key(double s) {
  if (s == 0.0) s = 0.0;  // folds -0.0 into +0.0
  const uint64_t bits = (uint64_t)__double_as_longlong(s);
  return (bits >> 63) ? ~bits : (bits | 0x8000000000000000ull);
}

// Inverse of order_key (a -0.0 score comes back as +0.0).
__device__ __forceinline__ double key_score(uint64_t key) {
  const uint64_t bits = (key >> 63) ? (key & 0x7FFFFFFFFFFFFFFFull) : ~key;
  return __longlong_as_double((long long)bits);
}

}  // namespace seer
