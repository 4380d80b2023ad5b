// Split-KV block-sparse decode of several new query tokens per sequence
// (speculative or chunked decode) for gfx950.
//
// Sequence b has T new tokens at positions L_b - T .. L_b - 1, their keys and
// values already in the cache.  For KV head g, the G query heads of each of
// the T tokens are one unit's R = G * T <= 16 query rows, row r = t * G + h.
// Token t attends to the tokens of the kept blocks at positions
// p <= L_b - T + t: "Sparse Attention Reasoning", Step 4, with query_len = T
// and the causal mask of autoregressive decoding; one selection per
// (sequence, KV head) serves all T tokens, so the kept K/V bytes are read
// once for T tokens.
//
// The work split is the single-token kernel's (equal ranges of 32-token tiles
// over all waves, one partial record per (unit, wave) segment, merged in wave
// order).  Per tile a wave:
//  * computes the 16 x 32 logits with v_mfma_f32_16x16x32_bf16 (fp32 data:
//    v_mfma_f32_16x16x4_f32), the R query rows being the A operand;
//  * masks each row to its token's causal limit, updates the online softmax
//    and writes the probabilities (fp32) to a 2 KiB LDS buffer;
//  * multiplies them with V on v_mfma_f32_16x16x4_f32 in fp32: V is loaded
//    16 lanes per token row, so lane (r, n) holds token 4k + r, dimensions
//    n*D/16 .. of load k, which is exactly the B operand of k-step k for
//    column n -- output column n of dimension step e is dimension n*D/16 + e,
//    and each lane's rows of the result are its rows of the softmax state.
#include "decode_common.h"
#include "gate_phase.h"
#include "select_device.h"

namespace seer {
namespace {

constexpr int kRows = kMultiRows;  // MFMA rows: G * T <= 16

template <typename T, int D>
struct MGeo {
  static constexpr int EB = sizeof(T);
  static constexpr int ROWB = D * EB;     // bytes per token row
  static constexpr int NKL = ROWB / 64;   // K chunks per lane per 16-token column
  static constexpr int VB = ROWB / 16;    // V bytes per lane per token row (16 lanes a row)
  static constexpr int DPL = D / 16;      // V dimensions per lane
  static constexpr int NVQ = (VB + 15) / 16;  // 16-byte pieces per lane per token row
  static constexpr int REC = kRows * D + 2 * kRows;  // record: acc[16][D], m[16], l[16]
};

// V element e (0 .. DPL-1) of a lane's token row piece, as fp32.
template <typename T, int NVQ>
__device__ __forceinline__ float v_elem(const uint4 (&v)[NVQ], int e);

template <>
__device__ __forceinline__ float v_elem<uint16_t, 1>(const uint4 (&v)[1], int e) {
  return chunk_elem<uint16_t>(v[0], e);
}
template <>
__device__ __forceinline__ float v_elem<float, 1>(const uint4 (&v)[1], int e) {
  return chunk_elem<float>(v[0], e);
}
template <>
__device__ __forceinline__ float v_elem<float, 2>(const uint4 (&v)[2], int e) {
  return chunk_elem<float>(v[e >> 2], e & 3);
}

// GATED: every workgroup first scores and selects the blocks of the units it
// streams (the gate of gate_phase.h with the query summed over the T tokens
// and the group's heads), as the single-token kernel does.
template <typename T, int D, bool GATED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_multi_kernel(DecodeArgs a) {
  using GE = MGeo<T, D>;
  constexpr int EB = GE::EB, ROWB = GE::ROWB, NKL = GE::NKL, VB = GE::VB, DPL = GE::DPL;
  constexpr int NVQ = GE::NVQ, REC = GE::REC;
  // bf16 caches with d = 128 multiply P V on bf16 matrix cores (MPV, as the
  // single-token kernel does); other caches on fp32 matrix cores.
  constexpr bool MPV = EB == 2 && D == 128;
  static_assert(!MPV || (NVQ == 1 && DPL == 8), "MPV: one 16-byte V chunk per lane and row");

  __shared__ __align__(16) float s_p[kWavesPerWG][kTile * kRows];
  extern __shared__ int s_dyn[];

  const int U = a.B * a.Hkv;
  const int tid = threadIdx.x;
  const int TQ = a.tokens, G = a.Hq / a.Hkv, R = G * TQ;
  int* s_prefix = s_dyn;                         // [U + 1]
  int* s_scan = s_dyn + U + 1;                   // [kWavesPerWG + 1]
  int* s_len = s_dyn + U + 1 + kWavesPerWG + 1;  // [U]

  const int nwg = (int)gridDim.x;
  const int wg = (nwg % kXcds == 0)
      ? (int)(blockIdx.x % kXcds) * (nwg / kXcds) + (int)(blockIdx.x / kXcds)
      : (int)blockIdx.x;
  const int wg0 = wg * kWavesPerWG;
  GatePreload<T, D, kRows> pre;  // the fused gate's entry loads
  pre.u = -1;

  // ---- plan: block prefix over units (every workgroup computes the same) ----
  {
    const int per = (U + kThreads - 1) / kThreads;
    const int u_lo = min(U, tid * per), u_hi = min(U, u_lo + per);
    // the thread's first unit's loads first, the gate's entry loads after them
    const int u_f = min(u_lo, U - 1);
    const int L_f = a.lens[u_f / a.Hkv];
    const int aux_f = unit_aux<GATED>(a, u_f);
    // (wg0 * U < 2^31: fewer than 2^15 waves, at most 2^13 units)
    if constexpr (GATED)
      issue_gate_preload<T, D, kRows, true>(a, (int)((uint32_t)(wg0 * U) / (uint32_t)a.W), pre);
    int local = 0;
    for (int u = u_lo; u < u_hi; ++u) {
      const int L = u == u_lo ? L_f : a.lens[u / a.Hkv];
      const int c = unit_blocks<GATED>(a, L, u == u_lo ? aux_f : unit_aux<GATED>(a, u));
      s_len[u] = L;
      s_prefix[u] = c;
      local += c;
    }
    int total;
    int base = block_excl_scan<kThreads>(local, s_scan, &total);
    for (int u = u_lo; u < u_hi; ++u) {
      const int c = s_prefix[u];
      s_prefix[u] = base;
      base += c;
    }
    if (tid == 0) s_prefix[U] = total;
    __syncthreads();
  }

  const int lane = tid & 63, wv = tid >> 6;
  const int r16 = lane >> 4, n16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(wg * kWavesPerWG + wv);
  const int tsh = 31 - __builtin_clz(a.S / kTile);
  const int Tot = __builtin_amdgcn_readfirstlane(s_prefix[U]) << tsh;
  const EqualSplit split(Tot, a.W);

  // ---- fused gate: the selections of every unit this workgroup streams, into
  // LDS (a unit shared by workgroups is selected by each, bit-identically) ----
  int32_t* s_ids = s_len + U;  // [ids_cap] kept ids of this workgroup's units, slot - ids_base
  int ids_base = 0;
  // The scores of the unit gated last stay in s_key (LDS) to the end.
  uint64_t* s_key = (uint64_t*)(((uintptr_t)(s_ids + a.ids_cap) + 7) & ~(uintptr_t)7);
  // The unit whose selection this workgroup writes out after its tiles (-1:
  // none): outputs still in flight would hold the first tile back (stores and
  // loads share one memory counter).  Only the last unit gated can wait: the
  // next unit's gate reuses s_key.
  int late_u = -1;
  if constexpr (GATED) {
    __shared__ double s_q[D];
    __shared__ double s_part[4 * 256];  // quarter sums of one pass
    __shared__ int s_hist[3 * 256];
    __shared__ int s_sel_scan[kWavesPerWG + 1];
    __shared__ int s_wgu[2];            // units of the workgroup's first and last tile
    const int Y0 = split.start(wg0);
    const int Y1 = split.start(wg0 + kWavesPerWG);
    if (Y0 < Y1) {
      {
        const int x0 = Y0 >> tsh, x1 = (Y1 - 1) >> tsh;  // their blocks
        for (int uu = tid; uu < U; uu += kThreads) {
          const int lo = s_prefix[uu], hi = s_prefix[uu + 1];
          if (lo <= x0 && x0 < hi) s_wgu[0] = uu;
          if (lo <= x1 && x1 < hi) s_wgu[1] = uu;
        }
        __syncthreads();
      }
      const int u0 = s_wgu[0], u1 = s_wgu[1];
      ids_base = s_prefix[u0];
      auto gate = [&](int u, auto pre_tag) {
        const int k = s_prefix[u + 1] - s_prefix[u];
        if (k == 0) return;
        // the owner holds the unit's first tile
        const int owner = tile_owner((int64_t)s_prefix[u] << tsh, a.W, Tot) / kWavesPerWG;
        const bool late = owner == wg && u == u1;
        if (late) late_u = u;
        fused_gate_unit<T, D, kRows, true, decltype(pre_tag)::value>(
            a, u, seq_blocks(s_len[u], a.S, a.NB), k, s_ids + (s_prefix[u] - ids_base),
            owner == wg && !late, s_key, s_q, s_part, s_hist, s_sel_scan, pre);
      };
      // The first unit may use the entry loads; peeled off, so that they are
      // dead in the loop.
      gate(u0, BoolTag<true>{});
      for (int u = u0 + 1; u <= u1; ++u) gate(u, BoolTag<false>{});
    }
  }
  // The stores that nothing in this launch reads, issued by every thread once
  // its own tiles are done (from LDS values that were final before a barrier
  // it has passed): workgroup 0's copy of the plan for the merge and, with the
  // gate, the (empty) selections of units without a kept block (a sequence of
  // length 0, which belong to nobody), and the late unit's outputs.
  auto write_late = [&]() {
    if (blockIdx.x == 0) {
      for (int uu = tid; uu <= U; uu += kThreads) a.prefix[uu] = s_prefix[uu];
      if (tid == 0) a.hdr[0] = a.W;
      if (GATED) {
        for (int uu = tid; uu < U; uu += kThreads) {
          if (s_prefix[uu] != s_prefix[uu + 1]) continue;
          for (int i = 0; i < a.k_max; ++i) a.sel_idx_out[(int64_t)uu * a.k_max + i] = -1;
          a.sel_cnt_out[uu] = 0;
        }
      }
    }
    if (GATED && late_u >= 0)
      fused_gate_write(a, late_u, seq_blocks(s_len[late_u], a.S, a.NB),
                       s_prefix[late_u + 1] - s_prefix[late_u],
                       s_ids + (s_prefix[late_u] - ids_base), s_key);
  };
  const int y0 = split.start(w), y1 = split.start(w + 1);
  if (y0 >= y1) {
    write_late();
    return;
  }

  const bool sparse = a.sel_idx != nullptr;
  const int Hkv = a.Hkv, S = a.S, NB = a.NB;
  const char* kbase = (const char*)a.k;
  const char* vbase = (const char*)a.v;
  float* pw = s_p[wv];
  const float sl = a.scale_log2;

  // First unit of the range: the largest u with s_prefix[u] <= block of y0.
  int u = 0;
  {
    int lo = 0, hi = U;  // s_prefix[lo] << tsh <= y0 < s_prefix[hi] << tsh
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((s_prefix[mid] << tsh) <= y0) lo = mid; else hi = mid;
    }
    u = __builtin_amdgcn_readfirstlane(lo);
  }

  int y = y0;
  while (y < y1) {
    while ((__builtin_amdgcn_readfirstlane(s_prefix[u + 1]) << tsh) <= y) ++u;
    const int Yu = __builtin_amdgcn_readfirstlane(s_prefix[u]) << tsh;
    const int ye = min(y1, __builtin_amdgcn_readfirstlane(s_prefix[u + 1]) << tsh);
    const int b = u / Hkv, g = u - b * Hkv;
    const int L = __builtin_amdgcn_readfirstlane(s_len[u]);

    // Per-lane descriptors of 64 consecutive kept blocks (slots) of unit u.
    int cs = -(1 << 30), ci_nv = 0, ci_j = 0;
    int64_t ci_off = 0;
    auto load_chunk = [&](int slot0) {
      cs = slot0;
      const int slot = slot0 + lane;
      int nv = 0, jj = 0;
      int64_t off = 0;
      if (slot < s_prefix[u + 1] - s_prefix[u]) {
        int j;
        if constexpr (GATED) j = s_ids[s_prefix[u] - ids_base + slot];
        else j = sparse ? a.sel_idx[(int64_t)u * a.k_max + slot] : slot;
        if (j >= 0 && j < NB && (int64_t)j * S < L) {
          nv = min(S, L - j * S);
          jj = j;
          if (a.page_table) {
            const int pg = a.page_table[(int64_t)b * NB + j];
            if (pg >= 0 && pg < a.num_pages) off = ((int64_t)pg * Hkv + g) * S * D;
            else nv = 0;
          } else {
            off = (((int64_t)b * Hkv + g) * NB + j) * (int64_t)S * D;
          }
        }
      }
      ci_nv = nv;
      ci_j = jj;
      ci_off = off;
    };
    // Tile yt: valid tokens (by length), element offset of its rows, and the
    // position of its first token.  Empty tiles re-read their block's last
    // valid tile (in bounds, masked).
    auto describe = [&](int yt, int& tv, int64_t& row0, int& tp0) {
      const int rel = yt - Yu;
      const int slot = rel >> tsh;
      const int tib = rel - (slot << tsh);
      const int li = slot - cs;
      const int nv = readlane_i(ci_nv, li);
      const int j = readlane_i(ci_j, li);
      const int64_t off = readlane64(ci_off, li);
      tv = min(kTile, max(0, nv - tib * kTile));
      const int tl = nv > 0 ? min(tib, (nv - 1) / kTile) : 0;
      row0 = off + (int64_t)tl * kTile * D;
      tp0 = j * S + tib * kTile;
    };

    // Query rows as the MFMA A operand: row n16 = token n16 / G, head n16 % G;
    // rows n16 >= R are zero (their loads are clamped and in bounds).
    uint4 qa[NKL];
    {
      const int rq = min(n16, R - 1), tq = rq / G, hq = rq - tq * G;
      const char* qr = (const char*)a.q +
                       (((int64_t)b * TQ + tq) * a.Hq + (int64_t)g * G + hq) * ROWB + r16 * 16;
#pragma unroll
      for (int c = 0; c < NKL; ++c) {
        const uint4 z = *(const uint4*)(qr + c * 64);
        qa[c] = n16 < R ? z : make_uint4(0, 0, 0, 0);
      }
    }
    // This lane's softmax rows 4 r16 + i: the causal limit of their token
    // (keys at positions < lim are visible); rows past R see nothing.
    int lim[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * r16 + i;
      lim[i] = row < R ? L - TQ + 1 + row / G : 0;
    }
    float m_run[4], l_run[4];
    f32x4 acc[DPL];
#pragma unroll
    for (int i = 0; i < 4; ++i) { m_run[i] = kNegInf; l_run[i] = 0.f; }
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Token of MFMA column n16 in 16-token column ct (any assignment gives the
    // same logits; MPV pairs each lane's two tokens for whole-word LDS writes).
    auto tok = [&](int ct) { return MPV ? 2 * n16 + ct : ct * 16 + n16; };
    uint4 kr[kCols][NKL];
    uint4 vr[8][NVQ];  // token 4k + r16 (MPV: 8 r16 + k) of the tile, bytes n16 * VB ..
    auto issue_k = [&](int64_t row0) {
      const char* kb = kbase + row0 * EB;
#pragma unroll
      for (int ct = 0; ct < kCols; ++ct)
#pragma unroll
        for (int c = 0; c < NKL; ++c)
          kr[ct][c] = *(const uint4*)(kb + tok(ct) * ROWB + c * 64 + r16 * 16);
    };
    auto issue_v = [&](int64_t row0) {
      const char* vb = vbase + row0 * EB;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const char* src = vb + (MPV ? 8 * r16 + k : 4 * k + r16) * ROWB + n16 * VB;
        if constexpr (VB == 8) {
          const uint2 h = *(const uint2*)src;
          vr[k][0] = make_uint4(h.x, h.y, 0u, 0u);
        } else {
#pragma unroll
          for (int c = 0; c < NVQ; ++c) vr[k][c] = *(const uint4*)(src + 16 * c);
        }
      }
    };

    auto qk = [&](f32x4 (&sc)[kCols]) {
#pragma unroll
      for (int ct = 0; ct < kCols; ++ct) sc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NKL; ++c) {
#pragma unroll
        for (int ct = 0; ct < kCols; ++ct) {
          if constexpr (EB == 2) {
            sc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[c]),
                                                             __builtin_bit_cast(bf16x8, kr[ct][c]),
                                                             sc[ct], 0, 0, 0);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(chunk_elem<float>(qa[c], e),
                                                            chunk_elem<float>(kr[ct][c], e),
                                                            sc[ct], 0, 0, 0);
          }
        }
      }
    };

    // Online softmax of the lane's rows 4 r16 + i over the tile's tokens
    // tok(ct); p to LDS (fp32 as [token][row], or split in bf16 parts for
    // MPV); acc rows rescaled.
    auto softmax = [&](const f32x4 (&sc)[kCols], int tv, int tp0) {
      float x[kCols][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tvr = min(tv, max(0, lim[i] - tp0));
        float mx = kNegInf;
#pragma unroll
        for (int ct = 0; ct < kCols; ++ct) {
          x[ct][i] = (tok(ct) < tvr) ? sc[ct][i] * sl : kNegInf;
          mx = fmaxf(mx, x[ct][i]);
        }
        mx = row_max16(mx);
        const float mn = fmaxf(m_run[i], mx);
        const float mu = (mn == kNegInf) ? 0.f : mn;
        // Arguments are <= 0 (or -inf): the hardware exp2 is accurate there.
        const float alpha = __builtin_amdgcn_exp2f(m_run[i] - mu);
        float ps = 0.f;
#pragma unroll
        for (int ct = 0; ct < kCols; ++ct) {
          x[ct][i] = __builtin_amdgcn_exp2f(x[ct][i] - mu);
          ps += x[ct][i];
        }
        l_run[i] = l_run[i] * alpha + ps;
        m_run[i] = mn;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e][i] *= alpha;
      }
      if constexpr (MPV) {
        store_p_split((uint32_t*)pw, x, r16, n16);
      } else {
#pragma unroll
        for (int ct = 0; ct < kCols; ++ct)
          *(float4*)(pw + (ct * 16 + n16) * kRows + r16 * 4) =
              make_float4(x[ct][0], x[ct][1], x[ct][2], x[ct][3]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // O += P V: MPV on bf16 matrix cores (pv_bf16; acc[e] is its oacc[e]);
    // else on fp32 MFMA, k-step k taking tokens 4k .. 4k + 3 (lane row group
    // r16 = token 4k + r16).  V rows past the length are zeroed (they may hold
    // anything, even NaN).
    auto pv = [&](int tv) {
      if constexpr (MPV) {
        uint4 v8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v8[k] = vr[k][0];
        pv_bf16((const uint32_t*)pw, v8, tv, acc, r16, n16);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        return;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float ap = pw[(4 * k + r16) * kRows + n16];
        const bool live = 4 * k + r16 < tv;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
          const float bv = live ? v_elem<T, NVQ>(vr[k], e) : 0.f;
          acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(ap, bv, acc[e], 0, 0, 0);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    };

    while (y < ye) {
      const int slot0 = (y - Yu) >> tsh;
      load_chunk(slot0);
      const int yc = min(ye, Yu + ((slot0 + kWave) << tsh));
      int tv, tp0;
      int64_t row0;
      describe(y, tv, row0, tp0);
      issue_k(row0);
      issue_v(row0);
      for (; y < yc; ++y) {
        int tv_n, tp_n;
        int64_t row_n;
        describe(min(y + 1, yc - 1), tv_n, row_n, tp_n);
        f32x4 sc[kCols];
        qk(sc);
        __builtin_amdgcn_sched_barrier(0);
        issue_k(row_n);
        softmax(sc, tv, tp0);
        pv(tv);
        __builtin_amdgcn_sched_barrier(0);
        issue_v(row_n);
        tv = tv_n;
        tp0 = tp_n;
      }
      y = yc;
    }

    // ---- segment result: partial record (u, w) at slot u + w, all 16 rows ----
    float lt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lt[i] = row_sum16(l_run[i]);
    float* rec = a.part + (int64_t)(u + w) * REC;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* dst = rec + (4 * r16 + i) * D + n16 * DPL;
#pragma unroll
      for (int e = 0; e < DPL; e += 4)
        *(float4*)(dst + e) = make_float4(acc[e][i], acc[e + 1][i], acc[e + 2][i], acc[e + 3][i]);
    }
    if (n16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rec[kRows * D + 4 * r16 + i] = m_run[i];
        rec[kRows * D + kRows + 4 * r16 + i] = lt[i];
      }
    }
  }
  write_late();
}

// Merges a unit's records for one query row (token t = row / G, head
// g*G + row % G) per workgroup, one thread per dimension.  Up to 32 records:
// every value loaded up front, then the maximum M of the records' maxima and
// the scaled sums in record (wave) order,
//   o = sum_w acc_w 2^(m_w - M),  l = sum_w l_w 2^(m_w - M),  out = o / l,
// lse = (M + log2 l) ln 2.  More records: the same merge with a running
// maximum.  Empty waves and records without a valid token are skipped; the
// order is fixed, so the result is deterministic.
template <int D, int NWB>
__device__ __forceinline__ void multi_shot(const CombineArgs& a, const float* part, int nw,
                                           int wlo, int W, int Tot, int row, int64_t oidx) {
  constexpr int REC = MGeo<float, D>::REC;
  const int dim = threadIdx.x;
  float x[NWB], mv[NWB], lv[NWB];
#pragma unroll
  for (int t = 0; t < NWB; ++t) {
    const float* r = part + (int64_t)min(t, nw - 1) * REC;  // past nw: re-read, unused
    x[t] = r[row * D + dim];
    mv[t] = r[kRows * D + row];
    lv[t] = r[kRows * D + kRows + row];
  }
  uint32_t skip = 0;
  if (Tot < W) {
    const EqualSplit sp(Tot, W);
    for (int t = 0; t < nw; ++t) skip |= wave_empty(sp, wlo + t) ? (1u << t) : 0u;
  }
  float M = kNegInf;
#pragma unroll
  for (int t = 0; t < NWB; ++t) M = (t < nw && !((skip >> t) & 1u)) ? fmaxf(M, mv[t]) : M;
  float o = 0.f, l = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int t = 0; t < NWB; ++t) {
      const bool use = t < nw && !((skip >> t) & 1u) && mv[t] != kNegInf;
      const float sc = __builtin_amdgcn_exp2f(mv[t] - M);  // argument <= 0
      o = use ? fmaf(x[t], sc, o) : o;
      l = use ? fmaf(lv[t], sc, l) : l;
    }
  }
  a.out[oidx * D + dim] = l > 0.f ? o / l : 0.f;
  if (a.lse && dim == 0) a.lse[oidx] = l > 0.f ? (M + log2f(l)) * 0.69314718055994530942f : kNegInf;
}

template <int D>
__global__ __launch_bounds__(D) void decode_multi_combine_kernel(CombineArgs a) {
  constexpr int REC = MGeo<float, D>::REC;
  const int u = blockIdx.x, row = blockIdx.y, dim = threadIdx.x;
  const int U = a.B * a.Hkv, TQ = a.tokens, G = a.Hq / a.Hkv, R = G * TQ;
  if (row >= R) return;
  const int tsh = 31 - __builtin_clz(a.S / kTile);
  const int W = a.hdr[0];
  const int Tot = a.prefix[U] << tsh;
  const int ylo = a.prefix[u] << tsh, yhi = a.prefix[u + 1] << tsh;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int tq = row / G, hq = row - tq * G;
  const int64_t oidx = ((int64_t)b * TQ + tq) * a.Hq + (int64_t)g * G + hq;
  if (yhi <= ylo) {  // no tokens: out = 0, lse = -inf
    a.out[oidx * D + dim] = 0.f;
    if (a.lse && dim == 0) a.lse[oidx] = kNegInf;
    return;
  }
  const int wlo = tile_owner(ylo, W, Tot), whi = tile_owner(yhi - 1, W, Tot);
  const int nw = whi - wlo + 1;
  const float* part = a.part + (int64_t)(u + wlo) * REC;
  if (nw <= 8) return multi_shot<D, 8>(a, part, nw, wlo, W, Tot, row, oidx);
  if (nw <= 16) return multi_shot<D, 16>(a, part, nw, wlo, W, Tot, row, oidx);
  if (nw <= 32) return multi_shot<D, 32>(a, part, nw, wlo, W, Tot, row, oidx);
  const EqualSplit sp(Tot, W);
  float M = kNegInf, l = 0.f, o = 0.f;
  for (int t = 0; t < nw; ++t) {
    if (Tot < W && wave_empty(sp, wlo + t)) continue;  // wrote no record
    const float* r = part + (int64_t)t * REC;
    const float mw = r[kRows * D + row];
    if (mw == kNegInf) continue;                        // no valid token in it
    const float mn = fmaxf(M, mw);
    const float sa = __builtin_amdgcn_exp2f(M - mn), sb = __builtin_amdgcn_exp2f(mw - mn);
    o = o * sa + r[row * D + dim] * sb;
    l = l * sa + r[kRows * D + kRows + row] * sb;
    M = mn;
  }
  a.out[oidx * D + dim] = l > 0.f ? o / l : 0.f;
  if (a.lse && dim == 0) a.lse[oidx] = l > 0.f ? (M + log2f(l)) * 0.69314718055994530942f : kNegInf;
}

template <typename T, int D, bool GATED>
const void* multi_fn() { return (const void*)&decode_multi_kernel<T, D, GATED>; }

template <bool GATED>
const void* multi_kernel(int dtype, int D) {
  if (dtype == 1)
    return D == 64 ? multi_fn<uint16_t, 64, GATED>() : multi_fn<uint16_t, 128, GATED>();
  return D == 64 ? multi_fn<float, 64, GATED>() : multi_fn<float, 128, GATED>();
}

}  // namespace

size_t decode_multi_workspace_bytes(int B, int Hkv, int D, int wmax) {
  const int U = B * Hkv;
  return decode_part_offset(U) + (size_t)(U + wmax) * (kRows * D + 2 * kRows) * sizeof(float);
}

hipError_t launch_decode_multi(const DecodeArgs& a, hipStream_t stream) {
  const int U = a.B * a.Hkv;
  DecodeArgs args = a;
  void* params[] = {&args};
  const size_t smem = (size_t)(2 * U + 1 + kWavesPerWG + 1) * sizeof(int);
  return hipLaunchKernel(multi_kernel<false>(a.dtype, a.D), dim3(a.W / kWavesPerWG),
                         dim3(kThreads), params, smem, stream);
}

hipError_t launch_gated_decode_multi(const DecodeArgs& a, hipStream_t stream) {
  const int U = a.B * a.Hkv;
  DecodeArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(multi_kernel<true>(a.dtype, a.D), dim3(a.W / kWavesPerWG),
                         dim3(kThreads), params, gated_decode_smem_bytes(U, a.NB, a.ids_cap),
                         stream);
}

size_t gated_decode_multi_static_smem(int dtype, int D) {
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, multi_kernel<true>(dtype, D)) != hipSuccess) return (size_t)-1;
  return attr.sharedSizeBytes;
}

hipError_t launch_decode_multi_combine(const CombineArgs& a, hipStream_t stream) {
  CombineArgs args = a;
  void* params[] = {&args};
  const void* fn = a.D == 64 ? (const void*)&decode_multi_combine_kernel<64>
                             : (const void*)&decode_multi_combine_kernel<128>;
  return hipLaunchKernel(fn, dim3(a.B * a.Hkv, kRows), dim3(a.D), params, 0, stream);
}

}  // namespace seer
