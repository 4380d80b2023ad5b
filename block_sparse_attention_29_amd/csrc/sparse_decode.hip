// Split-KV block-sparse decode attention for gfx950.
//
// Computes, for every query head h of sequence b (g = h / G its KV head),
// softmax(q_h . k_t * scale) v_t over the valid tokens t of the kept blocks
// only -- the masked attention of "Sparse Attention Reasoning", Step 4, where
// every key outside the kept blocks is -inf -- without touching any other key
// ("SeerAttention-R", Abstract: a sparse decoding kernel whose time follows the
// KV bytes it reads).
//
// Work split.  A "unit" is one (sequence, KV head); its kept blocks are cut
// into 32-token tiles.  The tiles of all units are concatenated (unit-major,
// then kept-block order, then tile) and the W waves of the launch take equal
// contiguous ranges of that list, so every wave streams the same number of KV
// bytes whatever the per-sequence lengths and counts.  A wave keeps one
// online-softmax state per unit segment it covers and writes it as a partial
// record to slot (unit + wave), which is unique because both coordinates only
// grow along the list.  The combine kernel merges a unit's records by
// log-sum-exp in wave order, so the result does not depend on timing.
//
// Per 32-token tile a wave:
//  * loads K as the B operand of v_mfma_f32_16x16x32_bf16 (bf16) or
//    v_mfma_f32_16x16x4_f32 (fp32): lane (r, n), r = lane/16, n = lane%16,
//    holds 16 bytes of token n's row at byte offset c*64 + r*16 for load c.
//    The query group is the A operand with the same lane mapping (head n, zero
//    rows for n >= G), so both operands share one k-index assignment and the
//    product is q . k whatever order the unit uses internally.  The 16x16
//    result holds logit (head 4*r + i, token n) in lane (r, n), register i.
//  * takes the tile max per head with DPP row reductions, rescales, and
//    writes exp2 probabilities to a 2 KiB LDS buffer per wave;
//  * streams V rows fully coalesced (16 bytes per lane, whole rows per
//    instruction) and multiplies:
//    - bf16, d = 128: on the matrix cores, v_mfma_f32_16x16x32_bf16 with the
//      tile's 32 tokens as k.  Each probability is split into two bf16 parts
//      (p = hi + lo to 16 significant bits; the products are exact and summed
//      in fp32), written to LDS as [head][token] and read back as the A
//      operand; lane (r, n) loads tokens 8r .. 8r + 7 at dimensions 8n ..
//      8n + 7, so the B operand of dimension step e is the e-th element of
//      its 8 chunks, packed in pairs.  The accumulators hold O[head][dim]
//      directly (no cross-lane sum at the end), in fp32.
//    - fp32 or d = 64: fp32 FMAs on the VALU, probabilities in fp32.
// The K registers are refilled with the next tile right after the QK product
// and the V registers right after the PV product, so each wave keeps about one
// tile of loads in flight while it computes.
#include <atomic>
#include <type_traits>

#include "decode_common.h"
#include "gate_phase.h"
#include "select_device.h"

namespace seer {
namespace {

// GIVEN (with GATED): the units' scores come from a.scores_in (the gate's
// score kernel ran first); the workgroups only select.
template <typename T, int D, int G, bool GATED, bool GIVEN = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_partial_kernel(DecodeArgs a) {
  static_assert(GATED || !GIVEN, "given scores need the gate phase");
  using GE = Geo<T, D>;
  constexpr int EB = GE::EB, ROWB = GE::ROWB, E = GE::E, NKL = GE::NKL;
  constexpr int LPR = GE::LPR, RPI = GE::RPI, NVL = GE::NVL;
  constexpr int REC = G * D + 16;  // partial record: acc[G][D], m[8], l[8] (floats)
  // bf16 caches with d = 128 multiply P V on the matrix cores (MPV); other
  // caches on the VALU.
  constexpr bool MPV = EB == 2 && D == 128;
  static_assert(!MPV || NVL == 8, "MPV: one 16-byte V chunk per lane and token row");

  __shared__ __align__(16) float s_p[kWavesPerWG][kTile * 16];
  extern __shared__ int s_dyn[];

  const int U = a.B * a.Hkv;
  const int tid = threadIdx.x;
  int* s_prefix = s_dyn;                      // [U + 1]
  int* s_scan = s_dyn + U + 1;                // [kWavesPerWG + 1]
  int* s_len = s_dyn + U + 1 + kWavesPerWG + 1;  // [U] sequence length of each unit

  const int lane = tid & 63, wv = tid >> 6;
  const int r16 = lane >> 4, n16 = lane & 15;
  // Workgroups are dealt to the XCDs round-robin (workgroup i runs on XCD
  // i % 8), each XCD with its own L2.  Consecutive tile ranges go to the
  // workgroups of one XCD, so the workgroups that share a unit mostly share an
  // L2 (its pooled table, read by each of them in the fused gate, comes from
  // HBM once).  Any other placement is still correct.
  const int nwg = (int)gridDim.x;
  const int wg = (nwg % kXcds == 0)
      ? (int)(blockIdx.x % kXcds) * (nwg / kXcds) + (int)(blockIdx.x / kXcds)
      : (int)blockIdx.x;
  const int wg0 = wg * kWavesPerWG;

  GatePreload<T, D, G> pre;  // the fused gate's entry loads
  pre.u = -1;

  // ---- plan: block prefix over units (every workgroup computes the same) ----
  {
    const int per = (U + kThreads - 1) / kThreads;
    const int u_lo = min(U, tid * per), u_hi = min(U, u_lo + per);
    // The loads of the thread's first unit go out first, the gate's entry
    // loads after them, so the plan waits for its own loads only.
    const int u_f = min(u_lo, U - 1);
    const int L_f = a.lens[u_f / a.Hkv];
    const int aux_f = unit_aux<GATED>(a, u_f);
    // (wg0 * U < 2^31: fewer than 2^15 waves, at most 2^13 units)
    if constexpr (GATED)
      issue_gate_preload<T, D, G, false, GIVEN>(a, (int)((uint32_t)(wg0 * U) / (uint32_t)a.W), pre);
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

  // The wave index is uniform per wave; say so, so that everything derived
  // from it (the tile range, the loop counters) lives in scalar registers.
  const int w = __builtin_amdgcn_readfirstlane(wg * kWavesPerWG + wv);
  // Tile coordinates fit in 32 bits: units * blocks * tiles per block < 2^31.
  const int tsh = 31 - __builtin_clz(a.S / kTile);  // log2(tiles per block)
  const int Tot = __builtin_amdgcn_readfirstlane(s_prefix[U]) << tsh;
  const EqualSplit split(Tot, a.W);  // wave w's tiles: [split.start(w), split.start(w + 1))

  // ---- units holding the first tile of each wave of this workgroup and the
  // workgroup's last tile, looked up by all threads at once (one pass over
  // the units instead of a serial binary search per wave) ----
  __shared__ int s_unit[kWavesPerWG + 1];
  {
    int xq[kWavesPerWG + 1];  // block index of each query tile
#pragma unroll
    for (int v = 0; v < kWavesPerWG; ++v) xq[v] = split.start(wg0 + v) >> tsh;
    xq[kWavesPerWG] = (split.start(wg0 + kWavesPerWG) - 1) >> tsh;
    for (int uu = tid; uu < U; uu += kThreads) {
      const int lo = s_prefix[uu], hi = s_prefix[uu + 1];
#pragma unroll
      for (int v = 0; v <= kWavesPerWG; ++v)
        if (lo <= xq[v] && xq[v] < hi) s_unit[v] = uu;
    }
    __syncthreads();
  }

  // ---- fused gate: the selections of every unit this workgroup streams, into
  // LDS (each workgroup selects on its own; a unit shared by workgroups is
  // selected by each of them, bit-identically) ----
  int32_t* s_ids = s_len + U;  // [ids_cap] kept ids of this workgroup's units, slot - ids_base
  int ids_base = 0;
  // The scores of the unit gated last stay in s_key (LDS) to the end.
  uint64_t* s_key = (uint64_t*)(((uintptr_t)(s_ids + a.ids_cap) + 7) & ~(uintptr_t)7);
  // The unit whose selection this workgroup writes out after its tiles (-1:
  // none).  Stores share the one memory counter with loads, so outputs still in
  // flight when the first tile is requested would hold its QK^T back until
  // they are acknowledged; written at the end they cost nothing.  Only the
  // last unit gated can wait: the next unit's gate reuses s_key.
  int late_u = -1;
  if constexpr (GATED) {
    __shared__ double s_q[D];
    __shared__ double s_part[4 * 256];  // quarter sums of one pass (4 x 64*VEC)
    __shared__ int s_hist[3 * 256];
    __shared__ int s_sel_scan[kWavesPerWG + 1];
    const int Y0 = split.start(wg0);
    const int Y1 = split.start(wg0 + kWavesPerWG);
    if (Y0 < Y1) {
      const int u0 = s_unit[0], u1 = s_unit[kWavesPerWG];
      ids_base = s_prefix[u0];
      auto gate = [&](int u, auto pre_tag) {
        const int k = s_prefix[u + 1] - s_prefix[u];
        if (k == 0) return;
        // the owner holds the unit's first tile
        const int owner = tile_owner((int64_t)s_prefix[u] << tsh, a.W, Tot) / kWavesPerWG;
        const bool late = owner == wg && u == u1;
        if (late) late_u = u;
        fused_gate_unit<T, D, G, false, decltype(pre_tag)::value, GIVEN>(
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
      fused_gate_write<GIVEN>(a, late_u, seq_blocks(s_len[late_u], a.S, a.NB),
                       s_prefix[late_u + 1] - s_prefix[late_u],
                       s_ids + (s_prefix[late_u] - ids_base), s_key);
  };
  const int y0 = split.start(w);
  const int y1 = split.start(w + 1);
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

  // First unit of the range: largest u with s_prefix[u] <= block of y0.
  int u = __builtin_amdgcn_readfirstlane(s_unit[wv]);

  int y = y0;
  while (y < y1) {
    // ---- one segment: the tiles of unit u inside [y, y1) ----
    while ((__builtin_amdgcn_readfirstlane(s_prefix[u + 1]) << tsh) <= y) ++u;  // skips units without blocks
    const int Yu = __builtin_amdgcn_readfirstlane(s_prefix[u]) << tsh;
    const int ye = min(y1, __builtin_amdgcn_readfirstlane(s_prefix[u + 1]) << tsh);
    const int b = u / Hkv, g = u - b * Hkv;
    const int L = __builtin_amdgcn_readfirstlane(s_len[u]);

    // Per-lane descriptors of 64 consecutive kept blocks (slots) of unit u.
    int cs = -(1 << 30);
    int ci_nv = 0;
    int64_t ci_off = 0;
    auto load_chunk = [&](int slot0) {
      cs = slot0;
      const int slot = slot0 + lane;
      int nv = 0;
      int64_t off = 0;
      if (slot < s_prefix[u + 1] - s_prefix[u]) {
        int j;
        if constexpr (GATED) j = s_ids[s_prefix[u] - ids_base + slot];
        else j = sparse ? a.sel_idx[(int64_t)u * a.k_max + slot] : slot;
        if (j >= 0 && j < NB && (int64_t)j * S < L) {
          nv = min(S, L - j * S);
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
      ci_off = off;
    };
    // Tile t of the segment: valid tokens and the element offset of the rows to
    // load.  Empty tiles re-read their block's last valid tile (in bounds).
    auto describe = [&](int yt, int& tv, int64_t& row0) {
      const int rel = yt - Yu;
      const int slot = rel >> tsh;
      const int tib = rel - (slot << tsh);
      const int li = slot - cs;  // within the loaded chunk by construction
      const int nv = readlane_i(ci_nv, li);
      const int64_t off = readlane64(ci_off, li);
      tv = min(kTile, max(0, nv - tib * kTile));
      const int tl = nv > 0 ? min(tib, (nv - 1) / kTile) : 0;
      row0 = off + (int64_t)tl * kTile * D;
    };

    // Unit state: the query group as the MFMA A operand, softmax state, acc.
    uint4 qa[NKL];
    {
      const char* qb = (const char*)a.q + ((int64_t)b * a.Hq + (int64_t)g * G) * ROWB;
      // Rows n16 >= G of the A operand are zero; their (clamped, in-bounds)
      // loads are issued anyway so that no load sits behind a branch.
      const bool qrow = n16 < G;
      const char* qr = qb + min(n16, G - 1) * ROWB + r16 * 16;
#pragma unroll
      for (int c = 0; c < NKL; ++c) {
        const uint4 z = *(const uint4*)(qr + c * 64);
        qa[c] = qrow ? z : make_uint4(0, 0, 0, 0);
      }
    }
    float m_run[4], l_run[4];
    float acc[MPV ? 1 : G][MPV ? 1 : E];  // VALU: (head, element of the lane's V chunk)
    f32x4 oacc[MPV ? 8 : 1];              // MPV: dimension step e (see pv)
#pragma unroll
    for (int i = 0; i < 4; ++i) { m_run[i] = kNegInf; l_run[i] = 0.f; }
#pragma unroll
    for (int h = 0; h < (MPV ? 1 : G); ++h)
#pragma unroll
      for (int e = 0; e < (MPV ? 1 : E); ++e) acc[h][e] = 0.f;
#pragma unroll
    for (int e = 0; e < (MPV ? 8 : 1); ++e) oacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Token of MFMA column n16 in the tile's 16-token column ct.  Any
    // assignment gives the same logits; MPV pairs each lane's two tokens
    // (2 n16, 2 n16 + 1) so that its probabilities go to LDS as whole words.
    auto tok = [&](int ct) { return MPV ? 2 * n16 + ct : ct * 16 + n16; };

    uint4 kr[kCols][NKL];
    uint4 vr[NVL];
    auto issue_k = [&](int64_t row0) {
      const char* kb = kbase + row0 * EB;
#pragma unroll
      for (int ct = 0; ct < kCols; ++ct)
#pragma unroll
        for (int c = 0; c < NKL; ++c)
          kr[ct][c] = *(const uint4*)(kb + tok(ct) * ROWB + c * 64 + r16 * 16);
    };
    // VALU: chunk rr holds token rr * RPI + lane / LPR, bytes (lane % LPR) * 16..
    // MPV: chunk j holds token 8 * r16 + j, dimensions 8 * n16 .. 8 * n16 + 7.
    // Either way each load instruction reads whole token rows.
    auto issue_v = [&](int64_t row0) {
      const char* vb = vbase + row0 * EB;
#pragma unroll
      for (int rr = 0; rr < NVL; ++rr)
        vr[rr] = MPV ? *(const uint4*)(vb + (8 * r16 + rr) * ROWB + n16 * 16)
                     : *(const uint4*)(vb + (rr * RPI + lane / LPR) * ROWB + (lane % LPR) * 16);
    };

    // S = Q K^T for the tile's two 16-token columns.
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

    // Online softmax (log2 domain).  Lane (r16, n16) register i holds head
    // 4*r16 + i at tokens n16 and 16 + n16.  Publishes p to LDS and rescales acc.
    auto softmax = [&](const f32x4 (&sc)[kCols], int tv) {
      float x[kCols][4], alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = kNegInf;
#pragma unroll
        for (int ct = 0; ct < kCols; ++ct) {
          x[ct][i] = (tok(ct) < tv) ? sc[ct][i] * sl : kNegInf;
          mx = fmaxf(mx, x[ct][i]);
        }
        mx = row_max16(mx);
        const float mn = fmaxf(m_run[i], mx);
        const float mu = (mn == kNegInf) ? 0.f : mn;
        // Arguments are <= 0 (or -inf): the hardware exp2 is accurate there.
        alpha[i] = __builtin_amdgcn_exp2f(m_run[i] - mu);
        float ps = 0.f;
#pragma unroll
        for (int ct = 0; ct < kCols; ++ct) {
          x[ct][i] = __builtin_amdgcn_exp2f(x[ct][i] - mu);
          ps += x[ct][i];
        }
        l_run[i] = l_run[i] * alpha[i] + ps;
        m_run[i] = mn;
      }
      if constexpr (MPV) {
        store_p_split((uint32_t*)pw, x, r16, n16);
        // Rescale (row 4 r16 + i of every accumulator is head 4 r16 + i).
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[e][i] *= alpha[i];
      } else {
        // Every lane writes (rows of heads >= G are never read): no branch.
#pragma unroll
        for (int ct = 0; ct < kCols; ++ct)
          *(float4*)(pw + (ct * 16 + n16) * 16 + r16 * 4) =
              make_float4(x[ct][0], x[ct][1], x[ct][2], x[ct][3]);
        // Rescale acc (alpha is exactly 1 for a head whose max did not move).
        // Unconditional: a branch here splits acc's live range into copies.
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ah = readlane_f(alpha[h & 3], (h >> 2) * 16);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] *= ah;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // O += P V with V rows streamed row-major, p from LDS, fp32 FMAs.  One row
    // step at a time (its p read one step ahead) keeps the temporaries small.
    auto read_p = [&](int rr, float (&pr)[G]) {
      const int trow = rr * RPI + lane / LPR;
      const float4 plo = *(const float4*)(pw + trow * 16);
      float4 phi = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (G > 4) phi = *(const float4*)(pw + trow * 16 + 4);
      const float all[8] = {plo.x, plo.y, plo.z, plo.w, phi.x, phi.y, phi.z, phi.w};
#pragma unroll
      for (int h = 0; h < G; ++h) pr[h] = all[h];
    };
    auto pv = [&](int tv) {
      if constexpr (MPV) {
        pv_bf16((const uint32_t*)pw, vr, tv, oacc, r16, n16);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
      } else {
        float pn[G];
        read_p(0, pn);
#pragma unroll
        for (int rr = 0; rr < NVL; ++rr) {
          float pc[G];
#pragma unroll
          for (int h = 0; h < G; ++h) pc[h] = pn[h];
          if (rr + 1 < NVL) read_p(rr + 1, pn);
          const int trow = rr * RPI + lane / LPR;
          // Rows past the length may hold anything (even NaN): zero them.
          const bool live = trow < tv;
          uint4 vv = vr[rr];
          vv.x = live ? vv.x : 0u;
          vv.y = live ? vv.y : 0u;
          vv.z = live ? vv.z : 0u;
          vv.w = live ? vv.w : 0u;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float ve = chunk_elem<T>(vv, e);
#pragma unroll
            for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pc[h], ve, acc[h][e]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    };

    // ---- tiles: K and V each re-issued as soon as their registers are consumed.
    // The segment is walked in chunks of at most 64 kept blocks, one block
    // descriptor per lane, so the steady-state loop has no branches.
    while (y < ye) {
      const int slot0 = (y - Yu) >> tsh;
      load_chunk(slot0);
      const int yc = min(ye, Yu + ((slot0 + kWave) << tsh));
      int tv;
      int64_t row0;
      describe(y, tv, row0);
      issue_k(row0);
      issue_v(row0);
      for (; y < yc; ++y) {
        // The last tile prefetches itself again (in bounds, cache-hot, unused).
        int tv_n;
        int64_t row_n;
        describe(min(y + 1, yc - 1), tv_n, row_n);
        f32x4 sc[kCols];
        qk(sc);
        __builtin_amdgcn_sched_barrier(0);
        issue_k(row_n);
        softmax(sc, tv);
        pv(tv);
        __builtin_amdgcn_sched_barrier(0);
        issue_v(row_n);
        tv = tv_n;
      }
      y = yc;
    }

    // ---- segment result: partial record (u, w) at slot u + w ----
    float lt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lt[i] = row_sum16(l_run[i]);
    float* rec = a.part + (int64_t)(u + w) * REC;
    if constexpr (MPV) {
      // lane (r16, n16): heads 4 r16 + i, dimensions 8 n16 .. 8 n16 + 7
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * r16 + i;
        if (h < G) {
          float* o = rec + h * D + 8 * n16;
          *(float4*)o = make_float4(oacc[0][i], oacc[1][i], oacc[2][i], oacc[3][i]);
          *(float4*)(o + 4) = make_float4(oacc[4][i], oacc[5][i], oacc[6][i], oacc[7][i]);
        }
      }
    }
    if constexpr (!MPV) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          // the lanes holding the same V columns: i, i ^ 8 (8 lanes per row),
          // then the other rows (VALU swaps, no LDS round trip)
          float x = acc[h][e];
          if constexpr (LPR == 8) x = x + dpp_f32<kDppRowRor8>(x);
          if constexpr (LPR <= 16) x = cross_row_sum_f32(x);
          else x = cross_half_sum_f32(x);
          acc[h][e] = x;
        }
      if (lane < LPR) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < E; e += 4)
            *(float4*)(rec + h * D + lane * E + e) =
                make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
      }
    }
    if (n16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = r16 * 4 + i;
        if (h < G) {
          rec[G * D + h] = m_run[i];
          rec[G * D + 8 + h] = lt[i];
        }
      }
    }
  }
  write_late();
}


// Merges the partial records of one unit per workgroup, in wave order.
//
// The waves that wrote a record for unit u are the non-empty waves among
// [wlo, whi], the first and last waves whose tile ranges meet the unit's
// tiles.  The merge: the maximum M of the used records' maxima, then
//   o = sum_w acc_w 2^(m_w - M),  l = sum_w l_w 2^(m_w - M)
// as fma chains in record order, out = o / l, lse = M + log2(l) (natural log
// on output).  Up to 32 records it runs in one shot (every load up front);
// beyond, over chunks of kHeadChunk records, each folded into a running
// maximum.  The order is fixed, so the result is deterministic, and the
// per-head kernel below runs the same schedule operation for operation, so
// the two give identical bits.
constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 16;   // acc loads in flight per thread (general path)
constexpr int kCombineFast = 32;    // units with at most this many records: one-shot path
constexpr int kHeadChunk = 64;      // records per chunk of the running merge (both kernels)

// One-shot merge of a unit with at most NWB records: thread tid owns the EPT
// consecutive elements tid*EPT.. of one head (EPT a power of two, so it
// divides D) and loads every value it needs from every record before any use.
// Two passes: the maximum M of the records' maxima, then the sums
//   o = sum_w acc_w 2^(m_w - M),  l = sum_w l_w 2^(m_w - M)
// in record order, so the only dependency chain is the fma chain.
template <int D, int G, int NWB>
__device__ __forceinline__ void combine_shot(const CombineArgs& a, const float* part, int nw,
                                             int wlo, int W, int Tot, int64_t head0) {
  constexpr int REC = G * D + 16;
  constexpr int EPT = G * D <= kCombineThreads ? 1 : G * D <= 2 * kCombineThreads ? 2 : 4;
  const int tid = threadIdx.x;
  if (tid * EPT >= G * D) return;
  const int idx0 = tid * EPT, h = idx0 / D;
  float x[NWB][EPT], mv[NWB], lv[NWB];
#pragma unroll
  for (int t = 0; t < NWB; ++t) {
    const float* r = part + (int64_t)min(t, nw - 1) * REC;  // past nw: re-read, unused
#pragma unroll
    for (int e = 0; e < EPT; ++e) x[t][e] = r[idx0 + e];
    mv[t] = r[G * D + h];
    lv[t] = r[G * D + 8 + h];
  }
  // Waves are only ever empty when there are fewer tiles than waves; the
  // divisions that tell are kept out of the merge.
  uint32_t skip = 0;
  if (Tot < W) {
    const EqualSplit sp(Tot, W);
    for (int t = 0; t < nw; ++t) skip |= wave_empty(sp, wlo + t) ? (1u << t) : 0u;
  }
  float M = kNegInf;
#pragma unroll
  for (int t = 0; t < NWB; ++t) {
    const bool use = t < nw && !((skip >> t) & 1u);
    M = use ? fmaxf(M, mv[t]) : M;
  }
  float l = 0.f, o[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) o[e] = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int t = 0; t < NWB; ++t) {
      // Records without a valid token (m = -inf) and skipped slots add nothing;
      // stale slots may hold anything, so they are selected away, not scaled.
      const bool use = t < nw && !((skip >> t) & 1u) && mv[t] != kNegInf;
      // Arguments are <= 0: the hardware exp2 is accurate there.
      const float sc = __builtin_amdgcn_exp2f(mv[t] - M);
#pragma unroll
      for (int e = 0; e < EPT; ++e) o[e] = use ? fmaf(x[t][e], sc, o[e]) : o[e];
      l = use ? fmaf(lv[t], sc, l) : l;
    }
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) a.out[head0 * D + idx0 + e] = l > 0.f ? o[e] / l : 0.f;
  if (a.lse && (idx0 % D) == 0)
    a.lse[head0 + h] = l > 0.f ? (M + log2f(l)) * 0.69314718055994530942f : kNegInf;
}

template <int D, int G>
__global__ __launch_bounds__(kCombineThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void decode_combine_kernel(CombineArgs a) {
  constexpr int REC = G * D + 16;
  constexpr int PER = (G * D + kCombineThreads - 1) / kCombineThreads;
  __shared__ float s_mw[kHeadChunk][G];  // a chunk's record maxima (-inf: empty wave)
  __shared__ float s_lw[kHeadChunk][G];  // and sums

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int U = a.B * a.Hkv;
  const int tsh = 31 - __builtin_clz(a.S / kTile);
  const int W = a.hdr[0];
  const int Tot = a.prefix[U] << tsh;
  const int ylo = a.prefix[u] << tsh, yhi = a.prefix[u + 1] << tsh;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int64_t head0 = (int64_t)b * a.Hq + (int64_t)g * G;
  if (yhi <= ylo) {  // no tokens: out = 0, lse = -inf
    for (int idx = tid; idx < G * D; idx += kCombineThreads) a.out[head0 * D + idx] = 0.f;
    if (a.lse && tid < G) a.lse[head0 + tid] = kNegInf;
    return;
  }
  const int wlo = tile_owner(ylo, W, Tot);
  const int whi = tile_owner(yhi - 1, W, Tot);
  const int nw = whi - wlo + 1;
  const float* part = a.part + (int64_t)(u + wlo) * REC;  // record of wave wlo + t at t * REC
  const EqualSplit sp(Tot, W);
  auto empty = [&](int t) { return wave_empty(sp, wlo + t); };  // wrote no record

  if (nw <= 8) return combine_shot<D, G, 8>(a, part, nw, wlo, W, Tot, head0);
  if (nw <= 16) return combine_shot<D, G, 16>(a, part, nw, wlo, W, Tot, head0);
  if (nw <= kCombineFast) return combine_shot<D, G, kCombineFast>(a, part, nw, wlo, W, Tot, head0);

  // General path (more than 32 records): the per-head kernel's schedule --
  // chunks of kHeadChunk records in order, each merged into the running
  // state by its maximum Mc: M' = max(M, Mc), the state rescaled by
  // 2^(M - M'), then the chunk's values rescaled by 2^(m_w - M') and added as
  // an fma chain in record order.  A chunk's (m, l) are staged through LDS,
  // its values fetched kCombineBatch records at a time.
  float o[PER], M[PER], l[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) { o[r] = 0.f; M[r] = kNegInf; l[r] = 0.f; }
  for (int c0 = 0; c0 < nw; c0 += kHeadChunk) {
    const int cn = min(kHeadChunk, nw - c0);
    if (c0 > 0) __syncthreads();  // the previous chunk's (m, l) fully consumed
    for (int t = tid; t < cn; t += kCombineThreads) {
      const bool e = empty(c0 + t);
      const float* r = part + (int64_t)(c0 + t) * REC;
      float mv[G], lv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) { mv[h] = r[G * D + h]; lv[h] = r[G * D + 8 + h]; }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_mw[t][h] = e ? kNegInf : mv[h];
        s_lw[t][h] = e ? 0.f : lv[h];
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int idx = r * kCombineThreads + tid;
      if (idx >= G * D) continue;
      const int h = idx / D;
      float Mc = kNegInf;
      for (int t = 0; t < cn; ++t) Mc = fmaxf(Mc, s_mw[t][h]);
      if (Mc == kNegInf) continue;  // no valid token in the chunk
      const float Mn = fmaxf(M[r], Mc);
      // Arguments are <= 0 (or -inf, giving 0): the hardware exp2 is accurate there.
      const float sres = __builtin_amdgcn_exp2f(M[r] - Mn);
      o[r] *= sres;
      l[r] *= sres;
      for (int t0 = 0; t0 < cn; t0 += kCombineBatch) {
        const int tn = min(kCombineBatch, cn - t0);
        const float* base = part + (int64_t)(c0 + t0) * REC;  // uniform
        float x[kCombineBatch];
#pragma unroll
        for (int t = 0; t < kCombineBatch; ++t) x[t] = base[min(t, tn - 1) * REC + idx];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kCombineBatch; ++t) {
          const float mw = t < tn ? s_mw[t0 + t][h] : kNegInf;
          // records without a valid token (m = -inf) and empty records add nothing
          const bool use = mw != kNegInf;
          const float sc = __builtin_amdgcn_exp2f(mw - Mn);
          o[r] = use ? fmaf(x[t], sc, o[r]) : o[r];
          l[r] = use ? fmaf(s_lw[t0 + t][h], sc, l[r]) : l[r];
        }
      }
      M[r] = Mn;
    }
  }
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int idx = r * kCombineThreads + tid;
    if (idx >= G * D) continue;
    a.out[head0 * D + idx] = l[r] > 0.f ? o[r] / l[r] : 0.f;
    if (a.lse && (idx % D) == 0)
      a.lse[head0 + idx / D] = l[r] > 0.f ? (M[r] + log2f(l[r])) * 0.69314718055994530942f : kNegInf;
  }
}

// The same merge with one workgroup per query head and one thread per element,
// for units with many records (few, long units): a head's records share their
// (m, l), so each thread loads only its element's values of every record.
// Records are merged in chunks of up to kHeadChunk = 64 (8, 16 or 32 when the
// unit has no more): the chunk's maximum Mc, then its values rescaled by
// 2^(m_w - M') and summed in record order into the running state,
// M' = max(M, Mc), which is rescaled once by 2^(M - M').  The per-unit kernel
// runs the same schedule with the same chunks (a unit with at most 32 records
// is one chunk there too: combine_shot), operation for operation, so the two
// kernels give bit-identical results.
template <int D, int G>
__global__ __launch_bounds__(D) void decode_combine_head_kernel(CombineArgs a) {
  constexpr int REC = G * D + 16;
  const int u = (int)blockIdx.x / G, h = (int)blockIdx.x - u * G;
  const int tid = threadIdx.x;  // element of head h
  const int U = a.B * a.Hkv;
  const int tsh = 31 - __builtin_clz(a.S / kTile);
  const int W = a.hdr[0];
  const int Tot = a.prefix[U] << tsh;
  const int ylo = a.prefix[u] << tsh, yhi = a.prefix[u + 1] << tsh;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int64_t head = (int64_t)b * a.Hq + (int64_t)g * G + h;
  if (yhi <= ylo) {  // no tokens: out = 0, lse = -inf
    a.out[head * D + tid] = 0.f;
    if (a.lse && tid == 0) a.lse[head] = kNegInf;
    return;
  }
  const int wlo = tile_owner(ylo, W, Tot);
  const int whi = tile_owner(yhi - 1, W, Tot);
  const int nw = whi - wlo + 1;
  const float* part = a.part + (int64_t)(u + wlo) * REC;  // record of wave wlo + t at t * REC
  const EqualSplit sp(Tot, W);
  float M = kNegInf, l = 0.f, o = 0.f;
  auto chunk = [&](int t0, auto ch_tag) {
    constexpr int CH = decltype(ch_tag)::value;
    const int tn = min(CH, nw - t0);
    float x[CH], mv[CH], lv[CH];
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const float* r = part + (int64_t)(t0 + min(t, tn - 1)) * REC;  // past tn: re-read, unused
      x[t] = r[h * D + tid];
      mv[t] = r[G * D + h];
      lv[t] = r[G * D + 8 + h];
    }
    // Waves are only ever empty when there are fewer tiles than waves.
    uint64_t skip = 0;
    if (Tot < W)
      for (int t = 0; t < tn; ++t) skip |= wave_empty(sp, wlo + t0 + t) ? (1ull << t) : 0ull;
    float Mc = kNegInf;
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const bool use = t < tn && !((skip >> t) & 1ull);
      Mc = use ? fmaxf(Mc, mv[t]) : Mc;
    }
    if (Mc == kNegInf) return;  // no valid token in the chunk
    const float Mn = fmaxf(M, Mc);
    // Arguments are <= 0 (or -inf, giving 0): the hardware exp2 is accurate there.
    const float s = __builtin_amdgcn_exp2f(M - Mn);
    o *= s;
    l *= s;
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      // Records without a valid token (m = -inf) and skipped slots add nothing;
      // stale slots may hold anything, so they are selected away, not scaled.
      const bool use = t < tn && !((skip >> t) & 1ull) && mv[t] != kNegInf;
      const float sc = __builtin_amdgcn_exp2f(mv[t] - Mn);
      o = use ? fmaf(x[t], sc, o) : o;
      l = use ? fmaf(lv[t], sc, l) : l;
    }
    M = Mn;
  };
  if (nw <= 8) chunk(0, std::integral_constant<int, 8>{});
  else if (nw <= 16) chunk(0, std::integral_constant<int, 16>{});
  else if (nw <= 32) chunk(0, std::integral_constant<int, 32>{});
  else
    for (int t0 = 0; t0 < nw; t0 += kHeadChunk) chunk(t0, std::integral_constant<int, kHeadChunk>{});
  a.out[head * D + tid] = l > 0.f ? o / l : 0.f;
  if (a.lse && tid == 0) a.lse[head] = l > 0.f ? (M + log2f(l)) * 0.69314718055994530942f : kNegInf;
}

template <typename T, int D, int G, bool GATED, bool GIVEN>
const void* partial_fn() { return (const void*)&decode_partial_kernel<T, D, G, GATED, GIVEN>; }

using KernelFn = const void* (*)();

template <typename T, int D, bool GATED, bool GIVEN>
KernelFn pick_g(int G) {
  switch (G) {
    case 1: return &partial_fn<T, D, 1, GATED, GIVEN>;
    case 2: return &partial_fn<T, D, 2, GATED, GIVEN>;
    case 3: return &partial_fn<T, D, 3, GATED, GIVEN>;
    case 4: return &partial_fn<T, D, 4, GATED, GIVEN>;
    case 5: return &partial_fn<T, D, 5, GATED, GIVEN>;
    case 6: return &partial_fn<T, D, 6, GATED, GIVEN>;
    case 7: return &partial_fn<T, D, 7, GATED, GIVEN>;
    case 8: return &partial_fn<T, D, 8, GATED, GIVEN>;
  }
  return nullptr;
}

template <bool GATED, bool GIVEN = false>
const void* pick_kernel(int dtype, int D, int G) {
  KernelFn f = nullptr;
  if (dtype == 1)
    f = D == 64 ? pick_g<uint16_t, 64, GATED, GIVEN>(G)
                : D == 128 ? pick_g<uint16_t, 128, GATED, GIVEN>(G) : nullptr;
  else
    f = D == 64 ? pick_g<float, 64, GATED, GIVEN>(G)
                : D == 128 ? pick_g<float, 128, GATED, GIVEN>(G) : nullptr;
  return f ? f() : nullptr;
}

const void* partial_kernel(int dtype, int D, int G) { return pick_kernel<false>(dtype, D, G); }
const void* gated_kernel(int dtype, int D, int G) { return pick_kernel<true>(dtype, D, G); }
const void* gated_given_kernel(int dtype, int D, int G) {
  return pick_kernel<true, true>(dtype, D, G);
}

template <int D, int G>
const void* combine_fn(bool per_head) {
  return per_head ? (const void*)&decode_combine_head_kernel<D, G>
                  : (const void*)&decode_combine_kernel<D, G>;
}

template <int D>
const void* combine_g(int G, bool per_head) {
  switch (G) {
    case 1: return combine_fn<D, 1>(per_head);
    case 2: return combine_fn<D, 2>(per_head);
    case 3: return combine_fn<D, 3>(per_head);
    case 4: return combine_fn<D, 4>(per_head);
    case 5: return combine_fn<D, 5>(per_head);
    case 6: return combine_fn<D, 6>(per_head);
    case 7: return combine_fn<D, 7>(per_head);
    case 8: return combine_fn<D, 8>(per_head);
  }
  return nullptr;
}

// Plan buffer: unit prefix [U + 1], scan scratch, unit lengths [U].
size_t prefix_smem_bytes(int U) { return (size_t)(2 * U + 1 + kWavesPerWG + 1) * sizeof(int); }

}  // namespace

size_t decode_part_offset(int U) {
  const size_t head = 64 + (size_t)(U + 1) * sizeof(int32_t);
  return (head + 255) & ~(size_t)255;
}

size_t decode_workspace_bytes(int B, int Hkv, int G, int D, int wmax) {
  const int U = B * Hkv;
  return decode_part_offset(U) + (size_t)(U + wmax) * (G * D + 16) * sizeof(float);
}

int decode_max_waves(int dtype, int D, int G) {
  const void* fn = partial_kernel(dtype, D, G);
  if (!fn) return 0;
  int dev = 0, cus = 0, blocks = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  // Cached per (device, instantiation): later calls (for example under stream
  // capture) make no device queries.
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev][2][2][9];
  std::atomic<int>* slot = nullptr;
  if (dev >= 0 && dev < kMaxDev) {
    slot = &cache[dev][dtype == 1][D == 128][G];
    const int c = slot->load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  // The kernel must fit on a CU with the largest plan buffer; it then runs
  // one workgroup per CU (see kDecodeWavesPerWG).
  const size_t smem = prefix_smem_bytes(kMaxUnits);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, kThreads, smem) != hipSuccess) return 0;
  if (blocks < 1) return 0;
  const int waves = cus * kWavesPerWG < kMaxWaves ? cus * kWavesPerWG : kMaxWaves;
  if (slot) slot->store(waves, std::memory_order_relaxed);
  return waves;
}

hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const void* fn = partial_kernel(a.dtype, a.D, G);
  if (!fn) return hipErrorInvalidValue;
  const int U = a.B * a.Hkv;
  DecodeArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(fn, dim3(a.W / kWavesPerWG), dim3(kThreads), params,
                         prefix_smem_bytes(U), stream);
}

size_t gated_decode_static_smem(int dtype, int D, int G) {
  const void* fn = gated_kernel(dtype, D, G);
  hipFuncAttributes attr;
  if (!fn || hipFuncGetAttributes(&attr, fn) != hipSuccess) return (size_t)-1;
  return attr.sharedSizeBytes;
}

size_t gated_decode_smem_bytes(int U, int NB, int ids_cap) {
  const size_t ints = prefix_smem_bytes(U) + (size_t)ids_cap * sizeof(int32_t);
  return ((ints + 7) & ~(size_t)7) + (size_t)NB * sizeof(uint64_t);
}

int gated_decode_ids_cap(int U, int k_max, int W) {
  // A workgroup's tile range holds at most ceil(total / workgroups) tiles; the
  // units it meets add at most the rest of the first and the last unit.
  const int64_t wgs = W / kWavesPerWG;
  const int64_t blocks = (int64_t)U * k_max;
  const int64_t cap = (blocks + wgs - 1) / wgs + 2 * (int64_t)k_max + 2;
  return (int)(cap < blocks ? cap : blocks);
}

hipError_t launch_gated_decode_partial(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const void* fn = a.scores_in ? gated_given_kernel(a.dtype, a.D, G) : gated_kernel(a.dtype, a.D, G);
  if (!fn) return hipErrorInvalidValue;
  const int U = a.B * a.Hkv;
  DecodeArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(fn, dim3(a.W / kWavesPerWG), dim3(kThreads), params,
                         gated_decode_smem_bytes(U, a.NB, a.ids_cap), stream);
}

// ---------------------------------------------------------------- static scratch
//
// Device memory of the allocation-free decode call: the same workspace layout
// as a caller's workspace, in a file-scope array that every GPU the library
// runs on holds (at its own address) until the process ends.  In host code
// the array's name only stands in for the symbol; its device address is
// looked up once per device, with that device current, and kept per device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

void* decode_static_scratch(hipError_t* err) {
  *err = hipSuccess;
  int dev = 0;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
  constexpr int kMaxDev = 64;
  static std::atomic<void*> addr[kMaxDev];
  if (dev < 0 || dev >= kMaxDev) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  // Two threads that get here first on one device look up the same address.
  if ((*err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return nullptr;
  if (!p) {
    *err = hipErrorInvalidSymbol;
    return nullptr;
  }
  addr[dev].store(p, std::memory_order_release);
  return p;
}

hipError_t launch_decode_combine(const CombineArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const bool ph = a.per_head != 0;
  const void* fn = a.D == 64 ? combine_g<64>(G, ph) : a.D == 128 ? combine_g<128>(G, ph) : nullptr;
  if (!fn) return hipErrorInvalidValue;
  CombineArgs args = a;
  void* params[] = {&args};
  if (ph)
    return hipLaunchKernel(fn, dim3(a.B * a.Hq), dim3(a.D), params, 0, stream);
  return hipLaunchKernel(fn, dim3(a.B * a.Hkv), dim3(kCombineThreads), params, 0, stream);
}

}  // namespace seer
