// qg_xs.h -- 2..32-row skinny GEMM over uniform b-bit codes on the matrix cores
// (v_mfma_f32_16x16x32_f16), with x held in LDS: the speculative-decode verify
// product y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] * (c[n][k] - o).
//
// Work split.  K is cut into S slices of whole quads (512 k).  A workgroup
// serves one slice: it copies that slice of x (all M rows) into LDS once, with
// buffer-to-LDS loads that need no registers, and then streams the codes of a
// run of tile groups through it.  A tile group is T tiles of 16 columns (the
// fused gate/up pass: one gate tile and the up tile beside it).  The
// workgroup's waves take the run's tile groups in turn, and each wave walks
// its (tile group, quad) units in order with the code loads of the next PD
// units in flight while it computes one.  So x is read from L2 once per
// workgroup and never again from memory, every A fragment a wave reads from
// LDS serves two tiles, and a wave's code loads are only ever waited for in
// the order they were issued (the x copy is issued before all of them).
//
// Arithmetic.  Codes are decoded at bit offset 1 (exact fp16 c * 2^-23) and
// form the B operand.  Each group's MFMA chain starts from the offset term
// -o * 2^-23 * sum_{k in g} x[m][k], from group sums computed once per
// workgroup out of LDS, so the chain yields 2^-23 * sum x (c - o); the fp16
// scale multiplies it into the fp32 accumulator.  The fused MLP's down pass
// (XSC) takes its x as fp16 values scaled by a power of two per (row, group)
// (the fp32 intermediate rounded once with a block exponent, qg_misc.h), and
// multiplies each row's chain by that row and group's 2^-e as well.
//
// Scale groups of 64 or 32 (SQ): one MFMA spans lanes of four different scales,
// so the scale goes into the B operand instead (decode_group_scaled: 2 (c - o)
// s rounded once to fp16); the chains then need no offset term and no group
// sums, run on across groups, and yield 2 y.
//
// MXFP4 (MX): the elements decode to fp16 values of their own (times 2^-14);
// the four lane quarters of a group carry E8M0 exponents of their own, so each
// quarter's operand is multiplied by 2^-(e_max - e) (exact while it stays in
// fp16's range, else rounded once) and the group's chain by 2^(e_max - 113),
// e_max the largest of the four (kept beside each exponent at create).  MXFP6
// likewise, its E3M2 elements decoded at 2^-12 and multiplied by 2^(15 - de)
// (the operand is the element times 2^(3 - de), exact for de <= 23), the chain
// by 2^(e_max - 130).
//
// K slices meet in one of two ways, both independent of the order of arrival.
// Few outputs: in fixed-point words (see fx_word), one integer atomic per
// output and slice, whose returned count tells the last slice to store the
// result -- one round trip.  Many outputs (where that many atomics would
// queue): in the fp32 workspace; a wave stores its slice's partials of its
// tile group, waits for its own stores and counts one arrival at the group's
// counter, and the wave that completes the count re-arms it, reads all S
// partials of each output (several slices' loads in flight at once) and adds
// them in slice order 0..S-1.  With one slice the result is stored directly.
#pragma once
#include "qg_common.h"

namespace qg {




template <int B, int T, int ND>
struct XsUnit {
  uint32_t cw[ND][T][4 * B];
  uint2 sc[ND][T];
};
template <int B, int T, int ND> constexpr int xs_loads() { return ND * T * (B + 1); }

// the code and scale loads of unit (tile group tg, quad q); a dead unit (or a
// tile past the segment) loads through an empty range: zeros, no memory access
template <int B, int T, int ND, bool SQ>
__device__ __forceinline__ void xs_load(XsUnit<B, T, ND>& c, const SegDev (&sd)[2], int tg, int q, bool live, int G4,
                                        uint32_t lane) {
  constexpr int sq = SQ ? 1 : 0;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int tile = tg * T + t;
      const bool ok = live && tile < sd[d].tiles;
      const size_t qb = ok ? (size_t)tile * G4 + q : 0;
      const __amdgpu_buffer_rsrc_t rc = make_rsrc(uniform_ptr(sd[d].codes) + qb * (B * 256), ok ? B * 1024u : 0u);
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(uniform_ptr(sd[d].scales) + qb * scale_quad_halves(sq), ok ? scale_quad_halves(sq) * 2u : 0u);
      buffer_quad<B>(rc, lane, 0, c.cw[d][t]);
      const u2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, scale_lane_byte(sq, lane), 0, 0);
      c.sc[d][t] = make_uint2(v.x, v.y);
    }
}

// one unit: groups gl0 .. gl0 + ngr - 1 of the slice against the unit's tiles;
// xa[mt][v]: this lane's A-fragment address of group 0 (add 256 per group)
template <int B, int T, int MT, int ND, bool XSC, bool SQ, bool MX>
__device__ __forceinline__ void xs_unit(const XsUnit<B, T, ND>& c, const char* const (&xa)[MT][4], const float* xsum,
                                        const float* xfac, int gl0, int ngr, int lane, f4_t (&R)[ND][T][MT]) {
  const int kq = lane >> 4;
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    if (gi >= ngr) break;
    const int gl = gl0 + gi;
    h8_t A[MT][4];
    f4_t C0[MT], F[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) A[mt][v] = *reinterpret_cast<const h8_t*>(xa[mt][v] + gl * 256);
      // chain start: rows 16 mt + 4 kq + e (sums past M are never stored either)
      if constexpr (!SQ) C0[mt] = *reinterpret_cast<const f4_t*>(xsum + gl * (16 * MT) + 16 * mt + 4 * kq);
      if constexpr (XSC) F[mt] = *reinterpret_cast<const f4_t*>(xfac + gl * (16 * MT) + 16 * mt + 4 * kq);
    }
    if constexpr (MX) {
      static_assert((B == 4 || B == 6) && ND == 1 && !XSC, "MXFP4 / MXFP6: one matrix, fp16 x");
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t sw = (gi < 2) ? c.sc[0][t].x : c.sc[0][t].y;
        const uint32_t ent = ((gi & 1) ? (sw >> 16) : sw) & 0xFFFFu;
        const uint32_t eq = ent & 0xFFu, emax = ent >> 8, de = emax - eq;
        // fp16 2^-de (E2M1 at 2^-14), or 2^(15 - de) (E3M2 at 2^-12: the operand is the element times 2^(3 - de))
        const uint32_t f = B == 6 ? mx6_operand_factor(de)
                                  : (de <= 14u ? (15u - de) << 10 : (de <= 24u ? 1u << (24u - de) : 0u));
        uint32_t r[16];
        if constexpr (B == 6) decode_group_mx6(c.cw[0][t], gi, r);
        else decode_group_mx(c.cw[0][t], gi, r);
#pragma unroll
        for (int i = 0; i < 16; ++i) r[i] = pk_mul_f16(r[i], f | (f << 16));
        const float s = e8m0_scale(emax, B == 6 ? -3 : 14);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f4_t cc = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int v = 0; v < 4; ++v) cc = mfma16(A[mt][v], as_h8(r[4 * v], r[4 * v + 1], r[4 * v + 2], r[4 * v + 3]), cc);
#pragma unroll
          for (int e = 0; e < 4; ++e) R[0][t][mt][e] = __builtin_fmaf(s, cc[e], R[0][t][mt][e]);
        }
      }
      continue;
    }
    if constexpr (SQ) {
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t sw = (gi < 2) ? c.sc[d][t].x : c.sc[d][t].y;
          const uint32_t sh = (gi & 1) ? (sw >> 16) : (sw & 0xFFFFu);
          uint32_t r[16];
          decode_group_scaled<B>(c.cw[d][t], gi, sh | (sh << 16), r);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            f4_t cc = XSC ? f4_t{0.0f, 0.0f, 0.0f, 0.0f} : R[d][t][mt];  // without factors: one chain throughout
#pragma unroll
            for (int v = 0; v < 4; ++v)
              cc = mfma16(A[mt][v], as_h8(r[4 * v], r[4 * v + 1], r[4 * v + 2], r[4 * v + 3]), cc);
            if constexpr (XSC) {
#pragma unroll
              for (int e = 0; e < 4; ++e) R[d][t][mt][e] = __builtin_fmaf(F[mt][e], cc[e], R[d][t][mt][e]);
            } else {
              R[d][t][mt] = cc;
            }
          }
        }
      continue;
    }
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        uint32_t r[16];
        decode_group_off1<B>(c.cw[d][t], gi, r);
        const uint32_t sw = (gi < 2) ? c.sc[d][t].x : c.sc[d][t].y;
        const float s = h2f((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f4_t cc = C0[mt];
#pragma unroll
          for (int v = 0; v < 4; ++v) cc = mfma16(A[mt][v], as_h8(r[4 * v], r[4 * v + 1], r[4 * v + 2], r[4 * v + 3]), cc);
          if constexpr (XSC) cc = cc * F[mt];
#pragma unroll
          for (int e = 0; e < 4; ++e) R[d][t][mt][e] = __builtin_fmaf(s, cc[e], R[d][t][mt][e]);
        }
      }
  }
}

template <int B, int T, int MT, int ND, int NQ, bool XSC, bool SQ, bool MX = false>
__device__ __forceinline__ void xs_body(const XsArgs& a, const SegDev (&sd)[2], int s, int q0, int nq, int tgb, int tge,
                                        int tgbase, char* smem) {
  constexpr float kOut = MX ? 1.0f : (SQ ? 0.5f : 8388608.0f);  // the chains' unit: y, 2 y (SQ) or 2^-23 y
  const int lane = threadIdx.x & 63;
  const int NW = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = a.M, G = a.G, G4 = a.G4, S = a.S;
  constexpr int RS = NQ * 1024;  // bytes per row of x in LDS
  char* xl = smem;
  float* xsum = reinterpret_cast<float*>(smem + xs_x_bytes(M, NQ));
  float* xfac = xsum + NQ * 4 * 16 * MT;  // XSC only
  int* cols = reinterpret_cast<int*>(smem + xs_x_bytes(M, NQ) + (XSC ? 2 : 1) * xs_sum_bytes(MT, NQ));
  // ---- the x slice -> LDS: one wave instruction per (row m, 4 groups) = 1 KiB;
  // groups past G read zeros
  {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(uniform_ptr(a.x), (uint32_t)M * a.K * 2u);
    const int gq = lane >> 4, p = lane & 15;
    int m = 0, part = wave;  // instruction wave + NW j = (row m, part) with part < nq
    while (part >= nq) {
      part -= nq;
      ++m;
    }
    while (m < M) {
      const int g = 4 * (q0 + part) + gq;
      const uint32_t voff = g < G ? (uint32_t)(((size_t)m * a.K + (size_t)g * 128 + (p ^ (m & 15)) * 8) * 2) : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(xl + (size_t)m * RS + (size_t)part * 1024), 16, voff, 0, 0, 0);
      part += NW;
      while (part >= nq) {
        part -= nq;
        ++m;
      }
    }
    // output columns of the run's tiles (256 per wave instruction)
    const int t0 = tgb * T, nt = min(tge * T, sd[0].tiles) - t0;
    const __amdgpu_buffer_rsrc_t rcm =
        make_rsrc(uniform_ptr(a.w[0].col_map) + 16 * (sd[0].tile0 + t0), (uint32_t)max(nt, 0) * 64u);
    for (int base = wave * 256; base < nt * 16; base += NW * 256)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rcm, (__attribute__((address_space(3))) void*)(cols + base), 16,
                                               (uint32_t)(base + 4 * lane) * 4u, 0, 0, 0);
  }
  // XSC: the factors of the slice's (group, row) pairs, [group][16 * MT] (rows
  // past M and groups past G: 0), loaded into registers ahead of the code loads
  constexpr int XFR = XSC ? NQ * MT : 1;  // factors per thread at one wave (fewer with more)
  float xfr[XFR];
  if constexpr (XSC) {
#pragma unroll
    for (int r = 0; r < XFR; ++r) {
      const int idx = threadIdx.x + r * (int)blockDim.x;
      const int gl = idx / (16 * MT), m = idx - gl * (16 * MT);
      const int g = 4 * q0 + gl;
      xfr[r] = (gl < 4 * nq && m < M && g < G) ? a.xf[(size_t)m * G + g] : 0.0f;
    }
  }
  // ---- this wave's tile group tgb + wave: its units are the slice's quads
  const int tg = tgb + wave;
  const bool mine = tg < tge;
  // Only XS_LEAD units' code loads go out before the x slice is waited for:
  // a wave that issues more stalls at the issue once the compute unit's
  // outstanding loads fill up, and cannot reach its first compute until the
  // whole batch has streamed in.
  static_assert(XS_LEAD >= 1 && XS_LEAD <= XS_PD, "lead units");
  XsUnit<B, T, ND> c[XS_PD];
#pragma unroll
  for (int i = 0; i < XS_LEAD; ++i) {
    xs_load<B, T, ND, SQ>(c[i], sd, tg, q0 + i, mine && i < nq, G4, (uint32_t)lane);
    __builtin_amdgcn_sched_barrier(0);  // unit by unit, in order of use
  }
  {
    constexpr int n = XS_LEAD * xs_loads<B, T, ND>();  // issued after the x copy
    static_assert(n < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
  }
  if constexpr (XSC) {
#pragma unroll
    for (int r = 0; r < XFR; ++r) {
      const int idx = threadIdx.x + r * (int)blockDim.x;
      if (idx < 4 * nq * 16 * MT) xfac[idx] = xfr[r];
    }
  }
  lds_barrier();  // every wave's share of the slice has landed
  // this lane's A-fragment addresses (group 0): row 16 mt + m16 (rows past M
  // repeat row M - 1, never stored), chunk 4 kq + v at its swizzled position
  const char* xa[MT][4];
  {
    const int kq = lane >> 4, m16 = lane & 15;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = min(16 * mt + m16, M - 1);
#pragma unroll
      for (int v = 0; v < 4; ++v) xa[mt][v] = xl + (size_t)row * RS + (((4 * kq + v) ^ (row & 15)) * 16);
    }
  }
  // ---- group sums of x on the matrix cores: group gl's A fragments against
  // an all-ones B operand, chained over the group's four 32-k blocks like the
  // products; lane (kq, n) gets the sums of rows 16 mt + 4 kq + e in every
  // column n, and the lanes of column 0 store them times -o * 2^-23 (the
  // chain start of the group's products).  A row's sum depends on that row's
  // values only, so it rounds the same at every row count.
  if constexpr (!SQ) {
    const h8_t ones = as_h8(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
    const float ko = off1_ko<B>();  // -o * 2^-23
    for (int gl = wave; gl < 4 * nq; gl += NW) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f4_t cc = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int v = 0; v < 4; ++v) cc = mfma16(*reinterpret_cast<const h8_t*>(xa[mt][v] + gl * 256), ones, cc);
        if ((lane & 15) == 0) *reinterpret_cast<f4_t*>(xsum + gl * (16 * MT) + 16 * mt + 4 * (lane >> 4)) = cc * ko;
      }
    }
  }
  lds_barrier();
  if (!mine) return;
  // ---- units
  f4_t R[ND][T][MT];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) R[d][t][mt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // Straight-line code over NQ units (a slice has nq <= NQ; units past nq are
  // skipped, their loads go through empty ranges): no loop carries the ring,
  // so no register copy waits for a load in flight, and the loads are issued
  // in the same order on every path, so each wait counts exactly.  Before
  // unit i is computed, the loads of every unit up to i + XS_PD - 1 are out
  // (unit i + XS_PD - 1 into the buffer unit i - 1 has just freed).
  // (scheduling barriers keep each unit's work after the previous unit's: the
  // scheduler would otherwise pull the next unit's decode forward, and with
  // it the wait for that unit's codes)
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
#pragma unroll
    for (int u = i == 0 ? XS_LEAD : i + XS_PD - 1; u <= i + XS_PD - 1; ++u)
      if (u < NQ) xs_load<B, T, ND, SQ>(c[u % XS_PD], sd, tg, q0 + u, u < nq, G4, (uint32_t)lane);
    __builtin_amdgcn_sched_barrier(0);
    if (i < nq) xs_unit<B, T, MT, ND, XSC, SQ, MX>(c[i % XS_PD], xa, xsum, xfac, 4 * i, min(4, G - 4 * (q0 + i)), lane, R);
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- results: stored directly (one slice), or added to the fixed-point
  // words of their outputs; the arrival that completes a word's S slices
  // stores the fp16 result and re-arms the word
  const int mq = lane >> 4, j = lane & 15;
  if (S == 1) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int tile = tg * T + t;
      if (tile >= sd[0].tiles) continue;
      const int n = cols[16 * (tile - tgb * T) + j];
      if (n < 0) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * mt + 4 * mq + e;
          if (m >= M) continue;
          const float v0 = R[0][t][mt][e] * kOut;
          const float v1 = R[ND - 1][t][mt][e] * kOut;
          store_y(a.y, (size_t)m * a.ldy + n, ND == 2 ? silu_mul(v0, v1) : v0, a.yf32);
        }
    }
    return;
  }
  if (a.acc) {
    // fixed-point words, one per output (see fx_word): each slice adds its part
    // with one integer atomic whose returned value also counts the arrivals; the
    // arrival that completes S slices stores the result and re-arms the word.
    // One round trip (two for the fused pass, whose up words are completed
    // before the gate words count); chosen when the outputs are few.
    unsigned long long* const W = a.acc;  // [ND][M][NP]
    const size_t up_off = (size_t)M * a.NP;
    __builtin_amdgcn_s_waitcnt(0);  // retire the empty-range loads: no waits among the atomics
    const bool live0 = tg * T < sd[0].tiles, live1 = tg * T + 1 < sd[0].tiles;
    if constexpr (ND == 2) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 16 * mt + 4 * mq + e;
            const int pc = 16 * (sd[0].tile0 + tg * T + t) + j;
            if ((t == 0 ? live0 : live1) && m < M)
              fx_add(W + up_off + (size_t)m * a.NP + pc, fx_word(R[1][t][mt][e] * kOut));
          }
      __builtin_amdgcn_s_waitcnt(0);
    }
    unsigned long long og[T][MT][4], ag[T][MT][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) ag[t][mt][e] = fx_word(R[0][t][mt][e] * kOut);
    unsigned long long* const wl = W + (size_t)(4 * mq) * a.NP + 16 * (sd[0].tile0 + tg * T) + j;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * mt + 4 * mq + e;
          og[t][mt][e] = ((t == 0 ? live0 : live1) && m < M)
                             ? fx_add(wl + (size_t)(16 * mt + e) * a.NP + 16 * t, ag[t][mt][e]) : 0ull;
        }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int tile = tg * T + t;
      if (tile >= sd[0].tiles) continue;
      const int pc = 16 * (sd[0].tile0 + tile) + j;
      const int n = cols[16 * (tile - tgb * T) + j];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * mt + 4 * mq + e;
          if (m >= M || fx_count(og[t][mt][e]) != S - 1) continue;
          unsigned long long* wg = W + (size_t)m * a.NP + pc;
          float v = fx_value(og[t][mt][e] + ag[t][mt][e]);
          if constexpr (ND == 2) {
            unsigned long long* wu = wg + up_off;
            v = silu_mul(v, fx_value(fx_add(wu, 0ull)));
            fx_rearm(wu);
          }
          fx_rearm(wg);
          if (n >= 0) store_y(a.y, (size_t)m * a.ldy + n, v, a.yf32);
        }
    }
    return;
  }
  // partials in the fp32 workspace, one block per (tile group, slice, matrix):
  // [T * MT quarter tiles][64 lanes][4] fp32, so each quarter tile is one
  // contiguous 1 KiB store, written through to the device coherence point
  // (sc1); then one arrival per wave at the tile group's counter.  Rows past M
  // and tiles past the segment are stored too (never read as outputs).
  constexpr int NQT = T * MT;
  constexpr uint32_t kSc1 = 16;  // cache policy: device-coherent access
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(uniform_ptr(a.partial) + (size_t)(tgbase + tg) * S * ND * NQT * 256,
                                              (uint32_t)S * ND * NQT * 1024u);
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f4_t v = R[d][t][mt] * kOut;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, v), rp,
                                               (uint32_t)(((s * ND + d) * NQT + t * MT + mt) * 1024 + lane * 16), 0, kSc1);
      }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(a.counters + tgbase + tg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old != S - 1) return;
  if (lane == 0) __hip_atomic_store(a.counters + tgbase + tg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the last slice to arrive: the other slices' blocks, KB slices at a time
  // with all their loads in flight, summed in slice order 0..S-1 (its own
  // slice from registers, the same values it stored)
  constexpr int KB = ND == 2 ? 2 : 4;
  f4_t acc[ND][T][MT];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[d][t][mt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < S; k0 += KB) {
    f4_t v[KB][ND][T][MT];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int k = k0 + kb;
            // slices past S, and its own, read outside the range: zeros, and
            // are not added from memory
            const uint32_t vo = (k < S && k != s) ? (uint32_t)(((k * ND + d) * NQT + t * MT + mt) * 1024 + lane * 16)
                                                  : 0xFFFFFFF0u;
            v[kb][d][t][mt] = __builtin_bit_cast(f4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, vo, 0, kSc1));
          }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int k = k0 + kb;
      if (k < S) {
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[d][t][mt] += k == s ? R[d][t][mt] * kOut : v[kb][d][t][mt];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int tile = tg * T + t;
    if (tile >= sd[0].tiles) continue;
    const int n = cols[16 * (tile - tgb * T) + j];
    if (n < 0) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mt + 4 * mq + e;
        if (m >= M) continue;
        store_y(a.y, (size_t)m * a.ldy + n,
                ND == 2 ? silu_mul(acc[0][t][mt][e], acc[ND - 1][t][mt][e]) : acc[0][t][mt][e], a.yf32);
      }
  }
}

// NQ: the most quads a slice may have (the kernel is straight-line code over them)
template <int T, int MT, bool DUAL, int BF, int NQ, bool XSC, bool SQ>
__global__ __launch_bounds__(512) void k_gemm_xs(XsArgs a) {
  static_assert(!(DUAL && XSC), "the fused gate/up pass reads plain fp16 x");
  extern __shared__ __align__(16) char smem[];
  constexpr int ND = DUAL ? 2 : 1;
  const int S = a.S, G4 = a.G4;
  const int s = blockIdx.x % S, pw = blockIdx.x / S;
  int si = 0;
  if (BF == 0)
    while (si + 1 < a.w[0].nseg && pw >= a.wg_prefix[si + 1]) ++si;
  SegDev sd[2];
  sd[0] = BF == 0 ? pick(a.w[0], si) : a.w[0].seg[0];
  sd[1] = DUAL ? (BF == 0 ? pick(a.w[1], si) : a.w[1].seg[0]) : sd[0];
  const int ngr = (sd[0].tiles + T - 1) / T;  // tile groups of the segment
  const int tgb = (pw - a.wg_prefix[si]) * a.GPW, tge = min(tgb + a.GPW, ngr);
  const int q0 = (int)((int64_t)s * G4 / S), q1 = (int)((int64_t)(s + 1) * G4 / S);
  const int bits = sd[0].bits;
  if constexpr (BF == 5) {  // MXFP4 (per-quarter scale entries, the 4-bit layout)
    if constexpr (!DUAL && !XSC) xs_body<4, T, MT, ND, NQ, XSC, true, true>(a, sd, s, q0, q1 - q0, tgb, tge, a.tg_prefix[si], smem);
  } else if constexpr (BF == 6) {  // MXFP6 (per-quarter scale entries, the two-plane 6-bit layout)
    if constexpr (!DUAL && !XSC) xs_body<6, T, MT, ND, NQ, XSC, true, true>(a, sd, s, q0, q1 - q0, tgb, tge, a.tg_prefix[si], smem);
  } else if (BF == 2 || (BF == 0 && bits == 2))
    xs_body<2, T, MT, ND, NQ, XSC, SQ>(a, sd, s, q0, q1 - q0, tgb, tge, a.tg_prefix[si], smem);
  else if (BF == 3 || (BF == 0 && bits == 3))
    xs_body<3, T, MT, ND, NQ, XSC, SQ>(a, sd, s, q0, q1 - q0, tgb, tge, a.tg_prefix[si], smem);
  else xs_body<4, T, MT, ND, NQ, XSC, SQ>(a, sd, s, q0, q1 - q0, tgb, tge, a.tg_prefix[si], smem);
}

}  // namespace qg
