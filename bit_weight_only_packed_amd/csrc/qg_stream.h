// qg_stream.h -- M = 1 GEMV over uniform b-bit codes on the vector ALU
// (v_dot2_f32_f16), for one matrix or the gate/up pair of an MLP.
//
// Work split.  A unit is one 16-column tile times one quad (4 groups, 512 k):
// B KiB of codes, read by B wave-wide 16-byte-per-lane loads, and 128 B of
// scales.  Each tile's G4 quads are cut into `nch` near-equal runs of at most
// SK_UPW consecutive quads, one run per wave; a wave walks its run in
// straight-line code with the next SK_PD - 1 units' loads in flight (SK_PD
// register sets in rotation), so every wait the compiler places is exact, and
// hands its partial of the tile on once, at the end.
//
// Activations.  Each wave stages the activations of its own run in an LDS
// region of its own (qg_stage.h: each element times 2^(e - class), e the
// wave's block exponent), so a pair decoded by one AND at its class offset
// times its staged x pair is c * x * 2^(e - 24) whatever the class: one dot2
// chain per group, no per-class accumulators.  Beside it, per quarter, the sum
// of the staged values: the code offset enters as -o * 2^-24 * sum, one fma
// per group.  The 16 lanes of a quarter read the same LDS addresses
// (broadcast).  The x loads go out first and the wave's first code loads right
// behind them, so staging x overlaps the first code fetches; no wave waits for
// another.
//
// The nch partials of one tile meet in a per-column 64-bit fixed-point word
// (fx_word, qg_common.h): each wave adds its partial with one integer atomic.
// Integer addition is exact and commutative, so the total is the same
// whatever the order of arrival (bit-identical results), and the word's low 6
// bits count the arrivals: the wave that brings the count to nch converts the sum
// to fp16, stores it and re-arms the word to 0 for the next launch.  With
// nch = 1 the sum is stored directly.  For the gate/up pair every wave adds its
// up partial, waits for that atomic to return, and only then adds its gate
// partial: the wave that completes the gate word therefore finds the up word
// complete too.
#pragma once
#include "qg_stage.h"

namespace qg {




template <int B, int ND>
struct SkUnit {
  uint32_t cw[ND][4 * B];
  uint2 sc[ND];
};

// code and scale base pointers of the segment's matrices (wave-uniform)
template <int ND>
struct SkPtrs {
  const uint32_t* codes[ND];
  const uint16_t* scales[ND];
  int sq;  // the scale layout (qg_common.h), the same for both matrices
};

// unit u (segment-local: tile u / G4, quad u % G4) of the segment's matrices
template <int B, int ND>
__device__ __forceinline__ void sk_load(const SkPtrs<ND>& p, SkUnit<B, ND>& c, int u, bool live, int lane) {
  const uint32_t uc = live ? (uint32_t)u : 0u;
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(p.scales[d] + (size_t)uc * scale_quad_halves(p.sq), live ? scale_quad_halves(p.sq) * 2u : 0u);
    const u2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, scale_lane_byte(p.sq, (uint32_t)lane), 0, 0);
    c.sc[d] = make_uint2(v.x, v.y);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.codes[d] + (size_t)uc * (B * 256), live ? B * 1024u : 0u);
    buffer_quad<B>(rc, (uint32_t)lane, 0, c.cw[d]);
  }
}

// The SK_PD register sets of a wave's load pipeline over one width segment.
template <int B, int ND>
struct SkPipe {
  SkPtrs<ND> ptr;
  SkUnit<B, ND> c[SK_PD];
};

// Issue the loads of the first SK_PD units of [u0, u1) (segment-local); a
// wave with an empty range issues loads that read nothing.
template <int B, int ND>
__device__ __forceinline__ void sk_prime(SkPipe<B, ND>& pp, const SegDev (&sd)[2], int u0, int u1, int lane) {
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    pp.ptr.codes[d] = uniform_ptr(sd[d].codes);
    pp.ptr.scales[d] = uniform_ptr(sd[d].scales);
  }
  pp.ptr.sq = __builtin_amdgcn_readfirstlane(sd[0].sq);
#pragma unroll
  for (int i = 0; i < SK_PD; ++i) sk_load<B, ND>(pp.ptr, pp.c[i], u0 + i, u0 + i < u1, lane);
}

// Walk the primed units [u0, u1) (segment-local, all of one tile, at most
// SK_UPW of them) and hand the tile's partial on.  tg0 = global index of the
// segment's first tile, xl / xsl = the run's staged x and quarter sums (group
// 0 = the run's first), unscale = 2^(24 - e).
template <int B, int ND, bool ONE>
__device__ __forceinline__ void sk_run(const SkArgs& a, SkPipe<B, ND>& pp, int u0, int u1, int tg0,
                                       const uint4* xl, const float* xsl, float unscale, int lane) {
  if (u0 >= u1) return;
  const int q = lane >> 4, j = lane & 15;
  const float ko = cls_ko<B>();  // -o * 2^-24
  float acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = 0.0f;
  const int tile = u0 / a.G4;
  auto step = [&](SkUnit<B, ND>& cu, int u) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int g = 4 * (u - u0) + gi;  // groups past G are staged as zeros and scaled by 0
      uint32_t xp[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 t = xl[(g * 4 + q) * 4 + v];
        xp[4 * v + 0] = t.x; xp[4 * v + 1] = t.y; xp[4 * v + 2] = t.z; xp[4 * v + 3] = t.w;
      }
      const float xs = xsl[g * 4 + q];
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        uint32_t r[16];
        decode_group_classes<B>(cu.cw[d], gi, r);
        float e0 = xs * ko, e1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          e0 = dot2(r[i], xp[i], e0);
          e1 = dot2(r[i + 1], xp[i + 1], e1);
        }
        const uint32_t sw = (gi < 2) ? cu.sc[d].x : cu.sc[d].y;
        const float s = h2f((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
        acc[d] = __builtin_fmaf(s, e0 + e1, acc[d]);
      }
    }
    if (u + SK_PD - u0 < SK_UPW) sk_load<B, ND>(pp.ptr, cu, u + SK_PD, u + SK_PD < u1, lane);
  };
#pragma unroll
  for (int k = 0; k < SK_UPW; ++k)
    if (u0 + k < u1) step(pp.c[k % SK_PD], u0 + k);
  // ---- hand this wave's partial of the tile on
  const int tg = tg0 + tile;  // tile index over all segments
  float v[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    float t = acc[d] * unscale;  // 2^(24 - e)
    t += __shfl_xor(t, 16);
    t += __shfl_xor(t, 32);
    v[d] = t;
  }
  const int pc = 16 * tg + j;
  // one width: columns are in order (padding only past N), no map needed
  const int n = lane >= 16 ? -1 : (ONE ? (pc < a.N ? pc : -1) : a.w[0].col_map[pc]);
  if (n < 0) return;
  const int nch = a.nch;
  if (nch == 1) {
    store_y(a.y, n, ND == 2 ? silu_mul(v[0], v[1]) : v[0], a.yf32);
    return;
  }
  unsigned long long* wg = a.acc + pc;
  const unsigned long long ag = fx_word(v[0]);
  if constexpr (ND == 2) {
    unsigned long long* wu = a.acc + 16 * (size_t)a.total_tiles + pc;
    const unsigned long long ou = fx_add(wu, fx_word(v[1]));
    __builtin_amdgcn_s_waitcnt(0);  // the up word holds this wave's part before gate counts it
    __asm__ volatile("" ::"v"(ou));
    const unsigned long long og = fx_add(wg, ag);
    if (fx_count(og) == nch - 1) {
      const unsigned long long tu = fx_add(wu, 0ull);
      store_y(a.y, n, silu_mul(fx_value(og + ag), fx_value(tu)), a.yf32);
      fx_rearm(wg);
      fx_rearm(wu);
    }
  } else {
    const unsigned long long og = fx_add(wg, ag);
    if (fx_count(og) == nch - 1) {
      store_y(a.y, n, fx_value(og + ag), a.yf32);
      fx_rearm(wg);
    }
  }
}

// range of segment si's units [v0, v1) (segment-local) inside the wave's [lo, hi)
__device__ __forceinline__ void sk_seg_range(const SegDev& sd, int G4, int64_t lo, int64_t hi, int& v0, int& v1) {
  const int64_t sg0 = (int64_t)sd.tile0 * G4, sg1 = sg0 + (int64_t)sd.tiles * G4;
  const int64_t u0 = max(lo, sg0), u1 = min(hi, sg1);
  v0 = (int)(u0 - sg0);
  v1 = (int)(max(u1, u0) - sg0);
}

// one wave's run over a segment of width B: its x loads, then its first
// units' loads, then its x staged (for width B) in its LDS region, then the run
template <int B, int ND, bool ONE, bool XF>
__device__ __forceinline__ void sk_body(const SkArgs& a, const SegDev (&sd)[2], int64_t lo, int64_t hi, char* wsm,
                                        int lane) {
  int v0, v1;
  sk_seg_range(sd[0], a.G4, lo, hi, v0, v1);
  // the run's activations: quads q0 .. q0 + nq - 1 of the row (zeros past G)
  constexpr int W = XIn<XF>::W;
  const int q0 = __builtin_amdgcn_readfirstlane(v0 - (v0 / a.G4) * a.G4);
  const int nq = __builtin_amdgcn_readfirstlane(v1 - v0);
  const int ng = __builtin_amdgcn_readfirstlane(max(0, min(4 * nq, a.G - 4 * q0)));
  const char* xb = reinterpret_cast<const char*>(a.x) + (size_t)4 * q0 * 128 * (XF ? 4 : 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(uniform_ptr(xb), (uint32_t)ng * 128u * (XF ? 4u : 2u));
  uint4 xv[SK_UPW][W];
#pragma unroll
  for (int r = 0; r < SK_UPW; ++r) {
    if (r >= nq) break;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const u4_t q = __builtin_amdgcn_raw_buffer_load_b128(rx, ((uint32_t)(lane + 64 * r) * W + k) * 16u, 0, 0);
      xv[r][k] = make_uint4(q.x, q.y, q.z, q.w);
    }
  }
  // the lane's row of the class-factor table, before the code loads
  uint4 tf, ti;
  stage_tab<B>(lane & 3, tf, ti);
  __builtin_amdgcn_sched_barrier(0);
  SkPipe<B, ND> pp;
  sk_prime<B, ND>(pp, sd, v0, v1, lane);
  uint4* xl = reinterpret_cast<uint4*>(wsm);
  float* xsl = reinterpret_cast<float*>(wsm + (size_t)a.runq * 1024);
  const int e = stage_wave<B, XF, SK_UPW>(xv, xl, xsl, lane, nq, tf, ti);
  sk_run<B, ND, ONE>(a, pp, v0, v1, sd[0].tile0, xl, xsl, pow2f(24 - e), lane);
}

// BF: the single code width of the matrices, or 0 (several width segments:
// every workgroup then belongs to one segment, so it stages x for one width)
template <int BF, int ND, bool XF>
__global__ __launch_bounds__(512) void k_gemv_sk(SkArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63;
  const int NW = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int si = 0;
  if (BF == 0)
    while (si + 1 < a.w[0].nseg && (int)blockIdx.x >= a.wg_prefix[si + 1]) ++si;
  SegDev sd[2];
  sd[0] = BF == 0 ? pick(a.w[0], si) : a.w[0].seg[0];
  sd[1] = ND == 2 ? (BF == 0 ? pick(a.w[1], si) : a.w[1].seg[0]) : sd[0];
  // wave gw (of the segment) takes run gw % nch of the segment's tile gw / nch
  // (global units [lo, hi)); waves past the segment's last tile have nothing to do
  const int gw = ((int)blockIdx.x - (BF == 0 ? a.wg_prefix[si] : 0)) * NW + wave;
  const int tl = gw / a.nch, ch = gw - tl * a.nch;
  const bool live = tl < sd[0].tiles;
  const int64_t t0 = (int64_t)(sd[0].tile0 + tl) * a.G4;
  if (!live) return;  // no wave waits for another
  const int64_t lo = t0 + ch * a.G4 / a.nch;
  const int64_t hi = t0 + (ch + 1) * a.G4 / a.nch;
  char* wsm = smem + (size_t)wave * a.runq * 1088;
  if constexpr (BF != 0) {
    sk_body<BF, ND, true, XF>(a, sd, lo, hi, wsm, lane);
  } else {
    if (sd[0].bits == 2) sk_body<2, ND, false, XF>(a, sd, lo, hi, wsm, lane);
    else if (sd[0].bits == 3) sk_body<3, ND, false, XF>(a, sd, lo, hi, wsm, lane);
    else sk_body<4, ND, false, XF>(a, sd, lo, hi, wsm, lane);
  }
}

}  // namespace qg
