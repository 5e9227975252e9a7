// qg_gemv.h -- M = 1 GEMV over uniform b-bit codes on the vector ALU
// (v_dot2_f32_f16), one workgroup per (16-column tile, K slice): the default
// from 256 tiles up, and the gate/up pass of the fused MLP at one row.
//
// Work split.  A workgroup = NW waves on one tile and one K slice of quads
// (512 k each); wave w owns NQ consecutive quads of the slice (the last wave's
// surplus lies outside its buffer ranges and reads nothing).  Each wave loads
// its activations, then its code and scale words quad by quad, all at once;
// stages its activations in an LDS region of its own (qg_stage.h: no wave
// waits for another), and consumes the codes in order.  The workgroup sums its
// waves' partials in LDS in wave order and hands the tile's column sums on:
//   * one K slice: stored directly;
//   * K slices: added into fixed-point column words (qg_common.h), the arrival
//     that completes a word's count stores the result -- exact in any order;
//   * or (pinned, or for the fused pass with K slices) through fp32 partials
//     summed in slice order by the last arrival.
// The fused gate/up pass runs one matrix per workgroup: the two workgroups of
// a tile meet in a per-column exchange word (one K slice) or, with K slices,
// in the partials; the one that completes a column writes h = SiLU(g) * u.
#pragma once
#include "qg_stage.h"

namespace qg {

// one wave's quads: returns this lane's partial (column j = lane & 15, quarter
// lane >> 4) over them, scaled back to true units (times 2^24 for the
// reduction's convention: the caller multiplies nothing more)
// MX: MXFP4 elements (B = 4 layout) or MXFP6 elements (B = 6, two planes):
// decoded to fp16 values of their own (times 2^-14, or 2^-12), x staged with
// its block exponent only, no offset term, and each group's E8M0 scale
// applied as an exact fp32 power of two.
template <int B, int NQ, bool XF, bool MX = false>
__device__ __forceinline__ float gemv_q_wave(const GvArgs& a, const SegDev& sd, int tile, int qw0, int q_end,
                                             char* wsm) {
  // several widths inline one body per width behind a branch: keep the
  // compiler from hoisting the bodies' common loads above it (they would then
  // hold registers through every body)
  __asm__ volatile("" ::: "memory");
  const int lane = threadIdx.x & 63;
  const int G = a.G, G4 = a.G4;
  // wave-uniform, and kept in scalar registers: a descriptor built from a
  // vector register is taken as divergent (each load wrapped in a per-lane
  // descriptor loop)
  const int nvalid = __builtin_amdgcn_readfirstlane(max(0, min(NQ, q_end - qw0)));
  const int ngw = __builtin_amdgcn_readfirstlane(max(0, min(4 * nvalid, G - 4 * qw0)));  // real groups
  const int qb = min(qw0, G4 - 1);
  // ---- loads: activations (NQ units of 8 per lane), then per quad its scales and codes
  uint4 xv[NQ][XIn<XF>::W];
  {
    const char* xb = reinterpret_cast<const char*>(a.x) + (size_t)4 * qb * 128 * (XF ? 4 : 2);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(uniform_ptr(xb), (uint32_t)ngw * 128u * (XF ? 4u : 2u));
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
      if (r >= nvalid) break;  // a wave's surplus quads (past the slice) need nothing
#pragma unroll
      for (int k = 0; k < XIn<XF>::W; ++k) {
        const u4_t q = __builtin_amdgcn_raw_buffer_load_b128(rx, ((uint32_t)(lane + 64 * r) * XIn<XF>::W + k) * 16u, 0, 0);
        xv[r][k] = make_uint4(q.x, q.y, q.z, q.w);
      }
    }
  }
  // the lane's row of the class-factor table, before the code loads
  uint4 tf = make_uint4(0u, 0u, 0u, 0u), ti = tf;
  if constexpr (!MX) stage_tab<B>(lane & 3, tf, ti);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t cw[NQ][4 * B];
  uint2 sc[NQ];
  {
    const size_t qoff = (size_t)tile * G4 + qb;
    const int sq = __builtin_amdgcn_readfirstlane(sd.sq);
    const uint32_t sqb = scale_quad_halves(sq) * 2u;  // scale bytes per quad
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(uniform_ptr(sd.codes) + qoff * (B * 256), (uint32_t)nvalid * (B * 1024u));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(uniform_ptr(sd.scales) + qoff * scale_quad_halves(sq), (uint32_t)nvalid * sqb);
    const uint32_t slane = scale_lane_byte(sq, (uint32_t)lane);
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const u2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, slane + (uint32_t)u * sqb, 0, 0);
      sc[u] = make_uint2(v.x, v.y);
      buffer_quad<B>(rc, (uint32_t)lane, u, cw[u]);
    }
  }
  // ---- the wave's activations -> its LDS region
  uint4* xl = reinterpret_cast<uint4*>(wsm);
  float* xq = reinterpret_cast<float*>(wsm + (size_t)NQ * 1024);
  const int q = lane >> 4;
  float R = 0.0f;
  if constexpr (MX) {
    static_assert((B == 4 || B == 6) && !XF, "MXFP4 / MXFP6 take fp16 x (4-bit layout / two-plane 6-bit layout)");
    const int e = stage_wave_plain<NQ>(xv, xl, lane, nvalid);
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int gl = 4 * u + gi;
        if (gl >= ngw) break;
        uint32_t xp[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 u4 = xl[gl * 16 + q * 4 + v];
          xp[4 * v + 0] = u4.x; xp[4 * v + 1] = u4.y; xp[4 * v + 2] = u4.z; xp[4 * v + 3] = u4.w;
        }
        uint32_t r[16];
        if constexpr (B == 6) decode_group_mx6(cw[u], gi, r);
        else decode_group_mx(cw[u], gi, r);
        float e0 = 0.0f, e1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          e0 = dot2(r[i], xp[i], e0);
          e1 = dot2(r[i + 1], xp[i + 1], e1);
        }
        const uint32_t sw = (gi < 2) ? sc[u].x : sc[u].y;
        const uint32_t eq = ((gi & 1) ? (sw >> 16) : sw) & 0xFFu;  // the lane's block exponent byte
        R = __builtin_fmaf(e8m0_scale(eq, 0), e0 + e1, R);
      }
    }
    return R * pow2f((B == 6 ? 12 : 14) - e);  // the products carry 2^(e - 14) (E2M1) or 2^(e - 12) (E3M2)
  }
  const int e = stage_wave<B, XF, NQ>(xv, xl, xq, lane, nvalid, tf, ti);
  // ---- compute
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int gl = 4 * u + gi;        // group index within the wave's region
      if (gl >= ngw) break;
      uint32_t xp[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 u4 = xl[gl * 16 + q * 4 + v];
        xp[4 * v + 0] = u4.x; xp[4 * v + 1] = u4.y; xp[4 * v + 2] = u4.z; xp[4 * v + 3] = u4.w;
      }
      uint32_t r[16];
      decode_group_classes<B>(cw[u], gi, r);
      // 2^(e-24) * sum x * (c - o) over the lane's 32 weights
      float e0 = xq[gl * 4 + q] * cls_ko<B>(), e1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        e0 = dot2(r[i], xp[i], e0);
        e1 = dot2(r[i + 1], xp[i + 1], e1);
      }
      const uint32_t sw = (gi < 2) ? sc[u].x : sc[u].y;
      const float s = h2f((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
      R = __builtin_fmaf(s, e0 + e1, R);
    }
  }
  return R * pow2f(24 - e);
}

// several widths (BF = 0): the three bodies' registers are allocated together;
// capped so that seven waves fit on each SIMD (the decode shapes' grids of
// 4- and 5-wave workgroups then stay resident; the cap spills a few registers,
// an eight-wave cap spills more and is slower than no cap)
// workgroup `bid` of the launch described by `a` (a tile and K slice of one
// matrix, or of one of the fused pass's two)
template <int NQ, int BF, bool XF>
__device__ __forceinline__ void gemv_q_block(const GvArgs& a, int bid, char* smem) {
  const int NW = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.S, G4 = a.G4;
  // fused pass: the two matrices are taken as extra K slices, slice index
  // dm * S + s for matrix dm; the last arrival of a tile sums each matrix's
  // slices and applies SiLU(g) * u
  const int P = a.pair ? 2 : 1;
  const int SP = S * P;
  const int sx = bid % SP, tsg = bid / SP;
  const int dm = sx / S, s = sx - dm * S;
  // single-width handles have one segment: no data-dependent argument loads
  int si = 0;
  if (BF == 0)
    while (si + 1 < a.w[0].nseg && tsg >= a.ts_prefix[si + 1]) ++si;
  SegDev sd;
  {
    const SegDev s0 = BF == 0 ? pick(a.w[0], si) : a.w[0].seg[0];
    const SegDev s1 = BF == 0 ? pick(a.w[1], si) : a.w[1].seg[0];
    sd = (P == 2 && dm == 1) ? s1 : s0;
  }
  const int tile = BF == 0 ? tsg - a.ts_prefix[si] : tsg;
  const int q_beg = (int)((int64_t)s * G4 / S), q_end = (int)((int64_t)(s + 1) * G4 / S);
  const int pc = 16 * (sd.tile0 + tile) + (tid & 15);
  // output column: the padded column itself for one width (no padding then);
  // with several widths looked up here, so the lookup is not on the tail
  int n_out = pc;
  if (BF == 0) n_out = tid < 16 ? a.w[0].col_map[pc] : -1;
  // this wave's LDS region, then the cross-wave partials and a flag
  char* wsm = smem + (size_t)wave * NQ * M1_WAVE_LDS;
  float* red = reinterpret_cast<float*>(smem + (size_t)NW * NQ * M1_WAVE_LDS);
  int* flag = reinterpret_cast<int*>(red + NW * 16);
  const int qw0 = q_beg + wave * NQ;
  float R;
  const int bits = sd.bits;
  if constexpr (BF == 5) R = gemv_q_wave<4, NQ, XF, true>(a, sd, tile, qw0, q_end, wsm);  // MXFP4
  else if constexpr (BF == 6) R = gemv_q_wave<6, NQ, XF, true>(a, sd, tile, qw0, q_end, wsm);  // MXFP6
  else if (BF == 2 || (BF == 0 && bits == 2)) R = gemv_q_wave<2, NQ, XF>(a, sd, tile, qw0, q_end, wsm);
  else if (BF == 3 || (BF == 0 && bits == 3)) R = gemv_q_wave<3, NQ, XF>(a, sd, tile, qw0, q_end, wsm);
  else R = gemv_q_wave<4, NQ, XF>(a, sd, tile, qw0, q_end, wsm);
  {
    float v = R;
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (lane < 16) red[wave * 16 + lane] = v;
  }
  __syncthreads();
  const bool mine = tid < 16;
  float v = 0.0f;
  if (mine)
    for (int w = 0; w < NW; ++w) v += red[w * 16 + tid];
  if (P == 2 && S == 1) {
    // one K slice: the two workgroups of a tile meet in a per-column word.
    // Each swaps in (matrix + 1) << 32 | its fp32 bits; the one that gets a
    // non-zero word back holds both values, writes SiLU(g) * u and re-arms the
    // word.  One round trip per workgroup, and the result does not depend on
    // which matrix arrives first.
    if (mine) {
      const unsigned long long w = ((unsigned long long)(dm + 1) << 32) | __float_as_uint(v);
      const unsigned long long o = __hip_atomic_exchange(a.xw + pc, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (o != 0ull) {
        const float other = __uint_as_float((uint32_t)o);
        const float g = dm == 0 ? v : other, u = dm == 0 ? other : v;
        fx_rearm(a.xw + pc);
        if (n_out >= 0) store_y(a.y, n_out, silu_mul(g, u), a.yf32);
      }
    }
    return;
  }
  if (P == 1 && S > 1 && a.fx) {
    // K slices meet in fixed-point words: one atomic round trip; the arrival
    // that completes the count stores the result and re-arms the word
    if (mine) {
      unsigned long long* w = a.xw + pc;
      const unsigned long long part = fx_word(v);
      const unsigned long long before = fx_add(w, part);
      if (fx_count(before) == S - 1) {
        if (n_out >= 0) store_y(a.y, n_out, fx_value(before + part), a.yf32);
        fx_rearm(w);
      }
    }
    return;
  }
  if (SP > 1) {
    // partials [matrix][slice][NP]; the arriving workgroup adds its own value
    // in its slot of the fixed order instead of reading it back
    if (mine) st_partial(a.partial + (size_t)(dm * S + s) * a.NP + pc, v);
    if (!splitk_last(a.counters + tsg, SP, flag)) return;
    if (mine) {
      float t[2] = {0.0f, 0.0f};
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        if (d == 1 && P == 1) break;
        t[d] = sum_partials(a.partial + (size_t)(d * S) * a.NP + pc, (size_t)a.NP, S, d == dm ? s : -1, v);
      }
      v = P == 2 ? silu_mul(t[0], t[1]) : t[0];
    }
  }
  if (mine && n_out >= 0) store_y(a.y, n_out, v, a.yf32);
}

template <int NQ, int BF, bool XF>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(BF == 0 && NQ <= 2 ? 7 : 1)))
void k_gemv_q(GvArgs a) {
  extern __shared__ __align__(16) char smem[];
  gemv_q_block<NQ, BF, XF>(a, blockIdx.x, smem);
}

// Several independent M = 1 products in one launch: task t owns workgroups
// [wg0[t], wg0[t + 1]) and runs exactly as its own launch would (same plan
// shape: every task is planned for the launch's NQ and NW).
template <int NQ, int BF>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(BF == 0 && NQ <= 2 ? 7 : 1)))
void k_gemv_batch(GvBatch b) {
  extern __shared__ __align__(16) char smem[];
  const int bid = blockIdx.x;
  int t = 0;
  while (t + 1 < b.n && bid >= b.wg0[t + 1]) ++t;
  gemv_q_block<NQ, BF, false>(b.task[t], bid - b.wg0[t], smem);
}

}  // namespace qg
