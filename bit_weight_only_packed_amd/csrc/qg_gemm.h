// qg_gemm.h -- 2..32-row skinny GEMM over uniform b-bit codes on the matrix
// cores (v_mfma_f32_16x16x32_f16): the speculative-decode verify product.
//
// Work split.  A workgroup owns a tile set (NW waves x T 16-column tiles) and a
// K slice of at most QMAX quads (512 k each); its waves share the slice of x,
// which the workgroup stages once in LDS, and each wave multiplies it into its
// own T tiles.  So x is read from L2 once per tile set and slice (not once per
// wave), and each A fragment a wave reads from LDS serves T tiles.  Each wave
// first issues its share of the x loads, then the loads of all its codes and
// scales (at most QMAX * T * B 16-byte loads per lane), waits for its x loads
// alone, stages them, and then consumes the codes in order.
//
// Arithmetic.  Codes are decoded with one AND per pair at their "class" bit
// offsets (value c * 2^(class-24), exact fp16) and form the B operand; x is
// staged already multiplied by 2^-class of the code position it meets, so every
// product is c * x * 2^-24 (as in the M = 1 GEMV).  Each group's chain starts
// from the code offset term -o * 2^-24 * sum_k x[m][k], from per-row group sums
// staged beside x, so the chain yields 2^-24 * sum x * (c - o); the fp16 scale
// multiplies it into the fp32 accumulator.
//
// K slices meet in an fp32 workspace: every workgroup writes its partials,
// and the one that arrives last at the tile set's counter adds the slices in
// slice order and stores the fp16 result, so the output does not depend on the
// order of arrival.
#pragma once
#include "qg_kernels.h"

namespace qg {

struct GmArgs {
  WSet w[2];                 // w[1]: up matrix of the fused gate/up pass
  const uint16_t* x;         // [M][K] fp16
  uint16_t* y;               // [M][ldy] fp16
  float* partial;            // [ND][S][M][NP] fp32 (S > 1)
  int* counters;             // one per tile set, zero between launches
  int M, K, G, G4, ldy, NP, S, NW;
  int ts_prefix[MAX_SEG + 1];  // tile sets before each segment
};

// LDS: x as [quad][group][row] rows of 128 fp16 (256 B); position p of row r
// holds the row's 16-byte chunk p ^ (r & 15), so the 16 rows of an A fragment
// read land on distinct banks.  Then the per-row group sums as
// [quad][group][row] floats, then the split-K flag.
__host__ __device__ constexpr int gm_rows(int MT) { return 16 * MT; }
__host__ __device__ constexpr size_t gm_x_bytes(int MT, int QMAX) { return (size_t)QMAX * 4 * gm_rows(MT) * 256; }
__host__ __device__ constexpr size_t gm_lds_bytes(int MT, int QMAX) {
  return gm_x_bytes(MT, QMAX) + (size_t)QMAX * 4 * gm_rows(MT) * 4 + 16;
}

// x staging, in two halves around the code loads.  16 consecutive threads
// hold one 128-element group row (one uint4 each); thread t takes uint4
// t, t + blockDim, ... of the QMAX * 4 * R rows (rows past M, quads past nq
// and groups past G stay zero), at most GM_XR of them (so 4 or more waves per
// workgroup).
constexpr int GM_XR = 16;

template <int MT, int QMAX>
__device__ __forceinline__ void gm_x_load(const GmArgs& a, int q0, int nq, uint4 (&xr)[GM_XR]) {
  constexpr int R = gm_rows(MT);
  const int total = R * QMAX * 64;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(uniform_ptr(a.x), (uint32_t)a.M * a.K * 2u);
#pragma unroll
  for (int it = 0; it < GM_XR; ++it) {
    if (it * (int)blockDim.x >= total) break;
    const int i = threadIdx.x + it * (int)blockDim.x;
    const int p = i & 15, gr = i >> 4;
    const int gi = gr & 3, qi = (gr >> 2) % QMAX, m = (gr >> 2) / QMAX;
    const int g = 4 * (q0 + qi) + gi;
    const bool ok = i < total && m < a.M && qi < nq && g < a.G;
    const uint32_t voff = ok ? (uint32_t)(((size_t)m * a.K + (size_t)g * 128 + p * 8) * 2) : 0xFFFFFFF0u;
    const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, voff, 0, 0);
    xr[it] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

template <int B, int MT, int QMAX>
__device__ __forceinline__ void gm_x_store(const uint4 (&xr)[GM_XR], char* smem) {
  constexpr int R = gm_rows(MT);
  const int total = R * QMAX * 64;
  float* xs = reinterpret_cast<float*>(smem + gm_x_bytes(MT, QMAX));
  const int pos = threadIdx.x & 3;  // uint4 position within a 32-element quarter
  uint32_t f[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t f0 = class_scale_pair<B>(e), f1 = class_scale_pair<B>(4 + e);
    const uint32_t f2 = class_scale_pair<B>(8 + e), f3 = class_scale_pair<B>(12 + e);
    f[e] = pos == 0 ? f0 : pos == 1 ? f1 : pos == 2 ? f2 : f3;
  }
  const uint32_t ones = 0x3C003C00u;
#pragma unroll
  for (int it = 0; it < GM_XR; ++it) {
    if (it * (int)blockDim.x >= total) break;  // whole waves (total and blockDim are multiples of 64)
    const int i = threadIdx.x + it * (int)blockDim.x;
    const int p = i & 15, gr = i >> 4;
    const int gi = gr & 3, qi = (gr >> 2) % QMAX, m = (gr >> 2) / QMAX;
    const uint4 v = xr[it];
    float ps = dot2(v.x, ones, 0.0f);
    ps = dot2(v.y, ones, ps);
    ps = dot2(v.z, ones, ps);
    ps = dot2(v.w, ones, ps);
    ps += dpp_row_ror<8>(ps);
    ps += dpp_row_ror<4>(ps);
    ps += dpp_xor2(ps);
    ps += dpp_xor1(ps);
    const int row = (qi * 4 + gi) * R + m;
    if (i < total) {
      *reinterpret_cast<uint4*>(smem + (size_t)row * 256 + ((p ^ (row & 15)) * 16)) =
          make_uint4(pk_mul_f16(v.x, f[0]), pk_mul_f16(v.y, f[1]), pk_mul_f16(v.z, f[2]), pk_mul_f16(v.w, f[3]));
      if (p == 0) xs[row] = ps;
    }
  }
}

template <int B, int T, int QMAX, int ND>
struct GmCodes {
  uint32_t cw[QMAX][ND][T][4 * B];
  uint2 sc[QMAX][ND][T];
};

template <int B, int T, int MT, int QMAX, int ND>
__device__ __forceinline__ void gm_body(const GmArgs& a, const SegDev (&sd)[2], int tl0, int q0, int nq, char* smem,
                                        f4_t (&acc)[ND][T][MT]) {
  constexpr int R = gm_rows(MT);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G4 = a.G4;
  // ---- this thread's share of x first, then every code and scale load of this wave
  uint4 xr[GM_XR];
  gm_x_load<MT, QMAX>(a, q0, nq, xr);
  GmCodes<B, T, QMAX, ND> c;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const bool live = tl0 + t < sd[d].tiles;
      const size_t qb = (size_t)min(tl0 + t, sd[d].tiles - 1) * G4 + q0;
      const __amdgpu_buffer_rsrc_t rc =
          make_rsrc(uniform_ptr(sd[d].codes) + qb * (B * 256), live ? (uint32_t)nq * (B * 1024u) : 0u);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(uniform_ptr(sd[d].scales) + qb * 64, live ? (uint32_t)nq * 128u : 0u);
#pragma unroll
      for (int qi = 0; qi < QMAX; ++qi) {
        const u2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, (uint32_t)(lane & 15) * 8u, (uint32_t)qi * 128u, 0);
        c.sc[qi][d][t] = make_uint2(v.x, v.y);
        buffer_quad<B>(rc, (uint32_t)lane, qi, c.cw[qi][d][t]);
      }
    }
  gm_x_store<B, MT, QMAX>(xr, smem);  // waits for the x loads only (they were issued first)
  lds_barrier();
  const float* xs = reinterpret_cast<const float*>(smem + gm_x_bytes(MT, QMAX));
  const int kq = lane >> 4, m16 = lane & 15;
  const float ko = -0.5f * (float)((1 << B) - 1) * 5.9604644775390625e-08f;  // -o * 2^-24
#pragma unroll
  for (int qi = 0; qi < QMAX; ++qi) {
    if (qi >= nq) break;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      h8_t A[MT][4];
      f4_t C0[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const char* rowp = smem + (size_t)((qi * 4 + gi) * R + 16 * mt + m16) * 256;
#pragma unroll
        for (int v = 0; v < 4; ++v) A[mt][v] = *reinterpret_cast<const h8_t*>(rowp + (((4 * kq + v) ^ m16) * 16));
        // chain start: the code offset times the rows' group sums (rows 4kq + e)
        const f4_t s4 = *reinterpret_cast<const f4_t*>(xs + (qi * 4 + gi) * R + 16 * mt + 4 * kq);
        C0[mt] = s4 * ko;
      }
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int t = 0; t < T; ++t) {
          uint32_t g3[B];
          quad_group<B>(c.cw[qi][d][t], gi, g3);
          uint32_t r[16];
          decode_classes<B>(g3, r);
          const uint32_t sw = (gi < 2) ? c.sc[qi][d][t].x : c.sc[qi][d][t].y;
          const float s = h2f((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            f4_t cc = C0[mt];
#pragma unroll
            for (int v = 0; v < 4; ++v) cc = mfma16(A[mt][v], as_h8(r[4 * v], r[4 * v + 1], r[4 * v + 2], r[4 * v + 3]), cc);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[d][t][mt][e] = __builtin_fmaf(s, cc[e], acc[d][t][mt][e]);
          }
        }
    }
  }
}

// BF: the single code width of the matrices, or 0 (several width segments;
// a tile set never spans two)
template <int T, int MT, int QMAX, bool DUAL, int BF>
__global__ __launch_bounds__(512) void k_gemm_v2(GmArgs a) {
  extern __shared__ __align__(16) char smem[];
  constexpr int ND = DUAL ? 2 : 1;
  const int NW = a.NW;
  const int lane = threadIdx.x & 63;
  (void)NW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = a.S, G4 = a.G4;
  const int s = blockIdx.x % S, tsg = blockIdx.x / S;
  int si = 0;
  if (BF == 0)
    while (si + 1 < a.w[0].nseg && tsg >= a.ts_prefix[si + 1]) ++si;
  SegDev sd[2];
  sd[0] = BF == 0 ? pick(a.w[0], si) : a.w[0].seg[0];
  sd[1] = DUAL ? (BF == 0 ? pick(a.w[1], si) : a.w[1].seg[0]) : sd[0];
  const int ts_local = BF == 0 ? tsg - a.ts_prefix[si] : tsg;
  const int tl0 = (ts_local * NW + wave) * T;  // this wave's first tile in the segment
  const int q0 = (int)((int64_t)s * G4 / S), q1 = (int)((int64_t)(s + 1) * G4 / S);
  f4_t acc[ND][T][MT];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[d][t][mt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int bits = sd[0].bits;
  if (BF == 2 || (BF == 0 && bits == 2)) gm_body<2, T, MT, QMAX, ND>(a, sd, tl0, q0, q1 - q0, smem, acc);
  else if (BF == 3 || (BF == 0 && bits == 3)) gm_body<3, T, MT, QMAX, ND>(a, sd, tl0, q0, q1 - q0, smem, acc);
  else gm_body<4, T, MT, QMAX, ND>(a, sd, tl0, q0, q1 - q0, smem, acc);
  // ---- epilogue: lane holds rows 16mt + 4(lane >> 4) + e of column (lane & 15) of each tile
  const int mq = lane >> 4, j = lane & 15;
  int* flag = reinterpret_cast<int*>(smem + gm_lds_bytes(MT, QMAX) - 16);
  if (S > 1) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (tl0 + t >= sd[0].tiles) continue;
      const int pc = 16 * (sd[0].tile0 + tl0 + t) + j;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * mt + 4 * mq + e;
          if (m >= a.M) continue;
#pragma unroll
          for (int d = 0; d < ND; ++d)
            st_partial(a.partial + ((size_t)(d * S + s) * a.M + m) * a.NP + pc, acc[d][t][mt][e] * 16777216.0f);  // 2^24
        }
    }
    if (!splitk_last(a.counters + tsg, S, flag)) return;
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (tl0 + t >= sd[0].tiles) continue;
    const int pc = 16 * (sd[0].tile0 + tl0 + t) + j;
    const int n = BF != 0 ? pc : a.w[0].col_map[pc];  // one width: no padding, identity
    if (n < 0) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mt + 4 * mq + e;
        if (m >= a.M) continue;
        float v[ND];
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          if (S > 1) {
            v[d] = sum_partials(a.partial + ((size_t)(d * S) * a.M + m) * a.NP + pc, (size_t)a.M * a.NP, S);
          } else {
            v[d] = acc[d][t][mt][e] * 16777216.0f;
          }
        }
        a.y[(size_t)m * a.ldy + n] = f2h(DUAL ? silu_mul(v[0], v[1]) : v[0]);
      }
  }
}

}  // namespace qg
