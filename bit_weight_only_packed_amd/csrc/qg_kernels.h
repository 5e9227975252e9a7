// qg_kernels.h -- HIP kernels for gfx950: weight re-layout, the M=1 GEMV (vector
// ALU, fp16 dot2), the 2..32-row skinny GEMM (MFMA 16x16x32 f16), the fixed-order
// split-K reduction and the checking kernels.  Layout and decode: qg_decode.h.
//
// Arithmetic (uniform b-bit codes, offset o = (2^b - 1)/2, group g of 128 k):
//   y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] * (c[n][k] - o)
// The GEMV forms sum x*c per group from the exact subnormal code values, adds
// the offset term as -o * s * sum_{k in g} x[k] (activation sums precomputed
// once per workgroup) and applies the scale per group, all in fp32.  The MFMA
// path feeds codes at scale 2^-23 and starts every group's accumulation from
// the offset product x * (-o * 2^-23), so each group's MFMA chain yields
// 2^-23 * sum x*(c - o) directly; the scale is applied per group in fp32.
// Workgroups never share an output element except through the split-K
// workspace, whose partials are summed in slice order: results are
// bit-reproducible.
#pragma once
#include "qg_decode.h"

namespace qg {

constexpr int MAX_SEG = 3;

struct SegDev {
  const uint32_t* codes;   // device layout, [tiles][G][64][bits]
  const uint16_t* scales;  // [tiles][G][16]
  int bits;                // 2, 3 or 4
  int tiles;               // 16-column tiles in this segment
  int tile0;               // index of the first tile in the handle's padded column space
};

struct WSet {
  SegDev seg[MAX_SEG];
  int nseg;
  const int32_t* col_map;  // [16 * total tiles]: original column of each padded column, or -1
};

struct RunArgs {
  WSet w[2];               // w[1] only for the fused gate/up pass
  const uint16_t* x;       // [M][K] fp16
  uint16_t* y;             // [M][ldy] fp16 (fused pass: h)
  float* partial;          // [2][S][M][NP] fp32 when S > 1
  int M, K, G, ldy, NP;
  int T, S;                // tiles per workgroup, K slices across workgroups
  int ts_prefix[MAX_SEG + 1];  // prefix sums of tile-sets per segment
};

__device__ __forceinline__ SegDev pick(const WSet& w, int si) {
  SegDev s = w.seg[0];
  if (si == 1) s = w.seg[1];
  if (si == 2) s = w.seg[2];
  return s;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ---------------------------------------------------------------------------
// create-time re-layout: canonical stream -> device layout (one thread per lane-slot)
// ---------------------------------------------------------------------------
__global__ void k_repack_uniform(const uint32_t* __restrict__ canon, const int64_t* __restrict__ row_off,
                                 const uint16_t* __restrict__ scales_in, const int32_t* __restrict__ cols,
                                 int bits, int tiles, int G, uint32_t* __restrict__ dcodes,
                                 uint16_t* __restrict__ dscales) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)tiles * G * 64;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  const int64_t tg = gid >> 6;              // tile * G + g
  const int g = (int)(tg % G);
  const int t = (int)(tg / G);
  const int j = lane & 15, q = lane >> 4;
  const int n = cols[16 * t + j];
  uint32_t out[4] = {0u, 0u, 0u, 0u};
  if (n >= 0) {
    const uint32_t* src = canon + row_off[n] + (int64_t)g * 4 * bits + q * bits;
    uint32_t in[4] = {0u, 0u, 0u, 0u};
    for (int u = 0; u < bits; ++u) in[u] = src[u];
    uint32_t c[32];
    for (int tt = 0; tt < 32; ++tt) {      // code tt = stream bits [bits*tt, bits*tt + bits)
      const int b0 = bits * tt;
      uint64_t two = (uint64_t)in[b0 >> 5] | ((b0 >> 5) + 1 < 4 ? ((uint64_t)in[(b0 >> 5) + 1] << 32) : 0ull);
      c[tt] = (uint32_t)(two >> (b0 & 31)) & ((1u << bits) - 1u);
    }
    for (int i = 0; i < 16; ++i) {
      const uint32_t lo = c[2 * i], hi = c[2 * i + 1];
      if (bits == 3 && i == 15) {
        for (int u = 0; u < 3; ++u) out[u] |= (((lo >> u) & 1u) << 15) | (((hi >> u) & 1u) << 31);
        continue;
      }
      int wd, off;
      if (bits == 2) { wd = i / 8; off = 2 * (i % 8); }
      else if (bits == 4) { wd = i / 4; off = 4 * (i % 4); }
      else { wd = i / 5; off = 3 * (i % 5); }
      out[wd] |= (lo << off) | (hi << (16 + off));
    }
  }
  uint32_t* dst = dcodes + gid * bits;
  for (int u = 0; u < bits; ++u) dst[u] = out[u];
  if (q == 0) dscales[tg * 16 + j] = (n >= 0) ? scales_in[(int64_t)n * G + g] : (uint16_t)0;
}

// ---------------------------------------------------------------------------
// M = 1 GEMV (VALU).  Workgroup = NW waves on T column tiles of one segment and
// one K slice; waves split the slice's groups; x slice and its per-quarter sums
// live in LDS.
// ---------------------------------------------------------------------------
template <int B, int T, bool DUAL>
__device__ __forceinline__ void gemv_m1_body(const SegDev& sg, const SegDev& sg2, int tl0, int G, int gw0,
                                             int gw1, int g_beg, const uint4* __restrict__ xl,
                                             const float* __restrict__ xs, int lane, float (&R)[2][T],
                                             float (&Ro)[2][T]) {
  constexpr int CH = 4;
  const int q = lane >> 4, j = lane & 15;
  using P = Pair<B>;
  for (int g = gw0; g < gw1; g += CH) {
    uint32_t cw[DUAL ? 2 : 1][CH][T][B];
    uint16_t sc[DUAL ? 2 : 1][CH][T];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int d = 0; d < (DUAL ? 2 : 1); ++d) {
          const SegDev& S_ = d ? sg2 : sg;
          const int tl = tl0 + t;
          if (g + c < gw1 && tl < S_.tiles) {
            const int64_t tg = (int64_t)tl * G + g + c;
            load_words<B>(S_.codes + (tg * 64 + lane) * B, cw[d][c][t]);
            sc[d][c][t] = S_.scales[tg * 16 + j];
          } else {
#pragma unroll
            for (int u = 0; u < B; ++u) cw[d][c][t][u] = 0u;
            sc[d][c][t] = 0;
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (g + c >= gw1) break;
      const int gl = g + c - g_beg;
      uint32_t xp[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 u4 = xl[gl * 16 + q * 4 + v];
        xp[4 * v + 0] = u4.x; xp[4 * v + 1] = u4.y; xp[4 * v + 2] = u4.z; xp[4 * v + 3] = u4.w;
      }
      const float xsum = xs[gl * 4 + q];
#pragma unroll
      for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int d = 0; d < (DUAL ? 2 : 1); ++d) {
          uint32_t r[16];
          decode_classes<B>(cw[d][c][t], r);
          float acc[9];
#pragma unroll
          for (int p = 0; p < 9; ++p) acc[p] = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[P::cls(i)] = dot2(r[i], xp[i], acc[P::cls(i)]);
          // sum x*c * 2^-24 = sum_p acc_p * 2^-p
          float sxc = acc[0];
#pragma unroll
          for (int p = 1; p < 9; ++p) {
            bool used = false;
#pragma unroll
            for (int i = 0; i < 16; ++i) used |= (P::cls(i) == p);
            if (used) sxc = __builtin_fmaf(acc[p], 1.0f / (float)(1 << p), sxc);
          }
          const float s = h2f(sc[d][c][t]);
          R[d][t] = __builtin_fmaf(s, sxc, R[d][t]);
          Ro[d][t] = __builtin_fmaf(s, xsum, Ro[d][t]);
        }
      }
    }
  }
}

template <int T, bool DUAL>
__global__ __launch_bounds__(512) void k_gemv_m1(RunArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int NW = blockDim.x >> 6;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int S = a.S, G = a.G;
  const int s = blockIdx.x % S, tsg = blockIdx.x / S;
  int si = 0;
  while (si + 1 < a.w[0].nseg && tsg >= a.ts_prefix[si + 1]) ++si;
  const SegDev sg = pick(a.w[0], si);
  const SegDev sg2 = DUAL ? pick(a.w[1], si) : sg;
  const int tl0 = (tsg - a.ts_prefix[si]) * T;
  const int g_beg = (int)((int64_t)s * G / S), g_end = (int)((int64_t)(s + 1) * G / S);
  const int Gs = g_end - g_beg;

  // stage x[g_beg*128, g_end*128) and its 32-element partial sums
  uint4* xl = reinterpret_cast<uint4*>(smem);
  float* xs = reinterpret_cast<float*>(smem + (size_t)Gs * 256);
  float* red = xs + Gs * 4;
  const uint4* xg = reinterpret_cast<const uint4*>(a.x + (size_t)g_beg * 128);
  for (int i = tid; i < Gs * 16; i += blockDim.x) xl[i] = xg[i];
  __syncthreads();
  for (int i = tid; i < Gs * 4; i += blockDim.x) {
    const _Float16* h = reinterpret_cast<const _Float16*>(xl) + i * 32;
    float acc = 0.0f;
    for (int e = 0; e < 32; ++e) acc += (float)h[e];
    xs[i] = acc;
  }
  __syncthreads();

  const int gw0 = g_beg + (int)((int64_t)wave * Gs / NW);
  const int gw1 = g_beg + (int)((int64_t)(wave + 1) * Gs / NW);
  float R[2][T], Ro[2][T];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t) R[d][t] = Ro[d][t] = 0.0f;

  switch (sg.bits) {
    case 2: gemv_m1_body<2, T, DUAL>(sg, sg2, tl0, G, gw0, gw1, g_beg, xl, xs, lane, R, Ro); break;
    case 3: gemv_m1_body<3, T, DUAL>(sg, sg2, tl0, G, gw0, gw1, g_beg, xl, xs, lane, R, Ro); break;
    default: gemv_m1_body<4, T, DUAL>(sg, sg2, tl0, G, gw0, gw1, g_beg, xl, xs, lane, R, Ro); break;
  }
  const float o = 0.5f * (float)((1 << sg.bits) - 1);
  constexpr int ND = DUAL ? 2 : 1;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float v = __builtin_fmaf(R[d][t], 16777216.0f, -o * Ro[d][t]);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) red[((d * NW + wave) * T + t) * 16 + lane] = v;
    }
  __syncthreads();
  if (tid < T * 16) {
    const int t = tid >> 4, jj = tid & 15;
    const int tl = tl0 + t;
    if (tl < sg.tiles) {
      float v[2] = {0.0f, 0.0f};
#pragma unroll
      for (int d = 0; d < ND; ++d)
        for (int w = 0; w < NW; ++w) v[d] += red[((d * NW + w) * T + t) * 16 + jj];
      const int pc = 16 * (sg.tile0 + tl) + jj;
      if (S == 1) {
        const int n = a.w[0].col_map[pc];
        if (n >= 0) a.y[n] = f2h(DUAL ? silu_mul(v[0], v[1]) : v[0]);
      } else {
#pragma unroll
        for (int d = 0; d < ND; ++d) a.partial[((size_t)(d * S + s) * a.M + 0) * a.NP + pc] = v[d];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2..32-row skinny GEMM (MFMA 16x16x32 f16).  Workgroup = NW waves on T tiles;
// waves split the K slice; per group each wave loads its A fragments (MT
// 16-row tiles of x) once and reuses them for all T tiles.
// ---------------------------------------------------------------------------
template <int B, int T, int MT, bool DUAL>
__device__ __forceinline__ void mfma_body(const SegDev& sg, const SegDev& sg2, int tl0, int G, int gw0,
                                          int gw1, const uint16_t* __restrict__ x, int M, int K, int lane,
                                          f4_t (&R)[2][T][MT]) {
  const int q = lane >> 4, j = lane & 15;
  const uint32_t op = off1_offset_pair<B>();
  const h8_t boff = as_h8(op, op, op, op);
  constexpr int ND = DUAL ? 2 : 1;
  for (int g = gw0; g < gw1; ++g) {
    uint32_t cw[ND][T][B];
    uint16_t sc[ND][T];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const SegDev& S_ = d ? sg2 : sg;
        const int tl = tl0 + t;
        if (tl < S_.tiles) {
          const int64_t tg = (int64_t)tl * G + g;
          load_words<B>(S_.codes + (tg * 64 + lane) * B, cw[d][t]);
          sc[d][t] = S_.scales[tg * 16 + j];
        } else {
#pragma unroll
          for (int u = 0; u < B; ++u) cw[d][t][u] = 0u;
          sc[d][t] = 0;
        }
      }
    h8_t A[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = 16 * mt + j;
      if (row < M) {
        const uint4* px = reinterpret_cast<const uint4*>(x + (size_t)row * K + (size_t)g * 128 + 32 * q);
#pragma unroll
        for (int v = 0; v < 4; ++v) A[mt][v] = __builtin_bit_cast(h8_t, px[v]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) A[mt][v] = __builtin_bit_cast(h8_t, make_uint4(0u, 0u, 0u, 0u));
      }
    }
    f4_t Coff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int v = 0; v < 4; ++v) c = mfma16(A[mt][v], boff, c);
      Coff[mt] = c;
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        uint32_t r[16];
        decode_off1<B>(cw[d][t], r);
        const float s = h2f(sc[d][t]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f4_t c = Coff[mt];
#pragma unroll
          for (int v = 0; v < 4; ++v) c = mfma16(A[mt][v], as_h8(r[4 * v], r[4 * v + 1], r[4 * v + 2], r[4 * v + 3]), c);
#pragma unroll
          for (int e = 0; e < 4; ++e) R[d][t][mt][e] = __builtin_fmaf(s, c[e], R[d][t][mt][e]);
        }
      }
  }
}

template <int T, int MT, bool DUAL>
__global__ __launch_bounds__(512) void k_gemm_mfma(RunArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int NW = blockDim.x >> 6;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int S = a.S, G = a.G;
  const int s = blockIdx.x % S, tsg = blockIdx.x / S;
  int si = 0;
  while (si + 1 < a.w[0].nseg && tsg >= a.ts_prefix[si + 1]) ++si;
  const SegDev sg = pick(a.w[0], si);
  const SegDev sg2 = DUAL ? pick(a.w[1], si) : sg;
  const int tl0 = (tsg - a.ts_prefix[si]) * T;
  const int g_beg = (int)((int64_t)s * G / S), g_end = (int)((int64_t)(s + 1) * G / S);
  const int Gs = g_end - g_beg;
  const int gw0 = g_beg + (int)((int64_t)wave * Gs / NW);
  const int gw1 = g_beg + (int)((int64_t)(wave + 1) * Gs / NW);
  constexpr int ND = DUAL ? 2 : 1;
  f4_t R[2][T][MT];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) R[d][t][mt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  switch (sg.bits) {
    case 2: mfma_body<2, T, MT, DUAL>(sg, sg2, tl0, G, gw0, gw1, a.x, a.M, a.K, lane, R); break;
    case 3: mfma_body<3, T, MT, DUAL>(sg, sg2, tl0, G, gw0, gw1, a.x, a.M, a.K, lane, R); break;
    default: mfma_body<4, T, MT, DUAL>(sg, sg2, tl0, G, gw0, gw1, a.x, a.M, a.K, lane, R); break;
  }
  // cross-wave reduction in LDS, fixed wave order
  float* red = reinterpret_cast<float*>(smem);
  constexpr int PER = T * MT * 4;  // floats per lane per matrix
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          red[(((size_t)(d * NW + wave) * PER) + (t * MT + mt) * 4 + e) * 64 + lane] = R[d][t][mt][e];
  __syncthreads();
  const int total = PER * 64;
  for (int idx = tid; idx < total; idx += blockDim.x) {
    const int ln = idx & 63, rest = idx >> 6;
    const int e = rest & 3, tm = rest >> 2;
    const int mt = tm % MT, t = tm / MT;
    const int row = 16 * mt + 4 * (ln >> 4) + e;
    const int tl = tl0 + t;
    if (row >= a.M || tl >= sg.tiles) continue;
    float v[2] = {0.0f, 0.0f};
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      for (int w = 0; w < NW; ++w) v[d] += red[((size_t)(d * NW + w) * PER + rest) * 64 + ln];
      v[d] *= 8388608.0f;  // 2^23
    }
    const int pc = 16 * (sg.tile0 + tl) + (ln & 15);
    if (S == 1) {
      const int n = a.w[0].col_map[pc];
      if (n >= 0) a.y[(size_t)row * a.ldy + n] = f2h(DUAL ? silu_mul(v[0], v[1]) : v[0]);
    } else {
#pragma unroll
      for (int d = 0; d < ND; ++d) a.partial[((size_t)(d * S + s) * a.M + row) * a.NP + pc] = v[d];
    }
  }
}

// ---------------------------------------------------------------------------
// split-K epilogue: sum the S slices in slice order, fp16 store (or SiLU(g)*u)
// ---------------------------------------------------------------------------
template <bool DUAL>
__global__ void k_splitk_reduce(const float* __restrict__ partial, int S, int M, int NP,
                                const int32_t* __restrict__ col_map, uint16_t* __restrict__ y, int ldy) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * NP) return;
  const int m = (int)(idx / NP), pc = (int)(idx % NP);
  const int n = col_map[pc];
  if (n < 0) return;
  float v = 0.0f;
  for (int s = 0; s < S; ++s) v += partial[((size_t)s * M + m) * NP + pc];
  if (DUAL) {
    float u = 0.0f;
    for (int s = 0; s < S; ++s) u += partial[((size_t)(S + s) * M + m) * NP + pc];
    v = silu_mul(v, u);
  }
  y[(size_t)m * ldy + n] = f2h(v);
}

// ---------------------------------------------------------------------------
// checking kernels: the GEMV decode of every lane-slot, written back in [N][K]
// ---------------------------------------------------------------------------
template <int B>
__device__ __forceinline__ void debug_slot(const SegDev& sg, const int32_t* col_map, int G, int K, int64_t gid,
                                           int32_t* codes, float* w, uint16_t* q16) {
  using P = Pair<B>;
  const int lane = (int)(gid & 63);
  const int64_t tg = gid >> 6;
  const int g = (int)(tg % G), tl = (int)(tg / G);
  const int j = lane & 15, q = lane >> 4;
  const int n = col_map[16 * (sg.tile0 + tl) + j];
  if (n < 0) return;
  uint32_t cw[B];
  load_words<B>(sg.codes + (tg * 64 + lane) * B, cw);
  uint32_t r[16];
  decode_classes<B>(cw, r);
  const float s = h2f(sg.scales[tg * 16 + j]);
  const float o = 0.5f * (float)((1 << B) - 1);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int p = P::cls(i);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = (int)((r[i] >> (16 * h + p)) & P::mask());
      const int64_t k = (int64_t)g * 128 + 32 * q + 2 * i + h;
      const int64_t at = (int64_t)n * K + k;
      if (codes) codes[at] = c;
      const float qv = (float)c - o;                 // exact
      if (w) w[at] = qv * s;                         // exact in fp32
      if (q16) q16[at] = f2h(qv);
    }
  }
}

__global__ void k_debug_uniform(SegDev sg, const int32_t* col_map, int G, int K, int32_t* codes, float* w,
                                uint16_t* q16) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)sg.tiles * G * 64) return;
  switch (sg.bits) {
    case 2: debug_slot<2>(sg, col_map, G, K, gid, codes, w, q16); break;
    case 3: debug_slot<3>(sg, col_map, G, K, gid, codes, w, q16); break;
    default: debug_slot<4>(sg, col_map, G, K, gid, codes, w, q16); break;
  }
}

}  // namespace qg
