// qg_stage.h -- activation staging of the M = 1 GEMVs (per-group and per-tile-run).
//
// A GEMV lane meets each code pair of class p (the pair's bit offset after its
// decode shift, qg_decode.h) with an x pair staged at 2^(e - p): the pair's
// exact subnormal code value c * 2^(p - 24) times it is c * x * 2^(e - 24),
// whatever the class, so one dot2 chain covers the lane's 32 weights.
//
// Each wave stages the activations of its own quads (512 k each) into an LDS
// region of its own, so no wave waits for another before it computes.  e is a
// power-of-two block exponent over those activations, chosen from their
// largest magnitude so that every staged value stays below 2^15 (no fp16
// overflow) while the largest is at least 2^6 after the class factor.  Small
// activations are thereby scaled up, which is exact: the staged values keep
// every bit whatever the magnitude of x, down to fp16 subnormal inputs.  (A
// fixed 2^-p factor would push small activations into fp16's subnormal range
// and drop their low bits.)  Only values more than 2^20 below the block's
// largest lose bits (the class factor then takes them under fp16's normal
// range), and only when that largest value is at least 2^7; their error is
// below 2^-31 of the largest value each.  The wave undoes e once, on its
// partial sums.
//
// Beside the staged words goes, per 32-element quarter, the sum of the staged
// values scaled back per class (2^e times the sum of the values the chain
// uses, for the code offset term).  fp32 activations (the fused MLP's
// intermediate) are rounded to fp16 (RNE) once, after the exponent is applied,
// so they keep 11 significant bits at any magnitude.
#pragma once
#include "qg_common.h"

namespace qg {

// 16-byte loads per 8 activations: fp16 (XF false) or fp32 (XF true)
template <bool XF> struct XIn {
  static constexpr int W = XF ? 2 : 1;
};

// magnitude bits of the largest of 8 activations (the order of a float's
// magnitude bits is the order of its magnitudes; NaN sorts above infinity)
template <bool XF>
__device__ __forceinline__ uint32_t maxbits8(const uint4 (&v)[XIn<XF>::W]) {
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < XIn<XF>::W; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (XF) {
        mx = max(mx, w[k] & 0x7FFFFFFFu);
      } else {
        const uint32_t a = w[k] & 0x7FFF7FFFu;
        mx = max(mx, max(a & 0xFFFFu, a >> 16));
      }
    }
  }
  return mx;
}

// wave-wide maximum (every lane of the wave takes part)
__device__ __forceinline__ uint32_t wave_max(uint32_t m) {
  m = max(m, (uint32_t)dpp_xor1_i((int)m));
  m = max(m, (uint32_t)dpp_xor2_i((int)m));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x124, 0xF, 0xF, false));  // row_ror 4
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x128, 0xF, 0xF, false));  // row_ror 8
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)m, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)m, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)m, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)m, 48);
  return max(max(a, b), max(c, d));
}

// Block exponent from the largest magnitude's bits: max < 2^(F - 14) (fp16,
// F = its biased exponent field) or 2^(F - 126) (fp32); e keeps max * 2^e below
// 2^15.  The fp16 bound e <= 15 keeps every class factor 2^(e - p) a normal
// fp16 (exponent field 15 - p + e in 5..30, p <= 8); the fp32 path applies the
// factor in fp32, where e is only clamped to stay far from the range ends.
template <bool XF> __device__ __forceinline__ int block_exp(uint32_t mx) {
  return XF ? min(60, max(-20, 141 - (int)(mx >> 23))) : min(15, 29 - (int)(mx >> 10));
}

// 2^k as fp32 (|k| < 127)
__device__ __forceinline__ float pow2f(int k) { return __builtin_bit_cast(float, (uint32_t)(127 + k) << 23); }

// select among the four per-position constants (pos = 0..3) without branches
__device__ __forceinline__ uint32_t sel4(int pos, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const bool b0 = (pos & 1) != 0, b1 = (pos & 2) != 0;
  const uint32_t lo = b0 ? b : a, hi = b0 ? d : c;
  return b1 ? hi : lo;
}

// The fp16x2 class factors 2^-p and their inverses 2^p of pairs 4 pos + k
// (pos = 0..3, k = 0..3) for codes of 2, 3 and 4 bits, as a table each lane
// reads its position's row of (two 16-byte loads, issued with the weight
// loads) instead of selecting among immediates.
struct StageTab {
  uint32_t v[3][2][4][4];  // [bits - 2][0: factor, 1: inverse][pos][k]
};
template <int B> constexpr void stage_tab_fill(StageTab& t) {
  for (int i = 0; i < 16; ++i) {
    const uint32_t p = (uint32_t)Pair<B>::cls(i);
    t.v[B - 2][0][i >> 2][i & 3] = ((15u - p) << 10) * 0x10001u;
    t.v[B - 2][1][i >> 2][i & 3] = ((15u + p) << 10) * 0x10001u;
  }
}
constexpr StageTab make_stage_tab() {
  StageTab t{};
  stage_tab_fill<2>(t);
  stage_tab_fill<3>(t);
  stage_tab_fill<4>(t);
  return t;
}
static __constant__ __align__(16) StageTab kStageTab = make_stage_tab();

// Per-thread constants of the staging: pos = the thread's 16-byte position
// within its quarter (4 consecutive lanes hold one quarter, pos = 0..3 in lane
// order), e = the workgroup's block exponent.
// a lane's row of the table (pos = its position in the quarter).  Issued
// before the wave's code loads, so waiting for it never waits for them.
template <int B>
__device__ __forceinline__ void stage_tab(int pos, uint4& fv, uint4& iv) {
  constexpr int bi = (B >= 2 && B <= 4) ? B - 2 : 0;  // (other widths never stage classes)
  fv = *reinterpret_cast<const uint4*>(&kStageTab.v[bi][0][pos][0]);
  iv = *reinterpret_cast<const uint4*>(&kStageTab.v[bi][1][pos][0]);
}

template <int B>
struct StageK {
  uint32_t f[4];    // fp16x2 class factors 2^(e - p) of the pairs 4 pos + k
  uint32_t inv[4];  // fp16x2 2^p of the same pairs
  int sh[4];        // e - p (the fp32 path)
  __device__ __forceinline__ StageK(int pos, int e, const uint4& fv, const uint4& iv) {
    using P = Pair<B>;
    const uint32_t de = (uint32_t)(e * 0x04000400);  // exponent field + e in both halves
    f[0] = fv.x + de; f[1] = fv.y + de; f[2] = fv.z + de; f[3] = fv.w + de;
    inv[0] = iv.x; inv[1] = iv.y; inv[2] = iv.z; inv[3] = iv.w;
#pragma unroll
    for (int k = 0; k < 4; ++k) sh[k] = e - (int)sel4(pos, P::cls(k), P::cls(4 + k), P::cls(8 + k), P::cls(12 + k));
  }
};

// Stage 8 activations (elements 8 pos .. 8 pos + 7 of a 32-element quarter):
// returns the staged fp16 words (pair 4 pos + k in word k) and sets qsum, the
// quarter's sum of staged values scaled back per class (the same in the
// quarter's four lanes).
template <int B, bool XF>
__device__ __forceinline__ uint4 stage8(const uint4 (&v)[XIn<XF>::W], const StageK<B>& K, float& qsum) {
  uint32_t t[4];
  if constexpr (XF) {
    const uint32_t w[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = __builtin_ldexpf(__builtin_bit_cast(float, w[2 * k]), K.sh[k]);
      const float b = __builtin_ldexpf(__builtin_bit_cast(float, w[2 * k + 1]), K.sh[k]);
      t[k] = (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
    }
  } else {
    t[0] = pk_mul_f16(v[0].x, K.f[0]);
    t[1] = pk_mul_f16(v[0].y, K.f[1]);
    t[2] = pk_mul_f16(v[0].z, K.f[2]);
    t[3] = pk_mul_f16(v[0].w, K.f[3]);
  }
  float s = dot2(t[0], K.inv[0], 0.0f);
  s = dot2(t[1], K.inv[1], s);
  s = dot2(t[2], K.inv[2], s);
  s = dot2(t[3], K.inv[3], s);
  s += dpp_xor1(s);
  s += dpp_xor2(s);
  qsum = s;
  return make_uint4(t[0], t[1], t[2], t[3]);
}

// Stage a wave's nu units of 8 activations (v[r] = unit lane + 64 r of the
// wave's region, quarter position lane & 3; nu <= NU, wave-uniform) into its LDS region: staged words at xl[unit], quarter sums at
// xq[unit / 4]; fv, iv: the lane's row of the class-factor table (stage_tab).
// Returns the block exponent e.  Every lane of the wave takes part.
template <int B, bool XF, int NU>
__device__ __forceinline__ int stage_wave(const uint4 (&v)[NU][XIn<XF>::W], uint4* xl, float* xq, int lane, int nu,
                                          const uint4& fv, const uint4& iv) {
  uint32_t mx = 0;
#pragma unroll
  for (int r = 0; r < NU; ++r) {
    if (r >= nu) break;
    mx = max(mx, maxbits8<XF>(v[r]));
  }
  const int e = block_exp<XF>(wave_max(mx));
  const StageK<B> K(lane & 3, e, fv, iv);
#pragma unroll
  for (int r = 0; r < NU; ++r) {
    if (r >= nu) break;
    float qs;
    const uint4 t = stage8<B, XF>(v[r], K, qs);
    xl[lane + 64 * r] = t;
    if ((lane & 3) == 0) xq[(lane + 64 * r) >> 2] = qs;
  }
  // the wave reads what its other lanes wrote: LDS keeps a wave's accesses in
  // order; this keeps the compiler from moving the reads above the writes
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  return e;
}

// MXFP4 staging: the wave's activations times 2^e (the block exponent) into
// its LDS region, no class factors (the decoded elements are fp16 values of
// their own) and no quarter sums (E2M1 has no code offset).  Returns e.
template <int NU>
__device__ __forceinline__ int stage_wave_plain(const uint4 (&v)[NU][1], uint4* xl, int lane, int nu) {
  uint32_t mx = 0;
#pragma unroll
  for (int r = 0; r < NU; ++r) {
    if (r >= nu) break;
    mx = max(mx, maxbits8<false>(v[r]));
  }
  const int e = block_exp<false>(wave_max(mx));
  const uint32_t f = (uint32_t)(15 + e) * 0x04000400u;  // fp16x2 (2^e, 2^e), e in -2..15
#pragma unroll
  for (int r = 0; r < NU; ++r) {
    if (r >= nu) break;
    xl[lane + 64 * r] = make_uint4(pk_mul_f16(v[r][0].x, f), pk_mul_f16(v[r][0].y, f), pk_mul_f16(v[r][0].z, f),
                                   pk_mul_f16(v[r][0].w, f));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  return e;
}

}  // namespace qg
