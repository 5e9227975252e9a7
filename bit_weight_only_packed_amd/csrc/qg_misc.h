// qg_misc.h -- kernels off the hot loop: the create-time re-layout of uniform
// codes, the checking kernels that expose the run kernels' decode (GEMV class
// decode and MFMA operand decode), the block-exponent rounding of the fused
// MLP's fp32 intermediate for the verify GEMM, and a plain streaming read (the
// measured read roofline the GEMV timings are set against).
#pragma once
#include "qg_common.h"

namespace qg {

// ---------------------------------------------------------------------------
// create-time re-layout: canonical stream -> device layout (one thread per
// tile, quad and lane)
// ---------------------------------------------------------------------------
// gs: the scale group size (128, 64 or 32; scales_in is [N][K / gs])
__global__ void k_repack_uniform(const uint32_t* __restrict__ canon, const int64_t* __restrict__ row_off,
                                 const uint16_t* __restrict__ scales_in, const int32_t* __restrict__ cols,
                                 int bits, int tiles, int G, int G4, int gs, uint32_t* __restrict__ dcodes,
                                 uint16_t* __restrict__ dscales) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)tiles * G4 * 64;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  const int64_t tq = gid >> 6;               // tile * G4 + quad
  const int qu = (int)(tq % G4);
  const int t = (int)(tq / G4);
  const int j = lane & 15, q = lane >> 4;
  const int n = cols[16 * t + j];
  uint32_t out[16];
  for (int u = 0; u < 16; ++u) out[u] = 0u;
  for (int gi = 0; gi < 4; ++gi) {
    const int g = 4 * qu + gi;
    if (n < 0 || g >= G) continue;
    const uint32_t* src = canon + row_off[n] + (int64_t)g * 4 * bits + q * bits;
    uint32_t in[4] = {0u, 0u, 0u, 0u};
    for (int u = 0; u < bits; ++u) in[u] = src[u];
    uint32_t c[32];
    for (int tt = 0; tt < 32; ++tt) {      // code tt = stream bits [bits*tt, bits*tt + bits)
      const int b0 = bits * tt;
      const uint64_t two = (uint64_t)in[b0 >> 5] | ((b0 >> 5) + 1 < 4 ? ((uint64_t)in[(b0 >> 5) + 1] << 32) : 0ull);
      c[tt] = (uint32_t)(two >> (b0 & 31)) & ((1u << bits) - 1u);
    }
    uint32_t* o = out + gi * bits;
    for (int i = 0; i < 16; ++i) {
      const uint32_t lo = c[2 * i], hi = c[2 * i + 1];
      if (bits == 3 && i == 15) {
        for (int u = 0; u < 3; ++u) o[u] |= (((lo >> u) & 1u) << 15) | (((hi >> u) & 1u) << 31);
        continue;
      }
      int wd, off;
      if (bits == 2) { wd = i / 8; off = 2 * (i % 8); }
      else if (bits == 4) { wd = i / 4; off = 4 * (i % 4); }
      else { wd = i / 5; off = 3 * (i % 5); }
      o[wd] |= (lo << off) | (hi << (16 + off));
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(dcodes);
  for (int p = 0; p < bits; ++p)
    dst[((size_t)tq * bits + p) * 64 + lane] = make_uint4(out[4 * p], out[4 * p + 1], out[4 * p + 2], out[4 * p + 3]);
  const int sq = gs < 128;
  if (dscales && (sq || q == 0)) {  // (MXFP4 scales are laid out by k_repack_mx_scales)
    const int gpr = G * (128 / gs);  // scales per row
    for (int gi = 0; gi < 4; ++gi) {
      const int g = 4 * qu + gi;
      const int sg = (g * 128 + 32 * q) / gs;  // the scale group of this lane's 32 weights
      dscales[scale_index(t, G4, g, j, q, sq)] = (n >= 0 && g < G) ? scales_in[(int64_t)n * gpr + sg] : (uint16_t)0;
    }
  }
}

// MXFP4 scales: E8M0 bytes [N][K/32] -> the per-quarter layout, each entry the
// block's own exponent byte | the largest of its 128-group's four << 8.  One
// thread per (tile, quad, lane); padding (columns or groups) gets 0.
__global__ void k_repack_mx_scales(const uint8_t* __restrict__ e8, const int32_t* __restrict__ cols, int tiles, int G,
                                   int G4, uint16_t* __restrict__ dscales) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)tiles * G4 * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t tq = gid >> 6;
  const int qu = (int)(tq % G4), t = (int)(tq / G4);
  const int j = lane & 15, q = lane >> 4;
  const int n = cols[16 * t + j];
  for (int gi = 0; gi < 4; ++gi) {
    const int g = 4 * qu + gi;
    uint16_t v = 0;
    if (n >= 0 && g < G) {
      const uint8_t* b = e8 + (int64_t)n * (4 * G) + 4 * g;
      const uint32_t mx = max(max(b[0], b[1]), max(b[2], b[3]));
      v = (uint16_t)(b[q] | (mx << 8));
    }
    dscales[scale_index(t, G4, g, j, q, 1)] = v;
  }
}

// MXFP6 codes: canonical 6-bit stream -> the two-plane quad layout of
// decode_group_mx6 (low nibbles in the 4-bit pair layout, top two bits in the
// 2-bit pair layout).  One thread per (tile, quad, lane); padding gets 0.
__global__ void k_repack_mx6(const uint32_t* __restrict__ canon, const int32_t* __restrict__ cols, int tiles, int G,
                             int G4, uint32_t* __restrict__ dcodes) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)tiles * G4 * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t tq = gid >> 6;
  const int qu = (int)(tq % G4), t = (int)(tq / G4);
  const int j = lane & 15, q = lane >> 4;
  const int n = cols[16 * t + j];
  uint32_t out[24];
  for (int u = 0; u < 24; ++u) out[u] = 0u;
  for (int gi = 0; gi < 4; ++gi) {
    const int g = 4 * qu + gi;
    if (n < 0 || g >= G) continue;
    // the lane's 32 codes: 192 stream bits, words 6q .. 6q + 5 of the group's 24
    const uint32_t* src = canon + ((int64_t)n * G + g) * 24 + 6 * q;
    uint32_t in[6];
    for (int u = 0; u < 6; ++u) in[u] = src[u];
    for (int i = 0; i < 16; ++i) {
      uint32_t c[2];
      for (int h = 0; h < 2; ++h) {
        const int b0 = 6 * (2 * i + h);
        const uint64_t two = (uint64_t)in[b0 >> 5] | ((b0 >> 5) + 1 < 6 ? ((uint64_t)in[(b0 >> 5) + 1] << 32) : 0ull);
        c[h] = (uint32_t)(two >> (b0 & 31)) & 63u;
      }
      const int o4 = 4 * (i & 3), o2 = 2 * (i & 7);
      out[4 * gi + (i >> 2)] |= ((c[0] & 15u) << o4) | ((c[1] & 15u) << (16 + o4));
      out[16 + 2 * gi + (i >> 3)] |= ((c[0] >> 4) << o2) | ((c[1] >> 4) << (16 + o2));
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(dcodes);
  for (int p = 0; p < 6; ++p)
    dst[((size_t)tq * 6 + p) * 64 + lane] = make_uint4(out[4 * p], out[4 * p + 1], out[4 * p + 2], out[4 * p + 3]);
}

// ---------------------------------------------------------------------------
// checking kernels: one thread per (tile, group, lane); the lane's quad is
// loaded as the run kernels hold it and group g of it is decoded by the run
// kernels' own functions, then written back per weight in [N][K]
// ---------------------------------------------------------------------------
template <int B>
__device__ __forceinline__ void debug_quad(const SegDev& sg, int G4, int tl, int g, int lane, uint32_t (&cw)[4 * B]) {
#pragma unroll
  for (int gi = 0; gi < 4; ++gi)
#pragma unroll
    for (int u = 0; u < B; ++u) cw[gi * B + u] = sg.codes[code_word_index(tl, G4, 4 * (g >> 2) + gi, lane, u, B)];
}

// MODE 0: the M = 1 GEMVs' class decode (codes, exact q = c - o and w = q * s).
// MODE 1: the verify GEMM's MFMA operand decode (codes read back out of the
// offset-1 operand registers, the operand's fp16 bits, and w rebuilt from the
// operand value and the kernel's offset constant: (op + ko) * 2^23 * s).  With
// scale groups of 64 or 32 the operand carries the scale: its fp16 bits are
// 2 (c - o) s rounded once, and w is half its value.
template <int B, int MODE>
__device__ __forceinline__ void debug_slot(const SegDev& sg, const int32_t* col_map, int G, int G4, int K,
                                           int64_t gid, int32_t* codes, float* w, uint16_t* q16) {
  using P = Pair<B>;
  const int lane = (int)(gid & 63);
  const int64_t tg = gid >> 6;
  const int g = (int)(tg % G), tl = (int)(tg / G);
  const int j = lane & 15, q = lane >> 4;
  const int n = col_map[16 * (sg.tile0 + tl) + j];
  if (n < 0) return;
  uint32_t cw[4 * B];
  debug_quad<B>(sg, G4, tl, g, lane, cw);
  uint32_t r[16], rs[16];
  const uint16_t s16 = sg.scales[scale_index(tl, G4, g, j, q, sg.sq)];
  if constexpr (B == 4) {
    if (sg.mx) {
      // MXFP4.  MODE 0: the GEMVs' element decode -- codes (the nibbles), w
      // exact in fp32 (element * 2^(e - 127)) and q16 the element's fp16 value.
      // MODE 1: the verify GEMM's operand -- its fp16 bits (element * 2^-14 *
      // 2^-(e_max - e), rounded once) and w = operand * 2^(e_max - 113).
      decode_group_mx(cw, g & 3, r);
      const uint32_t eq = s16 & 0xFFu, emax = (uint32_t)s16 >> 8, de = emax - eq;
      const uint32_t f = de <= 14u ? (15u - de) << 10 : (de <= 24u ? 1u << (24u - de) : 0u);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t op2 = MODE == 1 ? pk_mul_f16(r[i], f | (f << 16)) : r[i];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = g * 128 + 32 * q + 2 * i + h;
          const int64_t at = (int64_t)n * K + k;
          const uint32_t nib = (cw[(g & 3) * 4 + (i >> 2)] >> (16 * h + 4 * (i & 3))) & 15u;
          if (codes) codes[at] = (int32_t)nib;
          const uint16_t el = (uint16_t)(op2 >> (16 * h));
          if constexpr (MODE == 0) {
            if (q16) q16[at] = f2h(h2f(el) * 16384.0f);            // the element (exact)
            if (w) w[at] = h2f(el) * 16384.0f * e8m0_scale(eq, 0);  // exact in fp32
          } else {
            if (q16) q16[at] = el;
            if (w) w[at] = h2f(el) * e8m0_scale(emax, 14);
          }
        }
      }
      return;
    }
  }
  if constexpr (B == 6) {
    // MXFP6.  MODE 0: the GEMVs' element decode -- codes (read back out of the
    // decoded fp16: sign bit 15, magnitude bits 12..8), w exact in fp32
    // (element * 2^(e - 127)) and q16 the element's fp16 value.  MODE 1: the
    // verify GEMM's operand -- its fp16 bits (element * 2^(3 - (e_max - e)),
    // rounded once) and w = operand * 2^(e_max - 130).
    decode_group_mx6(cw, g & 3, r);
    const uint32_t eq = s16 & 0xFFu, emax = (uint32_t)s16 >> 8;
    const uint32_t f = mx6_operand_factor(emax - eq);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t op2 = MODE == 1 ? pk_mul_f16(r[i], f | (f << 16)) : r[i];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = g * 128 + 32 * q + 2 * i + h;
        const int64_t at = (int64_t)n * K + k;
        const uint32_t d = r[i] >> (16 * h);
        if (codes) codes[at] = (int32_t)((((d >> 15) & 1u) << 5) | ((d >> 8) & 31u));
        const uint16_t el = (uint16_t)(op2 >> (16 * h));
        if constexpr (MODE == 0) {
          if (q16) q16[at] = f2h(h2f(el) * 4096.0f);            // the element (exact)
          if (w) w[at] = h2f(el) * 4096.0f * e8m0_scale(eq, 0);  // exact in fp32
        } else {
          if (q16) q16[at] = el;
          if (w) w[at] = h2f(el) * e8m0_scale(emax, -3);
        }
      }
    }
    return;
  } else {
  if constexpr (MODE == 0) decode_group_classes<B>(cw, g & 3, r);
  else decode_group_off1<B>(cw, g & 3, r);
  if (MODE == 1 && sg.sq) decode_group_scaled<B>(cw, g & 3, (uint32_t)s16 | ((uint32_t)s16 << 16), rs);
  const float s = h2f(s16);
  const float o = 0.5f * (float)((1 << B) - 1);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int p = MODE == 0 ? P::cls(i) : 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = (int)((r[i] >> (16 * h + p)) & P::mask());
      const int64_t k = (int64_t)g * 128 + 32 * q + 2 * i + h;
      const int64_t at = (int64_t)n * K + k;
      if (codes) codes[at] = c;
      if constexpr (MODE == 0) {
        const float qv = (float)c - o;                 // exact
        if (w) w[at] = qv * s;                         // exact in fp32
        if (q16) q16[at] = f2h(qv);
      } else if (sg.sq) {
        const uint16_t op = (uint16_t)(rs[i] >> (16 * h));  // fp16 bits of 2 (c - o) s, rounded once
        if (q16) q16[at] = op;
        if (w) w[at] = 0.5f * h2f(op);
      } else {
        const uint16_t op = (uint16_t)(r[i] >> (16 * h));  // the operand element: fp16 bits of c * 2^-23
        if (q16) q16[at] = op;
        if (w) w[at] = (h2f(op) + off1_ko<B>()) * 8388608.0f * s;  // exact: (c - o) * s
      }
    }
  }
  }
}

template <int MODE>
__global__ void k_debug_uniform(SegDev sg, const int32_t* col_map, int G, int G4, int K, int32_t* codes, float* w,
                                uint16_t* q16) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)sg.tiles * G * 64) return;
  switch (sg.bits) {
    case 2: debug_slot<2, MODE>(sg, col_map, G, G4, K, gid, codes, w, q16); break;
    case 3: debug_slot<3, MODE>(sg, col_map, G, G4, K, gid, codes, w, q16); break;
    case 6: debug_slot<6, MODE>(sg, col_map, G, G4, K, gid, codes, w, q16); break;
    default: debug_slot<4, MODE>(sg, col_map, G, G4, K, gid, codes, w, q16); break;
  }
}

// ---------------------------------------------------------------------------
// The fused MLP's fp32 intermediate h [M][K] as the verify GEMM's input: per
// (row m, 128-group g) a power-of-two exponent e from the group's largest
// magnitude (so the largest scaled value lies in [2^14, 2^15)), x16 = fp16(h *
// 2^e) rounded once (RNE), and xf[m][g] = 2^-e for the GEMM to undo it.  One
// wave per (row, group), two values per lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_h_to_f16(const float* __restrict__ h, uint16_t* __restrict__ x16,
                                                  float* __restrict__ xf, int M, int K) {
  const int G = K / 128;
  const int wv = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  if (wv >= M * G) return;  // whole waves leave together (blockDim is a multiple of 64)
  const int lane = threadIdx.x & 63;
  const int m = wv / G, g = wv - m * G;
  const size_t base = (size_t)m * K + (size_t)g * 128 + 2 * lane;
  const float2 v = *reinterpret_cast<const float2*>(h + base);
  uint32_t mx = max(__float_as_uint(v.x) & 0x7FFFFFFFu, __float_as_uint(v.y) & 0x7FFFFFFFu);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, d));
  const int e = min(60, max(-20, 141 - (int)(mx >> 23)));
  const uint32_t t = (uint32_t)f2h(__builtin_ldexpf(v.x, e)) | ((uint32_t)f2h(__builtin_ldexpf(v.y, e)) << 16);
  *reinterpret_cast<uint32_t*>(x16 + base) = t;
  if (lane == 0) xf[(size_t)m * G + g] = __uint_as_float((uint32_t)(127 - e) << 23);
}

// ---------------------------------------------------------------------------
// Plain streaming read of [buf, buf + n16 * 16): each thread keeps four 16-byte
// loads in flight per step and the grid strides over the buffer; the loaded
// words are folded into a value whose (never taken) store keeps the loads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void k_stream_read(const uint4* __restrict__ buf, int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u && sink) sink[0] = acc;
}

// zero [p, p + n16 * 16): a plain kernel (not a memset node), so it can sit in
// a captured graph
__global__ __launch_bounds__(256) void k_fill_zero(uint4* __restrict__ p, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace qg
