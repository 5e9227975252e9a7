// qg_decode.h -- device layout of packed codes and the in-register decode used by
// every kernel of the library (run kernels and checking kernels alike).
//
// Device layout (written once by the repack kernel at create time).
//   Columns are grouped in tiles of 16.  Lane l of a wave owns column
//   16*t + (l & 15) and quarter q = l >> 4 of each 128-group: the 32 codes
//   c_0..c_31 at k = 128*g + 32*q + j, stored in B words (see below).  Groups
//   are bundled by four ("quads", the group count padded to a multiple of 4
//   with zero codes and zero scales): a lane's quad is 4*B words = B uint4
//   "parts", group i of the quad being words [i*B, i*B + B).  For tile t and
//   quad u the 64 lanes' part p is one contiguous 1 KiB block at uint4 index
//   ((t*G4 + u)*B + p)*64 + l, so every wave-wide load is a full-width
//   (16 B per lane), fully coalesced 1 KiB read.
//   Within a group the codes are stored as 16 pairs (c_{2i}, c_{2i+1}); pair i
//   keeps c_{2i} in the low 16-bit half and c_{2i+1} at the same bit offset in
//   the high half:
//     B = 2: word i/8, offset 2*(i%8)         (8 pairs per word)
//     B = 4: word i/4, offset 4*(i%4)         (4 pairs per word)
//     B = 3: i < 15: word i/5, offset 3*(i%5) (5 pairs per word, bit 15/31 spare)
//            i = 15: bit u of c30 is bit 15 of word u, bit u of c31 bit 31 of word u.
//   Scales: fp16 [tile][G4][16][4]: per quad, column, then group within the quad.
//
// Decode.  An fp16 whose bits are an integer v < 2048 has the value v * 2^-24
// exactly (exponent field 0: subnormal m * 2^-24; exponent field 1:
// (1024 + m) * 2^-24).  So masking a B-bit code field that sits at bit offset p
// (p + B <= 11) in both halves of a word yields, with one AND, the fp16 pair
// (c_lo * 2^(p-24), c_hi * 2^(p-24)) -- exact, no conversion instruction.
// gfx950's v_dot2_f32_f16 and v_mfma_f32_16x16x32_f16 consume such subnormal
// fp16 operands exactly.  Codes at offsets beyond the exact range are first
// shifted down.  The M = 1 GEMVs stage each x multiplied by 2^(e - class) of
// the code position it meets, e a power-of-two block exponent of its 32-element
// quarter (qg_stage.h), so one dot2 chain serves every class; the MFMA path
// shifts every pair to offset 1 so a whole operand shares one scale.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

template <int B> struct Pair {
  // word holding pair i, its bit offset, and (GEMV) the shift applied before masking
  static constexpr int word(int i) { return B == 2 ? i / 8 : B == 4 ? i / 4 : (i < 15 ? i / 5 : 0); }
  static constexpr int off(int i) { return B == 2 ? 2 * (i % 8) : B == 4 ? 4 * (i % 4) : 3 * (i % 5); }
  // (3-bit: word u is shifted by 9 - u, which also lines its spare bit 15 up at
  // bit 6 + u, so pair 15 is assembled from the shifted words with no extra shift)
  static constexpr int gshift(int i) {
    return B == 2 ? (i % 8 < 5 ? 0 : 10) : B == 4 ? (i % 4 < 2 ? 0 : 8) : (i % 5 < 3 ? 0 : 9 - i / 5);
  }
  // GEMV class of pair i: bit offset after the shift (3-bit pair 15 is built at 6)
  static constexpr int cls(int i) { return (B == 3 && i == 15) ? 6 : off(i) - gshift(i); }
  static constexpr uint32_t mask() { return (1u << B) - 1u; }
  static constexpr uint32_t m2(int p) { return (mask() << p) * 0x10001u; }  // field at p in both halves
};

// ---- GEMV decode: pair registers at their class offsets (1 AND per pair, shifts shared per word)
template <int B>
__device__ __forceinline__ void decode_classes(const uint32_t (&w)[B], uint32_t (&r)[16]) {
  using P = Pair<B>;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (B == 3 && i == 15) continue;
    const uint32_t v = w[P::word(i)] >> P::gshift(i);
    r[i] = v & P::m2(P::cls(i));
  }
  if constexpr (B == 3) {
    // spare bits 15/31 of the three words -> (c30, c31) at offset 6
    r[15] = ((w[0] >> 9) & 0x00400040u) | ((w[1] >> 8) & 0x00800080u) | ((w[2] >> 7) & 0x01000100u);
  }
}

// fp16x2 bits of (2^-p, 2^-p), p = the class of pair i: x scaled by it meets the
// pair's code at offset p, so every product lands at the common scale 2^-24
template <int B> __device__ constexpr uint32_t class_scale_pair(int i) {
  const uint32_t h = (uint32_t)(15 - Pair<B>::cls(i)) << 10;
  return h | (h << 16);
}
// fp16x2 bits of (2^p, 2^p): undoes the class scaling of a staged x pair
template <int B> __device__ constexpr uint32_t class_unscale_pair(int i) {
  const uint32_t h = (uint32_t)(15 + Pair<B>::cls(i)) << 10;
  return h | (h << 16);
}

// ---- MFMA decode: every pair at offset 1 (value 2*c*2^-24 = c*2^-23)
template <int B>
__device__ __forceinline__ void decode_off1(const uint32_t (&w)[B], uint32_t (&r)[16]) {
  using P = Pair<B>;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (B == 3 && i == 15) continue;
    const int o = P::off(i);
    const uint32_t v = (o == 0) ? (w[P::word(i)] << 1) : (w[P::word(i)] >> (o - 1));
    r[i] = v & P::m2(1);
  }
  if constexpr (B == 3) {
    r[15] = ((w[0] >> 14) & 0x00020002u) | ((w[1] >> 13) & 0x00040004u) | ((w[2] >> 12) & 0x00080008u);
  }
}

// -o_b * 2^-23: the code offset at the MFMA scale (codes decoded at offset 1,
// value c * 2^-23); a group's MFMA chain starts from this times the group sum
// of x, so it yields 2^-23 * sum x * (c - o_b)
template <int B> __host__ __device__ constexpr float off1_ko() {
  return -0.5f * (float)((1 << B) - 1) * 1.1920928955078125e-07f;
}
// -o_b * 2^-24: the same at the GEMV scale (codes decoded at their class
// offsets, met by x staged at 2^-class: every product lands at 2^-24)
template <int B> __host__ __device__ constexpr float cls_ko() {
  return -0.5f * (float)((1 << B) - 1) * 5.9604644775390625e-08f;
}

// the lane's group gi of a quad decoded for the MFMA B operand (offset 1)
template <int B>
__device__ __forceinline__ void decode_group_off1(const uint32_t (&w)[4 * B], int gi, uint32_t (&r)[16]);

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }

// packed fp16 multiply (used once per activation element when x is staged)
__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, as_h2(a) * as_h2(b));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

__device__ __forceinline__ h8_t as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 v = make_uint4(a, b, c, d);
  return __builtin_bit_cast(h8_t, v);
}

__device__ __forceinline__ f4_t mfma16(h8_t a, h8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// A pointer the compiler may not prove wave-uniform, made so (it is uniform in
// fact): buffer resources built from it then live in scalar registers.
template <typename T> __device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Buffer resource over [base, base + bytes): raw loads outside the range return 0
// and touch no memory, so a load can be issued unconditionally.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// A lane's quad (4 groups, 4*B words) through a buffer resource whose byte 0 is
// part 0 of the wave's first quad; `qu` is the quad index relative to it.  The
// whole byte offset goes into the per-lane offset, which the range check of a
// raw buffer access covers, so a quad past the resource's range reads nothing.
template <int B>
__device__ __forceinline__ void buffer_quad(__amdgpu_buffer_rsrc_t r, uint32_t lane, int qu, uint32_t (&w)[4 * B]) {
#pragma unroll
  for (int p = 0; p < B; ++p) {
    const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u + (uint32_t)(qu * B + p) * 1024u, 0, 0);
    w[4 * p + 0] = v.x; w[4 * p + 1] = v.y; w[4 * p + 2] = v.z; w[4 * p + 3] = v.w;
  }
}

// Group i of a quad as a B-word array
template <int B>
__device__ __forceinline__ void quad_group(const uint32_t (&w)[4 * B], int i, uint32_t (&g)[B]) {
#pragma unroll
  for (int u = 0; u < B; ++u) g[u] = w[i * B + u];
}

template <int B>
__device__ __forceinline__ void decode_group_off1(const uint32_t (&w)[4 * B], int gi, uint32_t (&r)[16]) {
  uint32_t g[B];
  quad_group<B>(w, gi, g);
  decode_off1<B>(g, r);
}

// MFMA operand with the scale inside (scale groups of 64 or 32, where one MFMA
// spans lanes of four different scales): each pair at offset 1 under the
// exponent of 1024 is the exact fp16 pair 1024 + 2c; one exact packed
// subtraction of 1024 + 2 o leaves 2 (c - o) (|.| <= 15), and one packed
// multiplication by the lane's scale pair s2 = (s, s) rounds 2 (c - o) s once
// to fp16 (RNE).  The MFMA chain then yields 2 y, halved on output.
template <int B>
__device__ __forceinline__ void decode_group_scaled(const uint32_t (&w)[4 * B], int gi, uint32_t s2, uint32_t (&r)[16]) {
  decode_group_off1<B>(w, gi, r);
  constexpr uint32_t kExp = 0x64006400u;  // fp16 1024 in both halves
  constexpr uint32_t kOff = (uint32_t)(0x8000u | 0x6400u | ((1u << B) - 1u));  // fp16 -(1024 + 2 o)
  const h2_t off = as_h2(kOff | (kOff << 16));
  const h2_t sc = as_h2(s2);
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = __builtin_bit_cast(uint32_t, (as_h2(r[i] | kExp) + off) * sc);
}

// MXFP4 elements in the 4-bit layout: each E2M1 nibble (sign, two exponent
// bits, one mantissa bit) of a pair becomes the fp16 with the sign at bit 15
// and the three magnitude bits at bits 11..9 -- exponent field e, mantissa m/2,
// and e = 0 the subnormal m 2^-15 -- which is exactly the element times 2^-14
__device__ __forceinline__ void decode_group_mx(const uint32_t (&w)[16], int gi, uint32_t (&r)[16]) {
  uint32_t g[4];
  quad_group<4>(w, gi, g);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t v = g[i >> 2];
    const int o = 4 * (i & 3);  // the pair's nibbles sit at bits o and 16 + o
    const uint32_t mag = (o <= 9 ? v << (9 - o) : v >> (o - 9)) & 0x0E000E00u;
    r[i] = mag | ((v << (12 - o)) & 0x80008000u);
  }
}

// MXFP6 elements (E3M2: sign bit 5, exponent bits 4..2, mantissa bits 1..0) in
// two planes of a 6-word lane quad (B = 6 in the load layout): words 0..15 the
// low nibbles (exponent bits 1..0 and the mantissa) in the 4-bit pair layout,
// words 16..23 the top two bits (exponent bit 2, sign) in the 2-bit pair
// layout, group gi at words 4 gi .. 4 gi + 3 and 16 + 2 gi .. 16 + 2 gi + 1.
// Each element of a pair becomes the fp16 with the sign at bit 15 and the five
// magnitude bits at bits 12..8 -- exponent field e, mantissa m/4, and e = 0
// the subnormal m 2^-16 -- which is exactly the element times 2^-12.
__device__ __forceinline__ void decode_group_mx6(const uint32_t (&w)[24], int gi, uint32_t (&r)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t lo = w[4 * gi + (i >> 2)], hi = w[16 + 2 * gi + (i >> 3)];
    const int o4 = 4 * (i & 3), o2 = 2 * (i & 7);  // bit offsets of the pair's fields
    const uint32_t nib = (o4 <= 8 ? lo << (8 - o4) : lo >> (o4 - 8)) & 0x0F000F00u;
    const uint32_t e2 = (o2 <= 12 ? hi << (12 - o2) : hi >> (o2 - 12)) & 0x10001000u;
    const uint32_t sg = (hi << (14 - o2)) & 0x80008000u;
    r[i] = nib | e2 | sg;
  }
}

// fp16 bits of 2^(15 - de): an MXFP6 element decoded at 2^-12 times it is the
// element times 2^(3 - de), exact for de <= 23 (its lowest bit stays at or
// above 2^-24), rounded once (RNE) beyond; 0 past fp16's range
__device__ __forceinline__ uint32_t mx6_operand_factor(uint32_t de) {
  return de <= 29u ? (30u - de) << 10 : (de <= 39u ? 1u << (39u - de) : 0u);
}

// fp32 2^(e - 127) of an E8M0 byte (e = 0: 2^-127; 255: NaN), times 2^k
// (|k| small; the result clamps to the fp32 range ends)
__device__ __forceinline__ float e8m0_scale(uint32_t e, int k) {
  if (e == 255u) return __builtin_nanf("");
  const int f = (int)e + k;  // biased fp32 exponent of 2^(e - 127 + k)
  if (f >= 255) return __builtin_bit_cast(float, 0x7F000000u);                // 2^127
  if (f >= 1) return __builtin_bit_cast(float, (uint32_t)f << 23);
  return f >= -22 ? __builtin_bit_cast(float, 0x00400000u >> (-f)) : 0.0f;   // subnormal
}

template <int B>
__device__ __forceinline__ void decode_group_classes(const uint32_t (&w)[4 * B], int gi, uint32_t (&r)[16]) {
  uint32_t g[B];
  quad_group<B>(w, gi, g);
  decode_classes<B>(g, r);
}

// Word u of group g of lane `lane` in tile t (plain pointer form; G4 quads per tile)
__device__ __forceinline__ size_t code_word_index(int t, int G4, int g, int lane, int u, int B) {
  const int qu = g >> 2, wi = (g & 3) * B + u;  // word within the lane's quad
  return ((((size_t)t * G4 + qu) * B + (wi >> 2)) * 64 + lane) * 4 + (wi & 3);
}

}  // namespace qg
