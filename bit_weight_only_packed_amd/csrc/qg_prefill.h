// qg_prefill.h -- the prefill route's dequantisation: uniform b-bit codes of a
// column range -> fp16 weights [n - n0][K] (row-major, one row per output
// column), each weight (c - o) * s rounded once to fp16 (RNE).  The matrix
// product that follows is a plain fp16 GEMM with fp32 accumulation (hipBLASLt).
#pragma once
#include "qg_common.h"

namespace qg {

// one wave per (tile, quad) of tiles [tl0, tl0 + ntl) of a segment: each
// lane's quad (B 16-byte words, one coalesced 1 KiB wave load each, as the
// GEMVs load it) decoded group by group into 4 runs of 32 consecutive weights
// of its column, written to the wave's LDS tile [16 columns][512 k] (rows
// padded by 16 bytes against bank conflicts); the kernel then stores the tile
// row by row, 1 KiB of one output row per wave instruction
template <int B>
__device__ __forceinline__ void dq_quad(const SegDev& sg, const int32_t* col_map, int G, int G4, int tl, int qu,
                                        int lane, int n0, int n1, uint4 (*tile)[65]) {
  using P = Pair<B>;
  const int j = lane & 15, q = lane >> 4;
  const int n = col_map[16 * (sg.tile0 + tl) + j];
  if (n < n0 || n >= n1) return;  // padding (n < 0) or outside the range: its row is not stored
  const size_t tq = (size_t)tl * G4 + qu;
  const uint4* src = reinterpret_cast<const uint4*>(sg.codes) + tq * B * 64 + lane;
  uint32_t cw[4 * B];
#pragma unroll
  for (int p = 0; p < B; ++p) {
    const uint4 v = src[p * 64];
    cw[4 * p] = v.x; cw[4 * p + 1] = v.y; cw[4 * p + 2] = v.z; cw[4 * p + 3] = v.w;
  }
  const uint2 sw = *reinterpret_cast<const uint2*>(sg.scales + scale_index(tl, G4, 4 * qu, j, q, sg.sq));
  if constexpr (B == 4) {
    if (sg.mx) {  // MXFP4: element * 2^(e - 127), rounded once to fp16
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int g = 4 * qu + gi;
        if (g >= G) break;
        uint32_t r[16];
        decode_group_mx(cw, gi, r);
        const uint32_t s2 = gi < 2 ? sw.x : sw.y;
        const float s = e8m0_scale(((gi & 1) ? (s2 >> 16) : s2) & 0xFFu, 14);  // also undoes the 2^-14
        uint32_t h[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          h[i] = (uint32_t)f2h(h2f((uint16_t)r[i]) * s) | ((uint32_t)f2h(h2f((uint16_t)(r[i] >> 16)) * s) << 16);
#pragma unroll
        for (int v = 0; v < 4; ++v) tile[j][16 * gi + 4 * q + v] = make_uint4(h[4 * v], h[4 * v + 1], h[4 * v + 2], h[4 * v + 3]);
      }
      return;
    }
  }
  if constexpr (B == 6) {  // MXFP6: element * 2^(e - 127), rounded once to fp16
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int g = 4 * qu + gi;
      if (g >= G) break;
      uint32_t r[16];
      decode_group_mx6(cw, gi, r);
      const uint32_t s2 = gi < 2 ? sw.x : sw.y;
      const float s = e8m0_scale(((gi & 1) ? (s2 >> 16) : s2) & 0xFFu, 12);  // also undoes the 2^-12
      uint32_t h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        h[i] = (uint32_t)f2h(h2f((uint16_t)r[i]) * s) | ((uint32_t)f2h(h2f((uint16_t)(r[i] >> 16)) * s) << 16);
#pragma unroll
      for (int v = 0; v < 4; ++v) tile[j][16 * gi + 4 * q + v] = make_uint4(h[4 * v], h[4 * v + 1], h[4 * v + 2], h[4 * v + 3]);
    }
    return;
  } else {
  const float o = 0.5f * (float)((1 << B) - 1);
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    const int g = 4 * qu + gi;
    if (g >= G) break;
    uint32_t r[16];
    decode_group_classes<B>(cw, gi, r);
    const uint32_t s2 = gi < 2 ? sw.x : sw.y;
    const float s = h2f((uint16_t)((gi & 1) ? (s2 >> 16) : (s2 & 0xFFFFu)));
    uint32_t h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = P::cls(i);
      const float w0 = ((float)((r[i] >> p) & P::mask()) - o) * s;         // exact in fp32
      const float w1 = ((float)((r[i] >> (16 + p)) & P::mask()) - o) * s;  // exact in fp32
      h[i] = (uint32_t)f2h(w0) | ((uint32_t)f2h(w1) << 16);                 // k = 32 q + 2 i, + 1
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) tile[j][16 * gi + 4 * q + v] = make_uint4(h[4 * v], h[4 * v + 1], h[4 * v + 2], h[4 * v + 3]);
  }
  }
}

__global__ __launch_bounds__(64) void k_dequant_f16(SegDev sg, const int32_t* col_map, int G, int G4, int K, int tl0,
                                                    int ntl, int n0, int n1, uint16_t* out) {
  __shared__ uint4 tile[16][65];
  const int64_t tq = blockIdx.x;  // (tile - tl0) * G4 + quad
  if (tq >= (int64_t)ntl * G4) return;
  const int lane = threadIdx.x;
  const int qu = (int)(tq % G4), tl = tl0 + (int)(tq / G4);
  switch (sg.bits) {
    case 2: dq_quad<2>(sg, col_map, G, G4, tl, qu, lane, n0, n1, tile); break;
    case 3: dq_quad<3>(sg, col_map, G, G4, tl, qu, lane, n0, n1, tile); break;
    case 6: dq_quad<6>(sg, col_map, G, G4, tl, qu, lane, n0, n1, tile); break;
    default: dq_quad<4>(sg, col_map, G, G4, tl, qu, lane, n0, n1, tile); break;
  }
  __syncthreads();
  // the tile's rows: lane l stores weights 8 l .. 8 l + 7 of the quad's 512 k
  // (past K: the padding groups of the last quad, not stored)
  const int k0 = qu * 512 + 8 * lane;
  const int* cm = col_map + 16 * (sg.tile0 + tl);
  for (int r = 0; r < 16; ++r) {
    const int n = cm[r];
    if (n < n0 || n >= n1 || k0 >= K) continue;
    *reinterpret_cast<uint4*>(out + (size_t)(n - n0) * K + k0) = tile[r][lane];
  }
}

}  // namespace qg
