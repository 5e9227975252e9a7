// qg_prefill.h -- the prefill route's dequantisation: uniform b-bit codes of a
// column range -> fp16 weights [n - n0][K] (row-major, one row per output
// column), each weight (c - o) * s rounded once to fp16 (RNE).  The matrix
// product that follows is a plain fp16 GEMM with fp32 accumulation (hipBLASLt).
#pragma once
#include "qg_common.h"

namespace qg {

// groups of a quad that one pass stages in LDS: the wave's tile holds 16
// columns x kDqGroups groups of 128 k (8.4 KB at 2), so that more waves fit
// on a CU than with the whole quad (16.6 KB) staged at once
constexpr int kDqGroups = 2;

// one wave per (tile, quad) of tiles [tl0, tl0 + ntl) of a segment: each
// lane's quad (B 16-byte words, one coalesced 1 KiB wave load each, as the
// GEMVs load it) decoded group by group into runs of 32 consecutive weights
// of its column; kDqGroups groups at a time go to the wave's LDS tile
// [16 columns][128 kDqGroups k] (rows padded by 16 bytes against bank
// conflicts), from which the wave stores them row by row (512 kDqGroups
// contiguous bytes per row, 1 KiB per wave instruction)
template <int B>
__device__ __forceinline__ void dq_group(const uint32_t (&cw)[4 * B], uint2 sw, bool mx, int gi, int j, int q,
                                         uint4 (*tile)[16 * kDqGroups + 1], int gl) {
  using P = Pair<B>;
  const uint32_t s2 = gi < 2 ? sw.x : sw.y;
  uint32_t h[16];
  if constexpr (B == 4 || B == 6) {
    if (B == 6 || mx) {  // MXFP4 / MXFP6: element * 2^(e - 127), rounded once to fp16
      uint32_t r[16];
      if constexpr (B == 4) decode_group_mx(cw, gi, r);
      else decode_group_mx6(cw, gi, r);
      // also undoes the decode's 2^-14 (E2M1) or 2^-12 (E3M2)
      const float s = e8m0_scale(((gi & 1) ? (s2 >> 16) : s2) & 0xFFu, B == 4 ? 14 : 12);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        h[i] = (uint32_t)f2h(h2f((uint16_t)r[i]) * s) | ((uint32_t)f2h(h2f((uint16_t)(r[i] >> 16)) * s) << 16);
#pragma unroll
      for (int v = 0; v < 4; ++v) tile[j][16 * gl + 4 * q + v] = make_uint4(h[4 * v], h[4 * v + 1], h[4 * v + 2], h[4 * v + 3]);
      return;
    }
  }
  if constexpr (B != 6) {
    const float o = 0.5f * (float)((1 << B) - 1);
    uint32_t r[16];
    decode_group_classes<B>(cw, gi, r);
    const float s = h2f((uint16_t)((gi & 1) ? (s2 >> 16) : (s2 & 0xFFFFu)));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = P::cls(i);
      const float w0 = ((float)((r[i] >> p) & P::mask()) - o) * s;         // exact in fp32
      const float w1 = ((float)((r[i] >> (16 + p)) & P::mask()) - o) * s;  // exact in fp32
      h[i] = (uint32_t)f2h(w0) | ((uint32_t)f2h(w1) << 16);                 // k = 32 q + 2 i, + 1
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) tile[j][16 * gl + 4 * q + v] = make_uint4(h[4 * v], h[4 * v + 1], h[4 * v + 2], h[4 * v + 3]);
  }
}

template <int B>
__device__ __forceinline__ void dq_quad(const SegDev& sg, const int32_t* col_map, int G, int G4, int K, int tl, int qu,
                                        int lane, int n0, int n1, uint16_t* out, uint4 (*tile)[16 * kDqGroups + 1]) {
  constexpr int RL = 16 * kDqGroups;  // lanes per stored row segment (16 bytes each)
  constexpr int RI = 64 / RL;               // rows per wave store instruction
  const int j = lane & 15, q = lane >> 4;
  const int* cm = col_map + 16 * (sg.tile0 + tl);
  const int n = cm[j];
  const bool mine = n >= n0 && n < n1;  // padding (n < 0) or outside the range: nothing decoded or stored
  const size_t tq = (size_t)tl * G4 + qu;
  const uint4* src = reinterpret_cast<const uint4*>(sg.codes) + tq * B * 64 + lane;
  uint32_t cw[4 * B] = {};
  uint2 sw = make_uint2(0u, 0u);
  if (mine) {
#pragma unroll
    for (int p = 0; p < B; ++p) {
      const uint4 v = src[p * 64];
      cw[4 * p] = v.x; cw[4 * p + 1] = v.y; cw[4 * p + 2] = v.z; cw[4 * p + 3] = v.w;
    }
    sw = *reinterpret_cast<const uint2*>(sg.scales + scale_index(tl, G4, 4 * qu, j, q, sg.sq));
  }
  const int rr = lane / RL, c = lane % RL;
#pragma unroll
  for (int g0 = 0; g0 < 4; g0 += kDqGroups) {
    if (4 * qu + g0 >= G) break;  // padding groups of the last quad (wave-uniform)
    if (mine) {
#pragma unroll
      for (int gl = 0; gl < kDqGroups; ++gl)
        if (4 * qu + g0 + gl < G) dq_group<B>(cw, sw, sg.mx != 0, g0 + gl, j, q, tile, gl);
    }
    __syncthreads();
    // lane (rr, c) stores weights 8 c .. 8 c + 7 of the pass's 128 kDqGroups k
    // of tile rows rr, rr + RI, ... (past K: the padding groups, not stored)
    const int k0 = qu * 512 + g0 * 128 + 8 * c;
#pragma unroll
    for (int r0 = 0; r0 < 16; r0 += RI) {
      const int r = r0 + rr;
      const int nr = cm[r];
      if (nr >= n0 && nr < n1 && k0 < K) *reinterpret_cast<uint4*>(out + (size_t)(nr - n0) * K + k0) = tile[r][c];
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(64) void k_dequant_f16(SegDev sg, const int32_t* col_map, int G, int G4, int K, int tl0,
                                                    int ntl, int n0, int n1, uint16_t* out) {
  __shared__ uint4 tile[16][16 * kDqGroups + 1];
  const int64_t tq = blockIdx.x;  // (tile - tl0) * G4 + quad
  if (tq >= (int64_t)ntl * G4) return;
  const int lane = threadIdx.x;
  const int qu = (int)(tq % G4), tl = tl0 + (int)(tq / G4);
  switch (sg.bits) {
    case 2: dq_quad<2>(sg, col_map, G, G4, K, tl, qu, lane, n0, n1, out, tile); break;
    case 3: dq_quad<3>(sg, col_map, G, G4, K, tl, qu, lane, n0, n1, out, tile); break;
    case 6: dq_quad<6>(sg, col_map, G, G4, K, tl, qu, lane, n0, n1, out, tile); break;
    default: dq_quad<4>(sg, col_map, G, G4, K, tl, qu, lane, n0, n1, out, tile); break;
  }
}

}  // namespace qg
