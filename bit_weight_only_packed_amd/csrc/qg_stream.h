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
// Activations.  Each workgroup stages x once in LDS, every element already
// multiplied by 2^-class of the code position it meets (class_scale_pair), so a
// pair decoded by one AND at its class offset times its staged x pair is
// c * x * 2^-24 whatever the class: one dot2 chain per group, no per-class
// accumulators.  Beside it, the sum of each 32-element quarter of x: the code
// offset enters as -o * 2^-24 * sum, one fma per group.  The 16 lanes of a
// quarter read the same LDS addresses (broadcast).  The x loads go out first
// and each wave's first code loads right behind them, so staging x overlaps
// the first code fetches.
//
// The nch partials of one tile meet in a per-column 64-bit word: each wave
// adds (round(v * 2^28) << 6) + 1 (v clamped to +-2^23) with one integer
// atomic.  Integer addition is exact and commutative, so the total is the same
// whatever the order of arrival (bit-identical results), and the low 6 bits
// count the arrivals: the wave that brings the count to nch converts the sum
// to fp16, stores it and re-arms the word to 0 for the next launch.  With
// nch = 1 the sum is stored directly.  For the gate/up pair every wave adds its
// up partial, waits for that atomic to return, and only then adds its gate
// partial: the wave that completes the gate word therefore finds the up word
// complete too.
#pragma once
#include "qg_kernels.h"

namespace qg {

constexpr int SK_UPW = 8;    // at most this many quads per wave
constexpr int SK_PD = 3;     // units whose loads are in flight while one is computed

struct SkArgs {
  WSet w[2];                   // w[1]: up matrix of the fused gate/up pass
  const uint16_t* x;           // [K] fp16
  uint16_t* y;                 // [N] fp16 (fused pass: h = SiLU(g) * u)
  unsigned long long* acc;     // [2][16 * total_tiles] column words, zero between launches
  int K, N, G, G4, total_tiles;
  int nch;                     // waves per tile
  int64_t U;                   // total_tiles * G4
  int wg_prefix[MAX_SEG + 1];  // several widths: workgroups before each width segment
};

// LDS: a copy of x scaled for the workgroup's width (4 * G4 * 64 uint32 =
// 4*G4 groups of 128 fp16), then the quarter sums (4 * G4 * 4 floats)
__host__ __device__ constexpr size_t sk_lds_bytes(int G4) { return (size_t)G4 * 1024 + (size_t)G4 * 64; }

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
};

// unit u (segment-local: tile u / G4, quad u % G4) of the segment's matrices
template <int B, int ND>
__device__ __forceinline__ void sk_load(const SkPtrs<ND>& p, SkUnit<B, ND>& c, int u, bool live, int lane) {
  const uint32_t uc = live ? (uint32_t)u : 0u;
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.scales[d] + (size_t)uc * 64, live ? 128u : 0u);
    const u2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, (uint32_t)(lane & 15) * 8u, 0, 0);
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
#pragma unroll
  for (int i = 0; i < SK_PD; ++i) sk_load<B, ND>(pp.ptr, pp.c[i], u0 + i, u0 + i < u1, lane);
}

// Walk the primed units [u0, u1) (segment-local, all of one tile, at most
// SK_UPW of them) and hand the tile's partial on.  tg0 = global index of the
// segment's first tile, xl / xsl = the segment's staged x and the quarter sums.
template <int B, int ND, bool ONE>
__device__ __forceinline__ void sk_run(const SkArgs& a, SkPipe<B, ND>& pp, int u0, int u1, int tg0,
                                       const uint4* xl, const float* xsl, int lane) {
  if (u0 >= u1) return;
  const int G4 = a.G4;
  const int q = lane >> 4, j = lane & 15;
  const float ko = -0.5f * (float)((1 << B) - 1) * 5.9604644775390625e-08f;  // -o * 2^-24
  float acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = 0.0f;
  const int tile = u0 / G4;
  auto step = [&](SkUnit<B, ND>& cu, int u) {
    const int quad = u - tile * G4;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int g = 4 * quad + gi;  // groups past G are staged as zeros and scaled by 0
      uint32_t xp[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 t = xl[(g * 4 + q) * 4 + v];
        xp[4 * v + 0] = t.x; xp[4 * v + 1] = t.y; xp[4 * v + 2] = t.z; xp[4 * v + 3] = t.w;
      }
      const float xs = xsl[g * 4 + q];
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        uint32_t g3[B];
        quad_group<B>(cu.cw[d], gi, g3);
        uint32_t r[16];
        decode_classes<B>(g3, r);
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
    float t = acc[d] * 16777216.0f;  // 2^24
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
    a.y[n] = f2h(ND == 2 ? silu_mul(v[0], v[1]) : v[0]);
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
    if ((int)(og & 63ull) == nch - 1) {
      const unsigned long long tu = fx_add(wu, 0ull);
      a.y[n] = f2h(silu_mul(fx_value(og + ag), fx_value(tu)));
      __hip_atomic_store(wg, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(wu, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    const unsigned long long og = fx_add(wg, ag);
    if ((int)(og & 63ull) == nch - 1) {
      a.y[n] = f2h(fx_value(og + ag));
      __hip_atomic_store(wg, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Stage x (scaled per class for each width segment) and the quarter sums in LDS.
// The loads go first (sk_x_load, into registers), so that a wave can issue its
// first code loads behind them and wait for x alone; sk_x_store then scales,
// sums and writes.  Thread t handles uint4 t, t + blockDim, ... of the padded
// row (G4 * 64 uint4, at most SK_XR per thread).
constexpr int SK_XR = 8;

__device__ __forceinline__ void sk_x_load(const uint16_t* x, int G, int G4, uint4 (&xr)[SK_XR]) {
  const int n16 = G4 * 64, nx = G * 16;
#pragma unroll
  for (int r = 0; r < SK_XR; ++r) {
    const int i = threadIdx.x + r * (int)blockDim.x;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)nx * 16u);
    const u4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)min(i, n16) * 16u, 0, 0);  // past nx: 0
    xr[r] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

template <int B>
__device__ __forceinline__ void sk_x_store(const uint4 (&xr)[SK_XR], int G4, uint4* xl, float* xsl, bool sums) {
  const int n16 = G4 * 64;
  const int pos = threadIdx.x & 3;  // position of the uint4 within its 32-element quarter
  uint32_t f[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t f0 = class_scale_pair<B>(e), f1 = class_scale_pair<B>(4 + e);
    const uint32_t f2 = class_scale_pair<B>(8 + e), f3 = class_scale_pair<B>(12 + e);
    f[e] = pos == 0 ? f0 : pos == 1 ? f1 : pos == 2 ? f2 : f3;
  }
  const uint32_t ones = 0x3C003C00u;  // fp16 (1, 1)
#pragma unroll
  for (int r = 0; r < SK_XR; ++r) {
    const int i = threadIdx.x + r * (int)blockDim.x;  // blockDim is a multiple of 64: whole waves pass
    if (r * (int)blockDim.x >= n16) break;
    const uint4 v = xr[r];
    float ps = dot2(v.x, ones, 0.0f);
    ps = dot2(v.y, ones, ps);
    ps = dot2(v.z, ones, ps);
    ps = dot2(v.w, ones, ps);
    ps += dpp_xor1(ps);
    ps += dpp_xor2(ps);
    if (i < n16) {
      xl[i] = make_uint4(pk_mul_f16(v.x, f[0]), pk_mul_f16(v.y, f[1]), pk_mul_f16(v.z, f[2]), pk_mul_f16(v.w, f[3]));
      if (sums && pos == 0) xsl[i >> 2] = ps;
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

// BF: the single code width of the matrices, or 0 (several width segments)
// one workgroup's runs over a segment of width B: x loads, then the first
// units' loads, then x staged (scaled for width B), then the runs
template <int B, int ND, bool ONE>
__device__ __forceinline__ void sk_body(const SkArgs& a, const SegDev (&sd)[2], int64_t lo, int64_t hi, char* smem,
                                        int lane) {
  const float* xsl = reinterpret_cast<const float*>(smem + (size_t)a.G4 * 1024);
  uint4 xr[SK_XR];
  sk_x_load(a.x, a.G, a.G4, xr);
  int v0, v1;
  sk_seg_range(sd[0], a.G4, lo, hi, v0, v1);
  SkPipe<B, ND> pp;
  sk_prime<B, ND>(pp, sd, v0, v1, lane);
  sk_x_store<B>(xr, a.G4, reinterpret_cast<uint4*>(smem), const_cast<float*>(xsl), true);
  lds_barrier();  // orders the staged x only (a full barrier would wait for the primed code loads)
  sk_run<B, ND, ONE>(a, pp, v0, v1, sd[0].tile0, reinterpret_cast<const uint4*>(smem), xsl, lane);
}

// BF: the single code width of the matrices, or 0 (several width segments:
// every workgroup then belongs to one segment, so it stages x for one width)
template <int BF, int ND>
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
  // (global units [lo, hi)); waves past the segment's last tile only help stage x
  const int gw = ((int)blockIdx.x - (BF == 0 ? a.wg_prefix[si] : 0)) * NW + wave;
  const int tl = gw / a.nch, ch = gw - tl * a.nch;
  const bool live = tl < sd[0].tiles;
  const int64_t t0 = (int64_t)(sd[0].tile0 + tl) * a.G4;
  const int64_t lo = live ? t0 + ch * a.G4 / a.nch : a.U;
  const int64_t hi = live ? t0 + (ch + 1) * a.G4 / a.nch : a.U;
  if constexpr (BF != 0) {
    sk_body<BF, ND, true>(a, sd, lo, hi, smem, lane);
  } else {
    if (sd[0].bits == 2) sk_body<2, ND, false>(a, sd, lo, hi, smem, lane);
    else if (sd[0].bits == 3) sk_body<3, ND, false>(a, sd, lo, hi, smem, lane);
    else sk_body<4, ND, false>(a, sd, lo, hi, smem, lane);
  }
}

}  // namespace qg
