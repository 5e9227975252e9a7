// qg_kernels.h -- HIP kernels for gfx950: weight re-layout, the M=1 GEMV (vector
// ALU, fp16 dot2), the 2..32-row skinny GEMM (MFMA 16x16x32 f16), the fixed-order
// split-K reduction and the checking kernels.  Layout and decode: qg_decode.h.
//
// Arithmetic (uniform b-bit codes, offset o = (2^b - 1)/2, group g of 128 k):
//   y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] * (c[n][k] - o)
// The GEMV stages x once per workgroup, each element times 2^-class of the code
// position it meets, so one dot2 chain over the exact subnormal code values
// gives 2^-24 * sum x*c whatever the class; the chain starts from the offset
// term -o * 2^-24 * (sum of the lane's 32 x, staged beside x) and the scale is
// applied per group, all in fp32.  The MFMA
// path feeds codes at scale 2^-23 and starts every group's accumulation from
// the offset product x * (-o * 2^-23), so each group's MFMA chain yields
// 2^-23 * sum x*(c - o) directly; the scale is applied per group in fp32.
// Workgroups never share an output element except through the split-K
// workspace, whose partials are summed in slice order: results are
// bit-reproducible.
//
// Memory-instruction discipline (measured on gfx950): every 64-lane load costs
// address-pipeline time even when it moves no data, so the run kernels issue
// only full-width 16-byte-per-lane loads, never a load for data they do not
// use, and issue all of them unconditionally so the compiler can count them
// and wait for exactly the one it needs next.
#pragma once
#include "qg_decode.h"

namespace qg {

constexpr int MAX_SEG = 3;

struct SegDev {
  const uint32_t* codes;   // device layout, [tiles][G4][bits][64][4] words
  const uint16_t* scales;  // [tiles][G4][16][4] fp16
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
  int* counters;           // one arrival counter per tile set (all zero between runs)
  int M, K, G, G4, ldy, NP;
  int T, S;                // tiles per workgroup, K slices across workgroups
  int pair;                // M = 1 gate/up pass with one matrix per workgroup (w[0], w[1])
  unsigned long long* xw;  // per padded column word, zero between runs: the pair pass's exchange
                           // word (one K slice) or, with fx, the K slices' fixed-point sum
  int fx;                  // one matrix, K slices: meet in fixed-point words (else partials)
  int ts_prefix[MAX_SEG + 1];  // prefix sums of tile-sets per segment
};

__device__ __forceinline__ SegDev pick(const WSet& w, int si) {
  SegDev s = w.seg[0];
  if (si == 1) s = w.seg[1];
  if (si == 2) s = w.seg[2];
  return s;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Workgroup barrier that orders LDS only: weight loads still in flight are not
// waited for (a full __syncthreads() would wait for every outstanding load).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float dpp_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}
// value of lane (l & ~15) | ((l - N) & 15): rotation right within each row of 16 lanes
template <int N> __device__ __forceinline__ float dpp_row_ror(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF, false));
}

// scale of group g, column j of tile t (scales layout [tile][G4][16][4])
__device__ __forceinline__ size_t scale_index(int t, int G4, int g, int j) {
  return (((size_t)t * G4 + (g >> 2)) * 16 + j) * 4 + (g & 3);
}

// ---------------------------------------------------------------------------
// create-time re-layout: canonical stream -> device layout (one thread per
// tile, quad and lane)
// ---------------------------------------------------------------------------
__global__ void k_repack_uniform(const uint32_t* __restrict__ canon, const int64_t* __restrict__ row_off,
                                 const uint16_t* __restrict__ scales_in, const int32_t* __restrict__ cols,
                                 int bits, int tiles, int G, int G4, uint32_t* __restrict__ dcodes,
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
  if (q == 0) {
    for (int gi = 0; gi < 4; ++gi) {
      const int g = 4 * qu + gi;
      dscales[((size_t)tq * 16 + j) * 4 + gi] = (n >= 0 && g < G) ? scales_in[(int64_t)n * G + g] : (uint16_t)0;
    }
  }
}

// ---------------------------------------------------------------------------
// split-K: each workgroup of a tile set writes its slice's partial sums to the
// workspace; the workgroup that arrives last (device-scope counter, one per
// tile set) adds the S partials in slice order 0..S-1 and stores the result,
// then re-arms the counter.  No floating-point atomics, so the order of
// arrival never changes a bit of the output.
//
// The partials are written and read only with agent-scope atomic accesses,
// which go to the device coherence point past the per-XCD L2 caches by
// themselves: so no cache write-back or invalidation (a device-wide fence,
// which writes back a whole L2) is needed.  Every thread waits until its own
// partial stores have completed, the workgroup synchronises, one thread counts
// the arrival, and only a workgroup that has seen every other slice arrive
// reads the partials.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_partial(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// sum_{k < n} (k == own ? own_v : p[k * stride]) in the order k = 0, 1, ...: the
// loads go out eight at a time (one round trip per eight partials, not one
// each); own < 0 means every partial comes from memory
__device__ __forceinline__ float sum_partials(const float* p, size_t stride, int n, int own = -1, float own_v = 0.0f) {
  float t = 0.0f;
  for (int k0 = 0; k0 < n; k0 += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + i;
      v[i] = (k < n && k != own) ? ld_partial(p + (size_t)k * stride) : own_v;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (k0 + i < n) t += v[i];
  }
  return t;
}
// Fixed-point accumulation words (the order-independent alternative to the
// partials above): each contributor adds (round(v * 2^28) << 6) + 1 (v clamped
// to +-2^23) to a 64-bit word with one integer atomic.  Integer addition is
// exact and commutative, so the total does not depend on the order of arrival,
// and the low 6 bits count the arrivals (at most 63 contributors per word).
constexpr int FX_FRAC = 28;  // fraction bits

__device__ __forceinline__ unsigned long long fx_word(float v) {
  const float vc = fminf(fmaxf(v, -8388608.0f), 8388608.0f);  // +-2^23
  return ((unsigned long long)__double2ll_rn((double)vc * (double)(1ll << FX_FRAC)) << 6) + 1ull;
}

__device__ __forceinline__ unsigned long long fx_add(unsigned long long* w, unsigned long long v) {
  return __hip_atomic_fetch_add(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float fx_value(unsigned long long total) {
  return (float)((double)((long long)total >> 6) * (1.0 / (double)(1ll << FX_FRAC)));
}

__device__ __forceinline__ bool splitk_last(int* counter, int S, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// ---------------------------------------------------------------------------
// M = 1 GEMV (VALU).  Workgroup = NW waves on one 16-column tile and one K
// slice of quads; wave w owns NQ consecutive quads (the last wave's surplus
// lies outside its buffer range and reads nothing).  Each wave issues all its
// code loads at once, right after the x and scale loads of the workgroup
// prologue, and consumes them in order.  The fused gate/up pass runs either
// with both matrices in each workgroup (DUAL) or, by default, with one matrix
// per workgroup (a.pair): the two workgroups of a tile then meet in an
// exchange word, or, with K slices, in the partials.
// ---------------------------------------------------------------------------

// LDS layout (bytes): x slice 4*nqs*256 | quarter sums 4*nqs*16 | scales
// ND*nqs*128 | cross-wave partials 2*NW*16*4 | flag 16
__host__ __device__ constexpr size_t m1_lds_bytes(int nqs, int ND, int NW) {
  return (size_t)nqs * 1024 + (size_t)nqs * 64 + (size_t)ND * nqs * 128 + (size_t)2 * NW * 64 + 16;
}

template <int B, int NQ, int ND>
__device__ __forceinline__ void gemv_q_body(const RunArgs& a, const SegDev (&sd)[2], int tile, int q_beg, int q_end,
                                            char* smem, float (&R)[2]) {
  using P = Pair<B>;
  // several widths inline one body per width behind a branch: keep the
  // compiler from hoisting the bodies' common loads above it (they would then
  // hold registers through every body)
  __asm__ volatile("" ::: "memory");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.G, G4 = a.G4;
  const int nqs = q_end - q_beg;                       // quads in the slice
  const int g_beg = 4 * q_beg, g_end = min(4 * q_end, G);
  const int ngs = g_end - g_beg;                        // real groups in the slice
  uint4* xl = reinterpret_cast<uint4*>(smem);
  float* xs = reinterpret_cast<float*>(smem + (size_t)nqs * 1024);
  uint16_t* sl = reinterpret_cast<uint16_t*>(smem + (size_t)nqs * 1088);
  // ---- prologue loads: x slice (16 B per thread per pass), scales (4 B per thread)
  const uint4* xg = reinterpret_cast<const uint4*>(a.x + (size_t)g_beg * 128);
  const int nx = ngs * 16;
  const uint4 xr0 = xg[min(tid, max(nx - 1, 0))];
  const uint4 xr1 = xg[min(tid + (int)blockDim.x, max(nx - 1, 0))];
  const int nsw = nqs * 32;                             // scale words per matrix
  uint32_t sr[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(sd[d].scales + ((size_t)tile * G4 + q_beg) * 64);
    sr[d] = sp[min(tid, nsw - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the prologue loads ahead of the code loads
  // ---- code loads: NQ quads per wave, buffer range = the wave's real quads
  const int qw0 = q_beg + wave * NQ;
  // wave-uniform, and kept in a scalar register: the compiler computes the clamp
  // with a vector instruction, and a descriptor built from a vector register
  // is taken as divergent (each load wrapped in a per-lane descriptor loop)
  const int nvalid = __builtin_amdgcn_readfirstlane(max(0, min(NQ, q_end - qw0)));
  uint32_t cw[ND][NQ][4 * B];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const uint32_t* base = sd[d].codes + ((size_t)tile * G4 + min(qw0, G4 - 1)) * (B * 256);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)nvalid * (B * 1024u));
#pragma unroll
    for (int u = 0; u < NQ; ++u) buffer_quad<B>(rs, (uint32_t)lane, u, cw[d][u]);
  }
  // ---- prologue stores: x (each element times 2^-class of the code position
  // it meets, so one dot2 chain serves every class), 32-element quarter sums
  // (of x itself), scales
  {
    const uint32_t ones = 0x3C003C00u;  // fp16 (1, 1)
    const int pos = tid & 3;            // uint4 position within a quarter (blockDim % 4 == 0)
    uint32_t f[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t f0 = class_scale_pair<B>(e), f1 = class_scale_pair<B>(4 + e);
      const uint32_t f2 = class_scale_pair<B>(8 + e), f3 = class_scale_pair<B>(12 + e);
      f[e] = pos == 0 ? f0 : pos == 1 ? f1 : pos == 2 ? f2 : f3;
    }
    auto stage = [&](const uint4& v, int i) {
      float ps = dot2(v.x, ones, 0.0f);
      ps = dot2(v.y, ones, ps);
      ps = dot2(v.z, ones, ps);
      ps = dot2(v.w, ones, ps);
      ps += dpp_xor1(ps);
      ps += dpp_xor2(ps);
      if (i < nx) {
        xl[i] = make_uint4(pk_mul_f16(v.x, f[0]), pk_mul_f16(v.y, f[1]), pk_mul_f16(v.z, f[2]), pk_mul_f16(v.w, f[3]));
        if ((i & 3) == 0) xs[i >> 2] = ps;
      }
    };
    stage(xr0, tid);
    if ((int)blockDim.x < nx) stage(xr1, tid + (int)blockDim.x);
    for (int r = 2; r * (int)blockDim.x < nx; ++r) {
      const int i = tid + r * (int)blockDim.x;
      stage(xg[min(i, nx - 1)], i);
    }
    uint32_t* slw = reinterpret_cast<uint32_t*>(sl);
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      if (tid < nsw) slw[d * nsw + tid] = sr[d];
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(sd[d].scales + ((size_t)tile * G4 + q_beg) * 64);
      for (int i = tid + (int)blockDim.x; i < nsw; i += blockDim.x) slw[d * nsw + i] = sp[i];
    }
  }
  lds_barrier();
  // ---- compute
  const int q = lane >> 4, j = lane & 15;
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int gl = 4 * (qw0 + u - q_beg) + gi;        // group index within the slice
      if (u >= nvalid || gl >= ngs) break;
      uint32_t xp[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 u4 = xl[gl * 16 + q * 4 + v];
        xp[4 * v + 0] = u4.x; xp[4 * v + 1] = u4.y; xp[4 * v + 2] = u4.z; xp[4 * v + 3] = u4.w;
      }
      const float xsum = xs[gl * 4 + q];
      const float ko = -0.5f * (float)((1 << B) - 1) * 5.9604644775390625e-08f;  // -o * 2^-24
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        uint32_t g3[B];
        quad_group<B>(cw[d][u], gi, g3);
        uint32_t r[16];
        decode_classes<B>(g3, r);
        // 2^-24 * sum x * (c - o) over the lane's 32 weights
        float e0 = xsum * ko, e1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          e0 = dot2(r[i], xp[i], e0);
          e1 = dot2(r[i + 1], xp[i + 1], e1);
        }
        const float sxc = e0 + e1;
        // scales staged as [quad][16][4]
        const float s = h2f(sl[d * nsw * 2 + ((gl >> 2) * 16 + j) * 4 + (gl & 3)]);
        R[d] = __builtin_fmaf(s, sxc, R[d]);
      }
    }
  }
}

// several widths (BF = 0): the three bodies' registers are allocated together;
// capped so that seven waves fit on each SIMD (the decode shapes' grids of
// 4- and 5-wave workgroups then stay resident; the cap spills 4 registers,
// an eight-wave cap spills 17 and is slower than no cap)
template <int NQ, bool DUAL, int BF>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(BF == 0 && !DUAL && NQ <= 2 ? 7 : 1)))
void k_gemv_q(RunArgs a) {
  extern __shared__ __align__(16) char smem[];
  constexpr int ND = DUAL ? 2 : 1;
  const int NW = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.S, G4 = a.G4;
  // paired gate/up pass (DUAL false, a.pair set): the two matrices are taken as
  // extra K slices, slice index dm * S + s for matrix dm; the last arrival of a
  // tile set sums each matrix's slices and applies SiLU(g) * u
  const int P = (!DUAL && a.pair) ? 2 : 1;
  const int SP = S * P;
  const int sx = blockIdx.x % SP, tsg = blockIdx.x / SP;
  const int dm = sx / S, s = sx - dm * S;
  // single-width handles have one segment: no data-dependent argument loads
  int si = 0;
  if (BF == 0)
    while (si + 1 < a.w[0].nseg && tsg >= a.ts_prefix[si + 1]) ++si;
  SegDev sd[2];
  {
    const SegDev s0 = BF == 0 ? pick(a.w[0], si) : a.w[0].seg[0];
    const SegDev s1 = BF == 0 ? pick(a.w[1], si) : a.w[1].seg[0];
    sd[0] = (P == 2 && dm == 1) ? s1 : s0;
    sd[1] = DUAL ? s1 : sd[0];
  }
  const int tile = BF == 0 ? tsg - a.ts_prefix[si] : tsg;
  const int q_beg = (int)((int64_t)s * G4 / S), q_end = (int)((int64_t)(s + 1) * G4 / S);
  const int pc = 16 * (sd[0].tile0 + tile) + (tid & 15);
  // output column: the padded column itself for one width (no padding then);
  // with several widths looked up here, so the lookup is not on the tail
  int n_out = pc;
  if (BF == 0) n_out = tid < 16 ? a.w[0].col_map[pc] : -1;
  float R[2] = {0.0f, 0.0f};
  const int bits = sd[0].bits;
  if (BF == 2 || (BF == 0 && bits == 2)) gemv_q_body<2, NQ, ND>(a, sd, tile, q_beg, q_end, smem, R);
  else if (BF == 3 || (BF == 0 && bits == 3)) gemv_q_body<3, NQ, ND>(a, sd, tile, q_beg, q_end, smem, R);
  else gemv_q_body<4, NQ, ND>(a, sd, tile, q_beg, q_end, smem, R);
  const int nqs = q_end - q_beg;
  float* red = reinterpret_cast<float*>(smem + (size_t)nqs * 1088 + (size_t)ND * nqs * 128);
  int* flag = reinterpret_cast<int*>(red + 2 * NW * 16);
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    float v = R[d] * 16777216.0f;  // 2^24
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (lane < 16) red[(d * NW + wave) * 16 + lane] = v;
  }
  __syncthreads();
  const bool mine = tid < 16;
  float v[2] = {0.0f, 0.0f};
  if (mine) {
#pragma unroll
    for (int d = 0; d < ND; ++d)
      for (int w = 0; w < NW; ++w) v[d] += red[(d * NW + w) * 16 + tid];
  }
  if (P == 2 && S == 1) {
    // one K slice: the two workgroups of a tile meet in a per-column word.
    // Each swaps in (matrix + 1) << 32 | its fp32 bits; the one that gets a
    // non-zero word back holds both values, writes SiLU(g) * u and re-arms the
    // word.  One round trip per workgroup, and the result does not depend on
    // which matrix arrives first.
    if (mine) {
      const unsigned long long w = ((unsigned long long)(dm + 1) << 32) | __float_as_uint(v[0]);
      const unsigned long long o = __hip_atomic_exchange(a.xw + pc, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (o != 0ull) {
        const float other = __uint_as_float((uint32_t)o);
        const float g = dm == 0 ? v[0] : other, u = dm == 0 ? other : v[0];
        __hip_atomic_store(a.xw + pc, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (n_out >= 0) a.y[n_out] = f2h(silu_mul(g, u));
      }
    }
    return;
  }
  if (!DUAL && P == 1 && S > 1 && a.fx) {
    // K slices meet in fixed-point words (see fx_word): one atomic round trip;
    // the arrival that completes the count stores the result and re-arms the word
    if (mine) {
      unsigned long long* w = a.xw + pc;
      const unsigned long long part = fx_word(v[0]);
      const unsigned long long before = fx_add(w, part);
      if ((int)(before & 63ull) == S - 1) {
        if (n_out >= 0) a.y[n_out] = f2h(fx_value(before + part));
        __hip_atomic_store(w, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }
  if (SP > 1) {
    // partials [matrix][slice][NP]; the arriving workgroup adds its own value
    // in its slot of the fixed order instead of reading it back
    if (mine) {
#pragma unroll
      for (int d = 0; d < ND; ++d) st_partial(a.partial + (size_t)((d + dm) * S + s) * a.NP + pc, v[d]);
    }
    if (!splitk_last(a.counters + tsg, SP, flag)) return;
    if (mine) {
      const float own = v[0];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        if (d == 1 && ND == 1 && P == 1) break;
        const bool is_own = P == 1 || d == dm;
        v[d] = sum_partials(a.partial + (size_t)(d * S) * a.NP + pc, (size_t)a.NP, S, is_own ? s : -1,
                            P == 1 ? v[d] : own);
      }
    }
  }
  if (mine && n_out >= 0) a.y[n_out] = f2h((DUAL || P == 2) ? silu_mul(v[0], v[1]) : v[0]);
}

// ---------------------------------------------------------------------------
// 2..32-row skinny GEMM (MFMA 16x16x32 f16).  Workgroup = NW waves on T tiles;
// the waves split the K slice's quads.  Each wave keeps one quad of codes (and
// its scales) in flight ahead of the one it computes; the A fragments (MT
// 16-row tiles of x, from L2) run one group ahead.  Each group's A is reused
// for all T tiles.
// ---------------------------------------------------------------------------
template <int B, int T, int ND>
struct MfQuad {
  uint32_t cw[ND][T][4 * B];
  uint2 sc[ND][T];
};

template <int T, int ND>
struct MfRs {
  __amdgpu_buffer_rsrc_t c[ND][T];   // codes of the wave's quads
  __amdgpu_buffer_rsrc_t s[ND][T];   // scales of the wave's quads
};

template <int B, int T, int ND>
__device__ __forceinline__ void mf_load_quad(MfQuad<B, T, ND>& c, const MfRs<T, ND>& rs, int u, uint32_t lane) {
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      buffer_quad<B>(rs.c[d][t], lane, u, c.cw[d][t]);
      const u2_t sv = __builtin_amdgcn_raw_buffer_load_b64(rs.s[d][t], (lane & 15u) * 8u, (uint32_t)u * 128u, 0);
      c.sc[d][t] = make_uint2(sv.x, sv.y);
    }
}

template <int MT>
__device__ __forceinline__ void mf_load_a(h8_t (&A)[MT][4], const uint16_t* __restrict__ x, int M, int K, int g,
                                          int glast, int lane) {
  const int q = lane >> 4, j = lane & 15;
  const int gg = min(g, glast);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = min(16 * mt + j, M - 1);  // rows past M re-read row M-1; never stored
    const uint4* px = reinterpret_cast<const uint4*>(x + (size_t)row * K + (size_t)gg * 128 + 32 * q);
#pragma unroll
    for (int v = 0; v < 4; ++v) A[mt][v] = __builtin_bit_cast(h8_t, px[v]);
  }
}

template <int B, int T, int MT, int ND>
__device__ __forceinline__ void mf_group(const MfQuad<B, T, ND>& c, int gi, const h8_t (&A)[MT][4],
                                         f4_t (&R)[2][T][MT]) {
  const uint32_t op = off1_offset_pair<B>();
  const h8_t boff = as_h8(op, op, op, op);
  f4_t Coff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    f4_t cc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int v = 0; v < 4; ++v) cc = mfma16(A[mt][v], boff, cc);
    Coff[mt] = cc;
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      uint32_t g3[B];
      quad_group<B>(c.cw[d][t], gi, g3);
      uint32_t r[16];
      decode_off1<B>(g3, r);
      const uint32_t sw = (gi < 2) ? c.sc[d][t].x : c.sc[d][t].y;
      const float s = h2f((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f4_t cc = Coff[mt];
#pragma unroll
        for (int v = 0; v < 4; ++v) cc = mfma16(A[mt][v], as_h8(r[4 * v], r[4 * v + 1], r[4 * v + 2], r[4 * v + 3]), cc);
#pragma unroll
        for (int e = 0; e < 4; ++e) R[d][t][mt][e] = __builtin_fmaf(s, cc[e], R[d][t][mt][e]);
      }
    }
}

template <int B, int T, int MT, int ND>
__device__ __forceinline__ void mfma_body(const RunArgs& a, const SegDev (&sd)[2], int tl0, int tiles, int qw0,
                                          int qw1, int lane, f4_t (&R)[2][T][MT]) {
  const int G = a.G, G4 = a.G4;
  const int nq = qw1 - qw0;
  const int glast = max(min(4 * qw1, G) - 1, 0);
  MfRs<T, ND> rs;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int tt = min(tl0 + t, tiles - 1);  // tiles past the segment re-read a valid one (never stored)
      const size_t qb = (size_t)tt * G4 + min(qw0, G4 - 1);
      rs.c[d][t] = make_rsrc(sd[d].codes + qb * (B * 256), (uint32_t)max(nq, 0) * (B * 1024u));
      rs.s[d][t] = make_rsrc(sd[d].scales + qb * 64, (uint32_t)max(nq, 0) * 128u);
    }
  MfQuad<B, T, ND> c0, c1;
  h8_t A0[MT][4], A1[MT][4];
  mf_load_a<MT>(A0, a.x, a.M, a.K, 4 * qw0, glast, lane);
  mf_load_quad(c0, rs, 0, (uint32_t)lane);
  mf_load_quad(c1, rs, 1, (uint32_t)lane);
  for (int u = 0; u < nq; u += 2) {
    const int g0 = 4 * (qw0 + u);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      if (gi % 2 == 0) {
        mf_load_a<MT>(A1, a.x, a.M, a.K, g0 + gi + 1, glast, lane);
        if (g0 + gi < G) mf_group<B, T, MT, ND>(c0, gi, A0, R);
      } else {
        mf_load_a<MT>(A0, a.x, a.M, a.K, g0 + gi + 1, glast, lane);
        if (g0 + gi < G) mf_group<B, T, MT, ND>(c0, gi, A1, R);
      }
    }
    mf_load_quad(c0, rs, u + 2, (uint32_t)lane);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      if (gi % 2 == 0) {
        mf_load_a<MT>(A1, a.x, a.M, a.K, g0 + 4 + gi + 1, glast, lane);
        if (u + 1 < nq && g0 + 4 + gi < G) mf_group<B, T, MT, ND>(c1, gi, A0, R);
      } else {
        mf_load_a<MT>(A0, a.x, a.M, a.K, g0 + 4 + gi + 1, glast, lane);
        if (u + 1 < nq && g0 + 4 + gi < G) mf_group<B, T, MT, ND>(c1, gi, A1, R);
      }
    }
    mf_load_quad(c1, rs, u + 3, (uint32_t)lane);
  }
}

template <int T, int MT, bool DUAL, int BF>
__global__ __launch_bounds__(512) void k_gemm_mfma(RunArgs a) {
  extern __shared__ __align__(16) char smem[];
  constexpr int ND = DUAL ? 2 : 1;
  const int NW = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.S, G4 = a.G4;
  const int s = blockIdx.x % S, tsg = blockIdx.x / S;
  int si = 0;
  if (BF == 0)
    while (si + 1 < a.w[0].nseg && tsg >= a.ts_prefix[si + 1]) ++si;
  SegDev sd[2];
  sd[0] = BF == 0 ? pick(a.w[0], si) : a.w[0].seg[0];
  sd[1] = DUAL ? (BF == 0 ? pick(a.w[1], si) : a.w[1].seg[0]) : sd[0];
  const SegDev& sg = sd[0];
  const int tl0 = (BF == 0 ? tsg - a.ts_prefix[si] : tsg) * T;
  const int q_beg = (int)((int64_t)s * G4 / S), q_end = (int)((int64_t)(s + 1) * G4 / S);
  const int nqs = q_end - q_beg;
  const int qw0 = q_beg + (int)((int64_t)wave * nqs / NW);
  const int qw1 = q_beg + (int)((int64_t)(wave + 1) * nqs / NW);
  f4_t R[2][T][MT];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) R[d][t][mt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  if (BF == 2 || (BF == 0 && sg.bits == 2)) mfma_body<2, T, MT, ND>(a, sd, tl0, sg.tiles, qw0, qw1, lane, R);
  else if (BF == 3 || (BF == 0 && sg.bits == 3)) mfma_body<3, T, MT, ND>(a, sd, tl0, sg.tiles, qw0, qw1, lane, R);
  else mfma_body<4, T, MT, ND>(a, sd, tl0, sg.tiles, qw0, qw1, lane, R);
  // cross-wave reduction in LDS, fixed wave order
  float* red = reinterpret_cast<float*>(smem);
  constexpr int PER = T * MT * 4;  // floats per lane per matrix
  int* flag = reinterpret_cast<int*>(red + (size_t)ND * NW * PER * 64);
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
  // pass 1: sum the waves in order into wave 0's slot
  for (int idx = tid; idx < total; idx += blockDim.x) {
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      float v = 0.0f;
      for (int w = 0; w < NW; ++w) v += red[(size_t)(d * NW + w) * PER * 64 + idx];
      red[(size_t)(d * NW) * PER * 64 + idx] = v * 8388608.0f;  // 2^23
    }
  }
  __syncthreads();
  if (S > 1) {
    for (int idx = tid; idx < total; idx += blockDim.x) {
      const int ln = idx & 63, rest = idx >> 6;
      const int e = rest & 3, tm = rest >> 2;
      const int mt = tm % MT, t = tm / MT;
      const int row = 16 * mt + 4 * (ln >> 4) + e;
      if (row >= a.M || tl0 + t >= sg.tiles) continue;
      const int pc = 16 * (sg.tile0 + tl0 + t) + (ln & 15);
#pragma unroll
      for (int d = 0; d < ND; ++d)
        st_partial(a.partial + ((size_t)(d * S + s) * a.M + row) * a.NP + pc, red[(size_t)(d * NW) * PER * 64 + idx]);
    }
    if (!splitk_last(a.counters + tsg, S, flag)) return;
  }
  for (int idx = tid; idx < total; idx += blockDim.x) {
    const int ln = idx & 63, rest = idx >> 6;
    const int e = rest & 3, tm = rest >> 2;
    const int mt = tm % MT, t = tm / MT;
    const int row = 16 * mt + 4 * (ln >> 4) + e;
    const int tl = tl0 + t;
    if (row >= a.M || tl >= sg.tiles) continue;
    const int pc = 16 * (sg.tile0 + tl) + (ln & 15);
    float v[2];
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      if (S > 1) {
        float acc = 0.0f;
        acc = sum_partials(a.partial + ((size_t)(d * S) * a.M + row) * a.NP + pc, (size_t)a.M * a.NP, S);
        v[d] = acc;
      } else {
        v[d] = red[(size_t)(d * NW) * PER * 64 + idx];
      }
    }
    const int n = BF != 0 ? pc : a.w[0].col_map[pc];  // one width: no padding, identity
    if (n >= 0) a.y[(size_t)row * a.ldy + n] = f2h(DUAL ? silu_mul(v[0], v[1]) : v[0]);
  }
}

// ---------------------------------------------------------------------------
// checking kernel: the GEMV decode of every lane-slot, written back in [N][K]
// ---------------------------------------------------------------------------
template <int B>
__device__ __forceinline__ void debug_slot(const SegDev& sg, const int32_t* col_map, int G, int G4, int K,
                                           int64_t gid, int32_t* codes, float* w, uint16_t* q16) {
  using P = Pair<B>;
  const int lane = (int)(gid & 63);
  const int64_t tg = gid >> 6;
  const int g = (int)(tg % G), tl = (int)(tg / G);
  const int j = lane & 15, q = lane >> 4;
  const int n = col_map[16 * (sg.tile0 + tl) + j];
  if (n < 0) return;
  uint32_t cw[B];
#pragma unroll
  for (int u = 0; u < B; ++u) cw[u] = sg.codes[code_word_index(tl, G4, g, lane, u, B)];
  uint32_t r[16];
  decode_classes<B>(cw, r);
  const float s = h2f(sg.scales[scale_index(tl, G4, g, j)]);
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

__global__ void k_debug_uniform(SegDev sg, const int32_t* col_map, int G, int G4, int K, int32_t* codes, float* w,
                                uint16_t* q16) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)sg.tiles * G * 64) return;
  switch (sg.bits) {
    case 2: debug_slot<2>(sg, col_map, G, G4, K, gid, codes, w, q16); break;
    case 3: debug_slot<3>(sg, col_map, G, G4, K, gid, codes, w, q16); break;
    default: debug_slot<4>(sg, col_map, G, G4, K, gid, codes, w, q16); break;
  }
}

}  // namespace qg
