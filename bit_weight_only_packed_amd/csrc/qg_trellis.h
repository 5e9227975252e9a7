// qg_trellis.h -- bitshift-trellis weights (3 bits/weight, 65536-entry fp16
// codebook) on gfx950: create-time re-layout, the in-register window decode,
// the Walsh-Hadamard rotation of x, the M = 1 GEMV (v_dot2_f32_f16), the
// M = 2..32 GEMM (v_mfma_f32_16x16x32_f16) and the checking kernel.
//
// Format (trellis family of "OrcaSAQ2-27B on AMD Radeon -- ROCm runtime", intro:
// EXL3 trellis weights near 3 bits/weight): a 16x16 tile (16 output rows n x 16
// input columns k) is a 768-bit stream, 48 uint16 words taken MSB first.
// Weight i = 16*r + c of the tile takes the 16-bit window of the stream that
// starts at bit 3*i, read cyclically (the windows of the last weights wrap to
// the start of the tile's stream), as an unsigned index into the codebook;
// w = codebook[state] * s[n][k/128].  Before the product x is rotated by the
// normalised 128-point Walsh-Hadamard transform of each 128-group (natural
// order, factor 2^-3.5).
//
// Device layout.  Row block rb = 16 rows; unit (rb, g) = the 8 tiles of group g
// (16 rows x 128 k).  Lane l of a wave owns row n = l & 15 and quarter
// kq = l >> 4 of the group: k = 128g + 32kq + j, j = 0..31, which is row n of
// the two tiles A = 8g + 2kq (j < 16) and B = A + 1 (j >= 16).  The lane's three
// words hold those two 48-bit rows back to back, MSB first:
//   Z2 = A[3n] << 16 | A[3n+1],  Z1 = A[3n+2] << 16 | B[3n],  Z0 = B[3n+1] << 16 | B[3n+2]
// at uint32 index (unit * 64 + l) * 3, so one wave-wide 12-byte-per-lane load
// reads a unit's 768 contiguous bytes once.  The 15 bits of look-ahead that the
// last windows of a row need are the first bits of the next row of the same
// tile (row 0 after row 15), which the lane of row n + 1 mod 16 in the same
// quarter holds: two DPP row rotations per unit.  Scales: fp16 [unit][16].
//
// Decode.  With a row as a 64-bit value R (row bits at 63..16, the next row's
// first 16 bits at 15..0), 2 * state_c = (R >> (47 - 3c)) & 0x1FFFE: one funnel
// shift (v_alignbit_b32) and one AND give the byte address of the codebook
// entry in LDS, whose fp16 value is used as is (exact); the scale multiplies
// each group's fp32 partial sum.
#pragma once
#include "qg_common.h"

namespace qg {


// ---------------------------------------------------------------------------
// create-time re-layout (one thread per unit and lane)
// ---------------------------------------------------------------------------
__global__ void k_repack_trellis(const uint16_t* __restrict__ tiles, const uint16_t* __restrict__ scales_in, int KT,
                                 int G, int64_t units, uint32_t* __restrict__ dcodes, uint16_t* __restrict__ dscales) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= units * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t u = gid >> 6;
  const int rb = (int)(u / G), g = (int)(u % G);
  const int n = lane & 15, kq = lane >> 4;
  const uint16_t* A = tiles + ((int64_t)rb * KT + 8 * g + 2 * kq) * 48 + 3 * n;
  const uint16_t* Bt = A + 48;
  uint32_t* o = dcodes + gid * 3;
  o[0] = ((uint32_t)A[0] << 16) | A[1];
  o[1] = ((uint32_t)A[2] << 16) | Bt[0];
  o[2] = ((uint32_t)Bt[1] << 16) | Bt[2];
  if (kq == 0) dscales[u * 16 + n] = scales_in[((int64_t)rb * 16 + n) * G + g];
}

// ---------------------------------------------------------------------------
// decode: codebook byte addresses of the lane's 32 weights (k = 32kq + j)
// ---------------------------------------------------------------------------
// the value of lane (l & ~15) | ((l + 1) & 15): a DPP rotate of each 16-lane row
// (row_ror by 15 moves every lane's value one lane down, the first to the last)
__device__ __forceinline__ uint32_t tr_from_next_row_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x12F, 0xF, 0xF, false);
}

// addr[j] = 2 * state of weight j; z = the lane's words, nz2 / nz1 = Z2 / Z1 of
// the lane holding row n + 1 mod 16 of the same tiles
__device__ __forceinline__ void tr_addrs(uint32_t z2, uint32_t z1, uint32_t z0, uint32_t nz2, uint32_t nz1,
                                         uint32_t (&addr)[32]) {
  // row A as (hi, lo) = (Z2, Z1.hi16 : next row's first 16 bits)
  const uint32_t la = __builtin_amdgcn_perm(z1, nz2, 0x07060302u);  // bytes z1[3:2], nz2[3:2]
  // row B as (hb, lb) = (Z1.lo16 : Z0.hi16, Z0.lo16 : next row's first 16 bits)
  const uint32_t hb = __builtin_amdgcn_perm(z1, z0, 0x05040302u);   // bytes z1[1:0], z0[3:2]
  const uint32_t lb = __builtin_amdgcn_perm(z0, nz1, 0x05040100u);  // bytes z0[1:0], nz1[1:0]
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const int s = 47 - 3 * c;
    uint32_t va, vb;
    if (s >= 32) {
      va = z2 >> (s - 32);
      vb = hb >> (s - 32);
    } else {
      va = __builtin_amdgcn_alignbit(z2, la, s);
      vb = __builtin_amdgcn_alignbit(hb, lb, s);
    }
    addr[c] = va & 0x1FFFEu;
    addr[16 + c] = vb & 0x1FFFEu;
  }
}

__device__ __forceinline__ _Float16 cb_at(const char* cbl, uint32_t a) {
  return *reinterpret_cast<const _Float16*>(cbl + a);
}

// the lane's 32 codebook values as 16 fp16 pairs (weights 2p, 2p+1 in pair p)
__device__ __forceinline__ void tr_gather(const char* cbl, const uint32_t (&addr)[32], uint32_t (&pr)[16]) {
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    h2_t v;
    v.x = cb_at(cbl, addr[2 * p]);
    v.y = cb_at(cbl, addr[2 * p + 1]);
    pr[p] = __builtin_bit_cast(uint32_t, v);
  }
}

// ---------------------------------------------------------------------------
// rotation: x'[m][128g + j] = 2^-3.5 * sum_i (-1)^popcount(i & j) x[m][128g + i]
// One wave per (row, group); lane l holds elements l and l + 64.  Butterflies in
// fp32 (the sums of 128 fp16 values with signs are exact to fp32 rounding), one
// rounding to fp16 at the end.
// ---------------------------------------------------------------------------
// value of lane l ^ 4: quad mirror (3 - i) then half-row mirror (7 - i)
__device__ __forceinline__ float dpp_xor4(float v) {
  const int m = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x1B, 0xF, 0xF, false);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, m, 0x141, 0xF, 0xF, false));
}

// the six cross-lane butterfly stages of a 128-point transform held as two
// values per lane (elements lane and lane + 64), partner lane l ^ h for
// h = 32, 16, 8, 4, 2, 1: the two across rows through the LDS crossbar, the
// four inside a 16-lane row as DPP moves (no LDS round trip)
__device__ __forceinline__ void fwht_lanes(float& a, float& b, int lane) {
  auto stage = [&](float pa, float pb, int h) {
    const bool upper = (lane & h) != 0;
    a = upper ? pa - a : a + pa;
    b = upper ? pb - b : b + pb;
  };
  stage(__shfl_xor(a, 32), __shfl_xor(b, 32), 32);
  stage(__shfl_xor(a, 16), __shfl_xor(b, 16), 16);
  stage(dpp_row_ror<8>(a), dpp_row_ror<8>(b), 8);  // (i + 8) mod 16 = i ^ 8
  stage(dpp_xor4(a), dpp_xor4(b), 4);
  stage(dpp_xor2(a), dpp_xor2(b), 2);
  stage(dpp_xor1(a), dpp_xor1(b), 1);
}

__global__ __launch_bounds__(256) void k_fwht(const uint16_t* __restrict__ x, uint16_t* __restrict__ xr, int M,
                                              int K) {
  const int G = K / 128;
  const int wv = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  if (wv >= M * G) return;
  const int lane = threadIdx.x & 63;
  const int m = wv / G, g = wv % G;
  const uint16_t* p = x + (size_t)m * K + (size_t)g * 128;
  float a = h2f(p[lane]), b = h2f(p[lane + 64]);
  {
    const float s = a + b, d = a - b;
    a = s;
    b = d;
  }
  fwht_lanes(a, b, lane);
  const float f = 0.08838834764831845f;  // 2^-3.5
  uint16_t* q = xr + (size_t)m * K + (size_t)g * 128;
  q[lane] = f2h(a * f);
  q[lane + 64] = f2h(b * f);
}

// ---------------------------------------------------------------------------
// M = 1 GEMV (dot2).  One workgroup per compute unit holds the codebook in LDS
// for the whole launch.  The RB * G units are split into W equal contiguous
// ranges in row-block-major order, one per wave (stream-K): a wave walks its
// range with the next units' loads in flight (PD register sets in rotation),
// accumulates while the row block stays the same and hands a partial sum on
// per row block it touches.  Where at most 63 waves share a row block the
// partials go into fixed-point output words (qg_common.h): one atomic round
// trip, and a sum that does not depend on the order of arrival.  Otherwise a
// row block's partials sit in fixed slots (slot = wave - first wave of the row
// block); the wave that completes the row block (device-scope arrival counter)
// adds the slots in slot order and stores the fp16 result.  Either way,
// repeated runs are bit-identical.
// ---------------------------------------------------------------------------

// first wave whose range holds unit x (ranges [w*U/W, (w+1)*U/W))
__device__ __forceinline__ int tr_wave_of(int64_t x, int64_t U, int W) {
  int w = (int)(x * W / U);
  while (w + 1 < W && ((int64_t)(w + 1) * U) / W <= x) ++w;
  while (w > 0 && ((int64_t)w * U) / W > x) --w;
  return w;
}


template <bool XL>
struct TrUnit {
  static constexpr int loads = 2 + (XL ? 0 : 4);  // load instructions per unit
  u3_t z;                                         // code words
  uint32_t s;                                     // this lane's scale (fp16 in the low half)
  uint4 xv[4];                                    // activations: the lane's 32 k (not XL)
};

template <bool XL>
__device__ __forceinline__ void tr_load(const TrArgs& a, TrUnit<XL>& t, int64_t u, int g, bool live, int lane) {
  const int uu = live ? 1 : 0;
  const int64_t uc = live ? u : 0;
  const int kq = lane >> 4;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes + uc * 192, uu * 768u);
  t.z = __builtin_amdgcn_raw_buffer_load_b96(rc, (uint32_t)lane * 12u, 0, 0);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + uc * 16, uu * 32u);
  t.s = __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(lane & 14) * 2u, 0, 0);
  if (lane & 1) t.s >>= 16;
  if constexpr (XL) return;
  // one descriptor over all of x (wave-uniform, so no per-lane descriptor
  // loop); the lane's quarter goes into the offset, and a dead unit takes an
  // offset past the range: zeros, no memory access
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(uniform_ptr(a.x), (uint32_t)a.K * 2u);
  const uint32_t off = live ? (uint32_t)(((size_t)g * 128 + 32 * kq) * 2) : 0x80000000u;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const u4_t q = __builtin_amdgcn_raw_buffer_load_b128(rx, off + (uint32_t)v * 16u, 0, 0);
    t.xv[v] = make_uint4(q.x, q.y, q.z, q.w);
  }
}

// A wave's partials (agent-scope atomic stores, which bypass the per-XCD L2)
// have completed before it counts its arrival at the row block's counter; the
// wave that arrives last re-arms the counter and reads the other partials with
// agent-scope atomic loads.  No device-wide fence (an L2 write-back) is needed.
__device__ __forceinline__ bool tr_arrive_last(int* counter, int nseg, int lane) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old != nseg - 1) return false;
  if (lane == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

template <bool XL = false>
__global__ __launch_bounds__(64 * TR_NW) void k_trellis(TrArgs a) {
  // static (not dynamic) LDS: its address is a compile-time constant, so the
  // gathers use the decoded byte address as is
  __shared__ __align__(16) char smem[TR_CB_BYTES + (XL ? TR_XL_BYTES : 0)];
  const int lane = threadIdx.x & 63;
  const int NW = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * NW + wave;
  // W <= U: every wave below W has a non-empty range (the row blocks' arrival
  // counts rely on it); waves past W only help load the codebook
  const int64_t lo = gw < a.W ? (int64_t)gw * a.U / a.W : a.U;
  const int64_t hi = gw < a.W ? (int64_t)(gw + 1) * a.U / a.W : a.U;
  constexpr int PD = TR_PD;
  // codebook -> LDS straight from memory (buffer loads to LDS, 1 KiB per wave
  // instruction), then this wave's first units: waiting for the codebook does
  // not wait for those
  {
    const __amdgpu_buffer_rsrc_t rcb = make_rsrc(uniform_ptr(a.cb), TR_CB_BYTES);
    for (int ci = wave; ci < TR_CB_BYTES / 1024; ci += NW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rcb, (__attribute__((address_space(3))) void*)(smem + (size_t)ci * 1024),
                                               16, (uint32_t)(ci * 1024 + lane * 16), 0, 0, 0);
  }
  // XL: this wave's groups of the unrotated x (groups wave, wave + NW, ...)
  uint16_t xa[XL ? TR_XL_GMAX : 1], xb[XL ? TR_XL_GMAX : 1];
  if constexpr (XL) {
#pragma unroll
    for (int i = 0; i < TR_XL_GMAX; ++i) {
      const int g = wave + i * NW;
      xa[i] = g < a.G ? a.x[(size_t)g * 128 + lane] : (uint16_t)0;
      xb[i] = g < a.G ? a.x[(size_t)g * 128 + 64 + lane] : (uint16_t)0;
    }
  }
  TrUnit<XL> c[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) tr_load<XL>(a, c[i], lo + i, (int)((lo + i) % a.G), lo + i < hi, lane);
  {
    constexpr int n = PD * TrUnit<XL>::loads;  // loads issued after the codebook's (and x's)
    static_assert(n < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
  }
  if constexpr (XL) {
    // rotate each group as k_fwht does (same operations in the same order, so
    // the same fp16 values) and keep it in LDS after the codebook
    uint16_t* xr = reinterpret_cast<uint16_t*>(smem + TR_CB_BYTES);
#pragma unroll
    for (int i = 0; i < TR_XL_GMAX; ++i) {
      const int g = wave + i * NW;
      if (g >= a.G) break;
      float p = h2f(xa[i]), q = h2f(xb[i]);
      {
        const float su = p + q, df = p - q;
        p = su;
        q = df;
      }
      fwht_lanes(p, q, lane);
      const float f = 0.08838834764831845f;  // 2^-3.5
      xr[g * 128 + lane] = f2h(p * f);
      xr[g * 128 + 64 + lane] = f2h(q * f);
    }
  }
  lds_barrier();  // every wave's share of the codebook (and of the rotated x) has landed
  if (lo >= hi) return;
  const char* cbl = smem;
  float acc1 = 0.0f;
  // row block and group of the unit being computed, group of the next unit to
  // load (kept as counters: no division per unit)
  int rb = (int)(lo / a.G), g = (int)(lo - (int64_t)rb * a.G);
  int gpf = (int)((lo + PD) % a.G);
  // one unit: decode, contract, reload the same registers with unit u + PD, and
  // hand the row block on at the end of a row block or of the range
  auto step = [&](TrUnit<XL>& cu, int64_t u) {
    const uint32_t z2 = cu.z.x, z1 = cu.z.y, z0 = cu.z.z;
    const uint32_t nz2 = tr_from_next_row_lane(z2), nz1 = tr_from_next_row_lane(z1);
    uint32_t addr[32];
    tr_addrs(z2, z1, z0, nz2, nz1, addr);
    uint32_t pr[16];
    tr_gather(cbl, addr, pr);
    const float s = h2f((uint16_t)(cu.s & 0xFFFFu));
    uint4 xv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if constexpr (XL)
        xv[v] = *reinterpret_cast<const uint4*>(smem + TR_CB_BYTES + ((size_t)g * 128 + 32 * (lane >> 4)) * 2 + v * 16);
      else
        xv[v] = cu.xv[v];
    }
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      d0 = dot2(pr[4 * v + 0], xv[v].x, d0);
      d1 = dot2(pr[4 * v + 1], xv[v].y, d1);
      d0 = dot2(pr[4 * v + 2], xv[v].z, d0);
      d1 = dot2(pr[4 * v + 3], xv[v].w, d1);
    }
    acc1 = __builtin_fmaf(s, d0 + d1, acc1);
    tr_load<XL>(a, cu, u + PD, gpf, u + PD < hi, lane);
    gpf = gpf + 1 == a.G ? 0 : gpf + 1;
    const bool last_unit = u + 1 == hi;
    g = g + 1 == a.G ? 0 : g + 1;
    const int rb_next = g == 0 ? rb + 1 : rb;
    if (!last_unit && rb_next == rb) return;
    const int w0 = tr_wave_of((int64_t)rb * a.G, a.U, a.W);
    const int w1 = tr_wave_of((int64_t)rb * a.G + a.G - 1, a.U, a.W);
    const int nseg = w1 - w0 + 1, seg = gw - w0;
    const int n = lane & 15;
    float* base = a.partial + ((size_t)rb * a.maxseg) * 16;
    float v = acc1;
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (nseg == 1) {
      if (lane < 16) a.y[(size_t)rb * 16 + n] = f2h(v);
    } else if (a.acc) {
      // fixed-point words: one round trip; the arrival that completes the
      // count stores the result and re-arms the word
      if (lane < 16) {
        unsigned long long* w = a.acc + (size_t)rb * 16 + n;
        const unsigned long long mine = fx_word(v);
        const unsigned long long before = fx_add(w, mine);
        if (fx_count(before) == nseg - 1) {
          a.y[(size_t)rb * 16 + n] = f2h(fx_value(before + mine));
          fx_rearm(w);
        }
      }
    } else {
      if (lane < 16) st_partial(base + (size_t)seg * 16 + n, v);
      if (tr_arrive_last(a.counters + rb, nseg, lane)) {
        const float t = sum_partials(base + n, 16, nseg, seg, v);
        if (lane < 16) a.y[(size_t)rb * 16 + n] = f2h(t);
      }
    }
    acc1 = 0.0f;
    rb = rb_next;
  };
  for (int64_t u = lo; u < hi; u += PD) {
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      if (u + i >= hi) break;
      step(c[i], u + i);
    }
  }
}

// ---------------------------------------------------------------------------
// Banded GEMM for 2..32 rows.  In the stream-K kernel above every unit loads
// its own 16 rows of x, one row per lane: 64 different cache lines per load
// instruction, which the address pipeline takes one by one.  Here a workgroup
// owns a band of NW row blocks (one per wave) and a K slice of groups, and its
// waves walk the slice's groups in step: the x fragment of each group (MR rows
// x 128 k) is copied once per workgroup into LDS beside the codebook (dword
// buffer-to-LDS copies, each wave its share of the rows, XB slots in rotation,
// PD groups ahead), and every wave reads its A fragments from there.  A wave
// keeps one row block's sums over the whole slice; K slices meet as in the
// stream-K kernel (fixed slots, arrival counter, sums in slot order), or, when
// the outputs are few, in fixed-point output words (one atomic round trip).
// ---------------------------------------------------------------------------


// 4 bytes per lane from a buffer into LDS at lds + 4 * lane (lds wave-uniform),
// as assembly so the compiler does not make LDS reads wait for it (the kernel
// orders it with explicit waits and barriers); no register receives data.
__device__ __forceinline__ void lds_copy4(__amdgpu_buffer_rsrc_t r, const void* lds, uint32_t voff) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const __attribute__((address_space(3))) char*)(lds));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r) : "memory", "m0");
}

template <int N> __device__ __forceinline__ void tb_vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

struct TbUnit {
  u3_t z;      // code words
  uint32_t s;  // this lane's scale (fp16 in the low half)
};

template <int MT>
__global__ __launch_bounds__(64 * TbShape<MT>::NW) void k_trellis_band(TbArgs a) {
  using TS = TbShape<MT>;
  constexpr int PD = TS::PD, XB = TS::XB, MR = TS::MR, XRD = TS::XRD, NW = TS::NW, SLOT = TS::SLOT;
  // static LDS: the codebook at address 0 (the gathers use the decoded byte
  // address as is), then the x slots
  __shared__ __align__(16) char smem[TR_CB_BYTES + XB * SLOT];
  char* const xl = smem + TR_CB_BYTES;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = a.S;
  const int s = blockIdx.x % S, band = blockIdx.x / S;
  const int rb = band * NW + wave;
  const bool mine = rb < a.RB;
  const int g0 = (int)((int64_t)s * a.G / S), g1 = (int)((int64_t)(s + 1) * a.G / S), ng = g1 - g0;
  // codebook -> LDS (1 KiB per wave instruction)
  {
    const __amdgpu_buffer_rsrc_t rcb = make_rsrc(uniform_ptr(a.cb), TR_CB_BYTES);
    for (int ci = wave; ci < TR_CB_BYTES / 1024; ci += NW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rcb, (__attribute__((address_space(3))) void*)(smem + (size_t)ci * 1024),
                                               16, (uint32_t)(ci * 1024 + lane * 16), 0, 0, 0);
  }
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(uniform_ptr(a.x), (uint32_t)a.M * a.K * 2u);
  // Step i's x fragment (group g0 + i): this wave's rows m = XRD * wave + r, lane
  // l holding elements 2l and 2l + 1 of a row (rows past M and steps past the
  // slice read zeros), loaded PD steps ahead into register set i % PD; one step
  // before use it is rotated in registers (the Walsh-Hadamard matrix is the same
  // under one bit permutation of both its indices, so the butterflies work on
  // this pairing: the local stage pairs index bit 0, the lane stages bits 1..6)
  // and written to its slot, the 16-byte chunk p of row m at position p ^ (m & 15).
  uint32_t xr[PD][XRD];
  auto load_x = [&](int i, uint32_t (&v)[XRD]) {
    const int g = g0 + i;
#pragma unroll
    for (int r = 0; r < XRD; ++r) {
      const int m = XRD * wave + r;
      const uint32_t voff = (m < a.M && i < ng) ? (uint32_t)(((size_t)m * a.K + (size_t)g * 128 + 2 * lane) * 2) : 0xFFFFFFF0u;
      v[r] = __builtin_amdgcn_raw_buffer_load_b32(rx, voff, 0, 0);
    }
  };
  auto put_x = [&](const uint32_t (&v)[XRD], int sl) {
#pragma unroll
    for (int r = 0; r < XRD; ++r) {
      const int m = XRD * wave + r;
      uint32_t out = v[r];
      if (a.rot) {
        float p0 = h2f((uint16_t)(v[r] & 0xFFFFu)), p1 = h2f((uint16_t)(v[r] >> 16));
        const float sum = p0 + p1, dif = p0 - p1;
        p0 = sum;
        p1 = dif;
        fwht_lanes(p0, p1, lane);
        const float f = 0.08838834764831845f;  // 2^-3.5
        out = (uint32_t)f2h(p0 * f) | ((uint32_t)f2h(p1 * f) << 16);
      }
      const int pc = (lane >> 2) ^ (m & 15);
      *reinterpret_cast<uint32_t*>(xl + (size_t)sl * SLOT + (size_t)m * 256 + pc * 16 + (lane & 3) * 4) = out;
    }
  };
  auto load_unit = [&](TbUnit& t, int i) {
    const bool live = mine && i < ng;
    const int64_t u = live ? (int64_t)rb * a.G + g0 + i : 0;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(uniform_ptr(a.codes) + u * 192, live ? 768u : 0u);
    t.z = __builtin_amdgcn_raw_buffer_load_b96(rc, (uint32_t)lane * 12u, 0, 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(uniform_ptr(a.scales) + u * 16, live ? 32u : 0u);
    t.s = __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(lane & 14) * 2u, 0, 0);
  };
  TbUnit c[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) {
    load_x(i, xr[i]);
    load_unit(c[i], i);
    __builtin_amdgcn_sched_barrier(0);
  }
  tb_vm_wait<2 + (PD - 1) * (XRD + 2)>();  // step 0's x
  put_x(xr[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  const char* cbl = smem;
  const int kq = lane >> 4, m16 = lane & 15;
  int xa[MT][4];  // this lane's A-fragment offsets within a slot
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 16 * mt + m16;
      xa[mt][v] = row * 256 + (((4 * kq + v) ^ (row & 15)) * 16);
    }
  f4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  int sl = 0;  // slot of the step being computed
  // one step: wait for the next step's x (and so for this step's unit, loaded
  // before it), meet the other waves (this step's fragment, written one step
  // ago by each wave, is then whole), compute the unit, rotate the next step's
  // x into its slot, then issue the x and code loads PD steps ahead.  Every step issues
  // the same loads (past the slice through empty ranges), so the wait count is
  // the same in every step.
  // (li = i % PD, a constant once the loop below is unrolled: the register sets
  // are indexed by it)
  auto step = [&](TbUnit& cu, int i, int li) {
    tb_vm_wait<2 + (PD - 2) * (XRD + 2)>();
    lds_barrier();
    if (mine && i < ng) {
      const uint32_t z2 = cu.z.x, z1 = cu.z.y, z0 = cu.z.z;
      const uint32_t nz2 = tr_from_next_row_lane(z2), nz1 = tr_from_next_row_lane(z1);
      uint32_t addr[32];
      tr_addrs(z2, z1, z0, nz2, nz1, addr);
      uint32_t pr[16];
      tr_gather(cbl, addr, pr);
      const float sc = h2f((uint16_t)((lane & 1) ? (cu.s >> 16) : (cu.s & 0xFFFFu)));
      const char* xs = xl + (size_t)sl * SLOT;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f4_t cg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int v = 0; v < 4; ++v)
          cg = mfma16(*reinterpret_cast<const h8_t*>(xs + xa[mt][v]), as_h8(pr[4 * v], pr[4 * v + 1], pr[4 * v + 2], pr[4 * v + 3]),
                      cg);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mt][e] = __builtin_fmaf(sc, cg[e], acc[mt][e]);
      }
    }
    // the next step's x into its slot, behind this step's MFMAs (every wave
    // has passed this step's barrier, so none still reads that slot)
    put_x(xr[(li + 1) % PD], sl + 1 == XB ? 0 : sl + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_x(i + PD, xr[li]);
    load_unit(cu, i + PD);
    __builtin_amdgcn_sched_barrier(0);
    sl = sl + 1 == XB ? 0 : sl + 1;
  };
  for (int u = 0; u < ng; u += PD) {
#pragma unroll
    for (int i = 0; i < PD; ++i) step(c[i], u + i, i);
  }
  if (!mine) return;
  // ---- results of this row block over the slice
  const int n = lane & 15, mq = lane >> 4;
  if (S == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mt + 4 * mq + e;
        if (m < a.M) a.y[(size_t)m * a.N + (size_t)rb * 16 + n] = f2h(acc[mt][e]);
      }
    return;
  }
  if (a.acc) {
    // few outputs: fixed-point words (see fx_word), one atomic per output and
    // slice whose returned count tells the last slice to store the result
    unsigned long long mine[MT][4], before[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mt + 4 * mq + e;
        mine[mt][e] = fx_word(acc[mt][e]);
        before[mt][e] = m < a.M ? fx_add(a.acc + (size_t)m * a.N + (size_t)rb * 16 + n, mine[mt][e]) : 0ull;
      }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mt + 4 * mq + e;
        if (m >= a.M || fx_count(before[mt][e]) != S - 1) continue;
        unsigned long long* w = a.acc + (size_t)m * a.N + (size_t)rb * 16 + n;
        a.y[(size_t)m * a.N + (size_t)rb * 16 + n] = f2h(fx_value(before[mt][e] + mine[mt][e]));
        fx_rearm(w);
      }
    return;
  }
  float* base = a.partial + ((size_t)rb * a.maxseg) * a.M * 16;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * mt + 4 * mq + e;
      if (m < a.M) st_partial(base + ((size_t)s * a.M + m) * 16 + n, acc[mt][e]);
    }
  if (tr_arrive_last(a.counters + rb, S, lane)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * mt + 4 * mq + e;
        if (m >= a.M) continue;
        const float t = sum_partials(base + (size_t)m * 16 + n, (size_t)a.M * 16, S, s, acc[mt][e]);
        a.y[(size_t)m * a.N + (size_t)rb * 16 + n] = f2h(t);
      }
  }
}

// ---------------------------------------------------------------------------
// Trellis GEMM for 2..8 rows with the K slice's x staged once: a workgroup
// of 16 waves (one row block each, as k_trellis_band) copies the codebook and
// its slice of x -- each (group, row) piece rotated by one wave in registers
// unless x comes rotated -- into LDS behind one barrier; then each wave walks
// its row block's groups on its own, with the code loads of the next TBX_PD
// groups in flight.  No workgroup barrier per group, so the waves' gathers and
// matrix-core work spread over the launch instead of meeting in lockstep.  The
// slice of x takes M * (groups) * 256 bytes beside the 128 KiB codebook: at
// most TBX_XBYTES, TBX_XPW pieces per wave.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * TbShape<1>::NW) void k_trellis_bx(TbArgs a) {
  constexpr int NW = TbShape<1>::NW, PD = TBX_PD;
  __shared__ __align__(16) char smem[TR_CB_BYTES + TBX_XBYTES];
  char* const xs = smem + TR_CB_BYTES;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = a.S, M = a.M;
  const int s = blockIdx.x % S, band = blockIdx.x / S;
  const int rb = band * NW + wave;
  const bool mine = rb < a.RB;
  const int g0 = (int)((int64_t)s * a.G / S), g1 = (int)((int64_t)(s + 1) * a.G / S), ng = g1 - g0;
  // codebook -> LDS (1 KiB per wave instruction)
  {
    const __amdgpu_buffer_rsrc_t rcb = make_rsrc(uniform_ptr(a.cb), TR_CB_BYTES);
    for (int ci = wave; ci < TR_CB_BYTES / 1024; ci += NW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rcb, (__attribute__((address_space(3))) void*)(smem + (size_t)ci * 1024),
                                               16, (uint32_t)(ci * 1024 + lane * 16), 0, 0, 0);
  }
  auto load_unit = [&](TbUnit& t, int i) {
    const bool live = mine && i < ng;
    const int64_t u = live ? (int64_t)rb * a.G + g0 + i : 0;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(uniform_ptr(a.codes) + u * 192, live ? 768u : 0u);
    t.z = __builtin_amdgcn_raw_buffer_load_b96(rc, (uint32_t)lane * 12u, 0, 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(uniform_ptr(a.scales) + u * 16, live ? 32u : 0u);
    t.s = __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(lane & 14) * 2u, 0, 0);
  };
  TbUnit c[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) load_unit(c[i], i);
  // the slice of x: piece (group i, row m) holds the group's 128 values of
  // row m, lane l holding values 2l and 2l + 1 (the pairing k_trellis_band
  // rotates), at xs + (i * M + m) * 256 with the 16-byte chunk p at position
  // p ^ (m & 15); this wave takes pieces wave, wave + 16, ...
  {
    const int np = M * ng;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(uniform_ptr(a.x), (uint32_t)M * a.K * 2u);
    uint32_t xv[TBX_XPW];
#pragma unroll
    for (int j = 0; j < TBX_XPW; ++j) {
      const int pc = wave + NW * j, i = pc / M, m = pc - i * M;
      const uint32_t voff = pc < np ? (uint32_t)(((size_t)m * a.K + (size_t)(g0 + i) * 128 + 2 * lane) * 2) : 0xFFFFFFF0u;
      xv[j] = __builtin_amdgcn_raw_buffer_load_b32(rx, voff, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < TBX_XPW; ++j) {
      const int pc = wave + NW * j, i = pc / M, m = pc - i * M;
      if (pc >= np) break;  // uniform across the wave
      uint32_t out = xv[j];
      if (a.rot) {
        float p0 = h2f((uint16_t)(out & 0xFFFFu)), p1 = h2f((uint16_t)(out >> 16));
        const float sum = p0 + p1, dif = p0 - p1;
        p0 = sum;
        p1 = dif;
        fwht_lanes(p0, p1, lane);
        const float f = 0.08838834764831845f;  // 2^-3.5
        out = (uint32_t)f2h(p0 * f) | ((uint32_t)f2h(p1 * f) << 16);
      }
      const int ch = (lane >> 2) ^ (m & 15);
      *reinterpret_cast<uint32_t*>(xs + (size_t)pc * 256 + ch * 16 + (lane & 3) * 4) = out;
    }
  }
  tb_vm_wait<0>();  // the codebook copies (and the first units) have landed
  __syncthreads();  // every wave's codebook part and x pieces are in LDS
  if (!mine) return;
  const char* cbl = smem;
  const int kq = lane >> 4, m16 = lane & 15;
  int xa[4];  // this lane's A-fragment offsets within a group's pieces (rows past M repeat row M - 1)
  {
    const int row = min(m16, M - 1);
#pragma unroll
    for (int v = 0; v < 4; ++v) xa[v] = row * 256 + (((4 * kq + v) ^ (row & 15)) * 16);
  }
  f4_t acc = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // one group: its codes (loaded PD groups ahead: every group issues the same
  // two loads, past the slice through empty ranges, so the wait count is the
  // same in every group), gathers, four MFMAs against the staged x, then the
  // loads of group i + PD into the freed register set
  auto step = [&](TbUnit& cu, int i) {
    tb_vm_wait<2 * (PD - 1)>();
    if (i < ng) {
      const uint32_t z2 = cu.z.x, z1 = cu.z.y, z0 = cu.z.z;
      const uint32_t nz2 = tr_from_next_row_lane(z2), nz1 = tr_from_next_row_lane(z1);
      uint32_t addr[32];
      tr_addrs(z2, z1, z0, nz2, nz1, addr);
      uint32_t pr[16];
      tr_gather(cbl, addr, pr);
      const float sc = h2f((uint16_t)((lane & 1) ? (cu.s >> 16) : (cu.s & 0xFFFFu)));
      const char* xg = xs + (size_t)i * M * 256;
      f4_t cg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int v = 0; v < 4; ++v)
        cg = mfma16(*reinterpret_cast<const h8_t*>(xg + xa[v]), as_h8(pr[4 * v], pr[4 * v + 1], pr[4 * v + 2], pr[4 * v + 3]), cg);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(sc, cg[e], acc[e]);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_unit(cu, i + PD);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int u = 0; u < ng; u += PD) {
#pragma unroll
    for (int i = 0; i < PD; ++i) step(c[i], u + i);
  }
  tb_vm_wait<0>();  // the loads past the slice (empty ranges) retire
  // ---- results of this row block over the slice (as k_trellis_band)
  const int n = lane & 15, mq = lane >> 4;
  if (S == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * mq + e;
      if (m < M) a.y[(size_t)m * a.N + (size_t)rb * 16 + n] = f2h(acc[e]);
    }
    return;
  }
  if (a.acc) {
    unsigned long long mw[4], before[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * mq + e;
      mw[e] = fx_word(acc[e]);
      before[e] = m < M ? fx_add(a.acc + (size_t)m * a.N + (size_t)rb * 16 + n, mw[e]) : 0ull;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * mq + e;
      if (m >= M || fx_count(before[e]) != S - 1) continue;
      unsigned long long* w = a.acc + (size_t)m * a.N + (size_t)rb * 16 + n;
      a.y[(size_t)m * a.N + (size_t)rb * 16 + n] = f2h(fx_value(before[e] + mw[e]));
      fx_rearm(w);
    }
    return;
  }
  float* base = a.partial + ((size_t)rb * a.maxseg) * M * 16;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = 4 * mq + e;
    if (m < M) st_partial(base + ((size_t)s * M + m) * 16 + n, acc[e]);
  }
  if (tr_arrive_last(a.counters + rb, S, lane)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * mq + e;
      if (m >= M) continue;
      const float t = sum_partials(base + (size_t)m * 16 + n, (size_t)M * 16, S, s, acc[e]);
      a.y[(size_t)m * a.N + (size_t)rb * 16 + n] = f2h(t);
    }
  }
}

// ---------------------------------------------------------------------------
// checking kernel: states (and cb[state] * s in fp32) of every weight, through
// the same decode as the run kernels.  One wave per unit.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_debug_trellis(const uint32_t* __restrict__ codes,
                                                       const uint16_t* __restrict__ scales,
                                                       const uint16_t* __restrict__ cb, int K, int G, int64_t U,
                                                       uint16_t* states, float* w) {
  const int64_t u = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (u >= U) return;  // whole waves leave together (blockDim is a multiple of 64)
  const int lane = threadIdx.x & 63;
  const int rb = (int)(u / G), g = (int)(u % G);
  const uint32_t* zp = codes + (u * 64 + lane) * 3;
  const uint32_t z2 = zp[0], z1 = zp[1], z0 = zp[2];
  const uint32_t nz2 = tr_from_next_row_lane(z2), nz1 = tr_from_next_row_lane(z1);
  uint32_t addr[32];
  tr_addrs(z2, z1, z0, nz2, nz1, addr);
  const int n = rb * 16 + (lane & 15);
  const int kq = lane >> 4;
  const float s = h2f(scales[u * 16 + (lane & 15)]);
  for (int j = 0; j < 32; ++j) {
    const size_t at = (size_t)n * K + (size_t)g * 128 + 32 * kq + j;
    const uint32_t st = addr[j] >> 1;
    if (states) states[at] = (uint16_t)st;
    if (w) w[at] = h2f(cb[st]) * s;  // exact: fp16 x fp16 fits fp32
  }
}

}  // namespace qg
