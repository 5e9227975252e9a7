// qg_common.h -- pieces every run kernel of the library shares: the segment
// descriptors of a handle's device layout, workgroup barriers and cross-lane
// moves, and the two ways K slices (or row blocks) meet: fp32 partials summed in
// a fixed order, and order-independent fixed-point words.  Layout and decode:
// qg_decode.h.
//
// Arithmetic of the uniform format (b-bit codes, offset o = (2^b - 1)/2, group
// g of 128 k):  y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] * (c[n][k] - o).
//
// Memory-instruction discipline (measured on gfx950): every 64-lane load costs
// address-pipeline time even when it moves no data, so the run kernels issue
// only full-width 16-byte-per-lane loads, never a load for data they do not
// use, and issue all of them unconditionally so the compiler can count them
// and wait for exactly the one it needs next.
#pragma once
#include "qg_args.h"
#include "qg_decode.h"

namespace qg {


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

__device__ __forceinline__ int dpp_xor1_i(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_xor2_i(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ float dpp_xor1(float v) { return __builtin_bit_cast(float, dpp_xor1_i(__builtin_bit_cast(int, v))); }
__device__ __forceinline__ float dpp_xor2(float v) { return __builtin_bit_cast(float, dpp_xor2_i(__builtin_bit_cast(int, v))); }
// value of lane (l & ~15) | ((l - N) & 15): rotation right within each row of 16 lanes
template <int N> __device__ __forceinline__ float dpp_row_ror(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF, false));
}

// an output element: fp16 (RNE), or fp32 where y is the fused MLP's intermediate
__device__ __forceinline__ void store_y(void* y, size_t i, float v, int yf32) {
  if (yf32) reinterpret_cast<float*>(y)[i] = v;
  else reinterpret_cast<uint16_t*>(y)[i] = f2h(v);
}

// Scales of a quad (4 groups of 128) in the device layout.  Group size 128:
// [16 columns][4 groups], 128 B, one scale per column and group.  Group size
// 64 or 32 ("sq"): [4 lane quarters][16 columns][4 groups], 512 B: lane l
// holds weights 32 (l >> 4) .. + 31 of each group of its column, which lie in
// one scale group (of 64: groups 2g + (l >> 5); of 32: 4g + (l >> 4)), so each
// lane still meets one scale per group of 128 and loads its 4 with one 8-byte
// load.
__host__ __device__ constexpr uint32_t scale_quad_halves(int sq) { return sq ? 256u : 64u; }
__device__ __forceinline__ uint32_t scale_lane_byte(int sq, uint32_t lane) {
  return ((sq ? (lane >> 4) << 4 : 0u) + (lane & 15u)) * 8u;
}
// scale of group g for column j, lane quarter q of tile t
__device__ __forceinline__ size_t scale_index(int t, int G4, int g, int j, int q, int sq) {
  return ((size_t)t * G4 + (g >> 2)) * scale_quad_halves(sq) + ((sq ? 16 * q : 0) + j) * 4 + (g & 3);
}

// ---------------------------------------------------------------------------
// fp32 partials: each contributor stores its partial in a fixed slot; the one
// that arrives last (device-scope counter) adds the slots in slot order and
// stores the result, then re-arms the counter.  No floating-point atomics, so
// the order of arrival never changes a bit of the output.
//
// The partials are written and read only with agent-scope atomic accesses,
// which go to the device coherence point past the per-XCD L2 caches by
// themselves: so no cache write-back or invalidation (a device-wide fence,
// which writes back a whole L2) is needed.  Every thread waits until its own
// partial stores have completed before the arrival is counted, and only a
// contributor that has seen every other one arrive reads the partials.
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

// Workgroup-wide arrival at a split-K counter (all threads call it): true in
// the workgroup whose arrival completes the count of S.
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
// Fixed-point accumulation words, the order-independent hand-over: each
// contributor adds one 64-bit word with one integer atomic.  Integer addition
// is exact and commutative, so the total does not depend on the order of
// arrival (bit-identical results).  Word layout, as a signed 64-bit integer:
//   bits  0..5   arrival count (at most 63 contributors per word)
//   bits  6..11  count of non-finite contributions (NaN or +-inf partials)
//   bits 12..63  round(v * 2^28) for a finite v clamped to +-2^17
// A finite contribution adds (round(v * 2^28) << 12) + 1, a non-finite one
// (1 << 6) + 1.  The low 12 bits never carry into the value field (at most
// 63 + 63 * 64 < 4096), and 63 values of magnitude <= 2^45 sum to less than
// 2^51, so the field never overflows.  The clamp is past the fp16 output range
// (65504): a partial that large still gives +-inf unless slices cancel it.
// A total with any non-finite contribution reads as NaN.
// ---------------------------------------------------------------------------
constexpr int FX_FRAC = 28;  // fraction bits

__device__ __forceinline__ unsigned long long fx_word(float v) {
  if (!(fabsf(v) <= 3.402823466e38f)) return (1ull << 6) + 1ull;  // NaN or +-inf
  const float vc = fminf(fmaxf(v, -131072.0f), 131072.0f);        // +-2^17
  return ((unsigned long long)__double2ll_rn((double)vc * (double)(1ll << FX_FRAC)) << 12) + 1ull;
}

__device__ __forceinline__ unsigned long long fx_add(unsigned long long* w, unsigned long long v) {
  return __hip_atomic_fetch_add(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int fx_count(unsigned long long total) { return (int)(total & 63ull); }

__device__ __forceinline__ float fx_value(unsigned long long total) {
  if ((total >> 6) & 63ull) return __builtin_nanf("");
  return (float)((double)((long long)total >> 12) * (1.0 / (double)(1ll << FX_FRAC)));
}

__device__ __forceinline__ void fx_rearm(unsigned long long* w) {
  __hip_atomic_store(w, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qg
