// k_m1sk.hip -- launcher of the per-tile-run M = 1 GEMV (qg_stream.h): one
// instantiation per (code width, matrices, fp32 x); the fused gate/up pass
// reads fp16 x only.
#include "qg_launch.h"
#include "qg_stream.h"

namespace qg {
namespace {

template <int BF, int ND, bool XF>
void lsk(const SkArgs& a, int NW, size_t lds, unsigned grid, hipStream_t st) {
  k_gemv_sk<BF, ND, XF><<<grid, NW * 64, lds, st>>>(a);
}

template <int BF>
void lsk_b(const SkArgs& a, bool dual, int NW, size_t lds, unsigned grid, bool xf, hipStream_t st) {
  if (dual) lsk<BF, 2, false>(a, NW, lds, grid, st);
  else if (xf) lsk<BF, 1, true>(a, NW, lds, grid, st);
  else lsk<BF, 1, false>(a, NW, lds, grid, st);
}

template <int BF>
hipError_t allow_b() {
  hipError_t e = hipSuccess;
  const void* f[] = {reinterpret_cast<const void*>(&k_gemv_sk<BF, 1, false>),
                     reinterpret_cast<const void*>(&k_gemv_sk<BF, 1, true>),
                     reinterpret_cast<const void*>(&k_gemv_sk<BF, 2, false>)};
  for (const void* p : f) {
    const hipError_t r = hipFuncSetAttribute(p, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
    if (r != hipSuccess) e = r;
  }
  return e;
}

}  // namespace

hipError_t launch_gemv_sk(const SkArgs& a, bool dual, int NW, size_t lds, unsigned grid, int bf, bool xf,
                          hipStream_t st) {
  if (dual && xf) return hipErrorInvalidValue;
  switch (bf) {
    case 2: lsk_b<2>(a, dual, NW, lds, grid, xf, st); break;
    case 3: lsk_b<3>(a, dual, NW, lds, grid, xf, st); break;
    case 4: lsk_b<4>(a, dual, NW, lds, grid, xf, st); break;
    default: lsk_b<0>(a, dual, NW, lds, grid, xf, st); break;
  }
  return hipGetLastError();
}

hipError_t m1_allow_lds() {
  hipError_t e = hipSuccess;
  const hipError_t r[] = {allow_b<0>(), allow_b<2>(), allow_b<3>(), allow_b<4>()};
  for (hipError_t x : r)
    if (x != hipSuccess) e = x;
  return e;
}

}  // namespace qg
