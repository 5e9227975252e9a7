// k_xs_impl.h -- launcher of the verify GEMM (qg_xs.h) for one row-tile count
// MT, included by k_xs1.hip (MT = 1, up to 16 rows) and k_xs2.hip (MT = 2, up
// to 32 rows): one instantiation per (tiles per group, fused pass, code width,
// slice length, x factors).
#pragma once
#include "qg_launch.h"
#include "qg_xs.h"

namespace qg {
namespace xsl {

constexpr int kNQs[] = {4, 5, 8};  // slice lengths (quads) compiled

template <int MT, int T, bool DUAL, int BF, int NQ, bool XSC>
void l(const XsArgs& a, int NW, size_t lds, unsigned grid, hipStream_t st) {
  k_gemm_xs<T, MT, DUAL, BF, NQ, XSC><<<grid, NW * 64, lds, st>>>(a);
}

template <int MT, int T, bool DUAL, int NQ, bool XSC>
void l_b(const XsArgs& a, int bf, int NW, size_t lds, unsigned grid, hipStream_t st) {
  switch (bf) {
    case 2: l<MT, T, DUAL, 2, NQ, XSC>(a, NW, lds, grid, st); break;
    case 3: l<MT, T, DUAL, 3, NQ, XSC>(a, NW, lds, grid, st); break;
    case 4: l<MT, T, DUAL, 4, NQ, XSC>(a, NW, lds, grid, st); break;
    default: l<MT, T, DUAL, 0, NQ, XSC>(a, NW, lds, grid, st); break;
  }
}

template <int MT, int NQ>
void l_q(const XsArgs& a, int T, bool dual, bool xsc, int bf, int NW, size_t lds, unsigned grid, hipStream_t st) {
  if (dual) l_b<MT, 1, true, NQ, false>(a, bf, NW, lds, grid, st);
  else if (T == 1) {
    if (xsc) l_b<MT, 1, false, NQ, true>(a, bf, NW, lds, grid, st);
    else l_b<MT, 1, false, NQ, false>(a, bf, NW, lds, grid, st);
  } else {
    if (xsc) l_b<MT, 2, false, NQ, true>(a, bf, NW, lds, grid, st);
    else l_b<MT, 2, false, NQ, false>(a, bf, NW, lds, grid, st);
  }
}

template <int MT>
hipError_t launch(const XsArgs& a, int T, bool dual, bool xsc, int NQ, int bf, int NW, size_t lds, unsigned grid,
                  hipStream_t st) {
  if ((dual && (xsc || T != 1)) || (T != 1 && T != 2)) return hipErrorInvalidValue;
  switch (NQ) {
    case 4: l_q<MT, 4>(a, T, dual, xsc, bf, NW, lds, grid, st); break;
    case 5: l_q<MT, 5>(a, T, dual, xsc, bf, NW, lds, grid, st); break;
    case 8: l_q<MT, 8>(a, T, dual, xsc, bf, NW, lds, grid, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MT, int T, bool DUAL, int BF, bool XSC>
hipError_t allow_one() {
  hipError_t e = hipSuccess;
  const void* f[] = {reinterpret_cast<const void*>(&k_gemm_xs<T, MT, DUAL, BF, 4, XSC>),
                     reinterpret_cast<const void*>(&k_gemm_xs<T, MT, DUAL, BF, 5, XSC>),
                     reinterpret_cast<const void*>(&k_gemm_xs<T, MT, DUAL, BF, 8, XSC>)};
  for (const void* p : f) {
    const hipError_t r = hipFuncSetAttribute(p, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
    if (r != hipSuccess) e = r;
  }
  return e;
}

template <int MT, int BF>
hipError_t allow_b() {
  hipError_t e = hipSuccess;
  const hipError_t r[] = {allow_one<MT, 1, false, BF, false>(), allow_one<MT, 2, false, BF, false>(),
                          allow_one<MT, 1, false, BF, true>(), allow_one<MT, 2, false, BF, true>(),
                          allow_one<MT, 1, true, BF, false>()};
  for (hipError_t x : r)
    if (x != hipSuccess) e = x;
  return e;
}

template <int MT>
hipError_t allow() {
  hipError_t e = hipSuccess;
  const hipError_t r[] = {allow_b<MT, 0>(), allow_b<MT, 2>(), allow_b<MT, 3>(), allow_b<MT, 4>()};
  for (hipError_t x : r)
    if (x != hipSuccess) e = x;
  return e;
}

}  // namespace xsl
}  // namespace qg
