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

template <int MT, int T, bool DUAL, int BF, int NQ, bool XSC, bool SQ>
void l(const XsArgs& a, int NW, size_t lds, unsigned grid, hipStream_t st) {
  k_gemm_xs<T, MT, DUAL, BF, NQ, XSC, SQ><<<grid, NW * 64, lds, st>>>(a);
}

// per-quarter scales (SQ) are compiled for the width-generic body only
template <int MT, int T, bool DUAL, int NQ, bool XSC>
void l_b(const XsArgs& a, int bf, bool sq, int NW, size_t lds, unsigned grid, hipStream_t st) {
  if (bf == 5) {  // MXFP4: one matrix, fp16 x
    if constexpr (!DUAL && !XSC) l<MT, T, DUAL, 5, NQ, XSC, false>(a, NW, lds, grid, st);
    return;
  }
  if (bf == 6) {  // MXFP6: one matrix, fp16 x
    if constexpr (!DUAL && !XSC) l<MT, T, DUAL, 6, NQ, XSC, false>(a, NW, lds, grid, st);
    return;
  }
  if (sq) {
    l<MT, T, DUAL, 0, NQ, XSC, true>(a, NW, lds, grid, st);
    return;
  }
  switch (bf) {
    case 2: l<MT, T, DUAL, 2, NQ, XSC, false>(a, NW, lds, grid, st); break;
    case 3: l<MT, T, DUAL, 3, NQ, XSC, false>(a, NW, lds, grid, st); break;
    case 4: l<MT, T, DUAL, 4, NQ, XSC, false>(a, NW, lds, grid, st); break;
    default: l<MT, T, DUAL, 0, NQ, XSC, false>(a, NW, lds, grid, st); break;
  }
}

template <int MT, int NQ>
void l_q(const XsArgs& a, int T, bool dual, bool xsc, int bf, bool sq, int NW, size_t lds, unsigned grid,
         hipStream_t st) {
  if (dual) l_b<MT, 1, true, NQ, false>(a, bf, sq, NW, lds, grid, st);
  else if (T == 1) {
    if (xsc) l_b<MT, 1, false, NQ, true>(a, bf, sq, NW, lds, grid, st);
    else l_b<MT, 1, false, NQ, false>(a, bf, sq, NW, lds, grid, st);
  } else {
    if (xsc) l_b<MT, 2, false, NQ, true>(a, bf, sq, NW, lds, grid, st);
    else l_b<MT, 2, false, NQ, false>(a, bf, sq, NW, lds, grid, st);
  }
}

template <int MT>
hipError_t launch(const XsArgs& a, int T, bool dual, bool xsc, int NQ, int bf, bool sq, int NW, size_t lds,
                  unsigned grid, hipStream_t st) {
  if ((dual && (xsc || T != 1)) || (T != 1 && T != 2)) return hipErrorInvalidValue;
  switch (NQ) {
    case 4: l_q<MT, 4>(a, T, dual, xsc, bf, sq, NW, lds, grid, st); break;
    case 5: l_q<MT, 5>(a, T, dual, xsc, bf, sq, NW, lds, grid, st); break;
    case 8: l_q<MT, 8>(a, T, dual, xsc, bf, sq, NW, lds, grid, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MT, int T, bool DUAL, int BF, bool XSC, bool SQ>
hipError_t allow_one() {
  hipError_t e = hipSuccess;
  const void* f[] = {reinterpret_cast<const void*>(&k_gemm_xs<T, MT, DUAL, BF, 4, XSC, SQ>),
                     reinterpret_cast<const void*>(&k_gemm_xs<T, MT, DUAL, BF, 5, XSC, SQ>),
                     reinterpret_cast<const void*>(&k_gemm_xs<T, MT, DUAL, BF, 8, XSC, SQ>)};
  for (const void* p : f) {
    const hipError_t r = hipFuncSetAttribute(p, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
    if (r != hipSuccess) e = r;
  }
  return e;
}

template <int MT, int BF, bool SQ>
hipError_t allow_b() {
  hipError_t e = hipSuccess;
  const hipError_t r[] = {allow_one<MT, 1, false, BF, false, SQ>(), allow_one<MT, 2, false, BF, false, SQ>(),
                          allow_one<MT, 1, false, BF, true, SQ>(), allow_one<MT, 2, false, BF, true, SQ>(),
                          allow_one<MT, 1, true, BF, false, SQ>()};
  for (hipError_t x : r)
    if (x != hipSuccess) e = x;
  return e;
}

template <int MT>
hipError_t allow() {
  hipError_t e = hipSuccess;
  const hipError_t r[] = {allow_b<MT, 0, false>(), allow_b<MT, 2, false>(), allow_b<MT, 3, false>(),
                          allow_b<MT, 4, false>(), allow_b<MT, 0, true>(), allow_one<MT, 1, false, 5, false, false>(),
                          allow_one<MT, 2, false, 5, false, false>(), allow_one<MT, 1, false, 6, false, false>(),
                          allow_one<MT, 2, false, 6, false, false>()};
  for (hipError_t x : r)
    if (x != hipSuccess) e = x;
  return e;
}

}  // namespace xsl
}  // namespace qg
