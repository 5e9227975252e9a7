// k_m1q.hip -- launcher of the per-group M = 1 GEMV (qg_gemv.h): one
// instantiation per (quads per wave, code width, fp32 x).
#include "qg_gemv.h"
#include "qg_launch.h"

namespace qg {
namespace {

template <int NQ, int BF, bool XF>
void lq(const GvArgs& a, int NW, size_t lds, unsigned grid, hipStream_t st) {
  k_gemv_q<NQ, BF, XF><<<grid, NW * 64, lds, st>>>(a);
}

// bf: the single code width, 0 for several, 5 for MXFP4, 6 for MXFP6 (fp16 x only)
template <int NQ, bool XF>
void lq_b(const GvArgs& a, int NW, size_t lds, unsigned grid, int bf, hipStream_t st) {
  switch (bf) {
    case 5:
      if constexpr (!XF) lq<NQ, 5, XF>(a, NW, lds, grid, st);
      break;
    case 6:
      if constexpr (!XF) lq<NQ, 6, XF>(a, NW, lds, grid, st);
      break;
    case 2: lq<NQ, 2, XF>(a, NW, lds, grid, st); break;
    case 3: lq<NQ, 3, XF>(a, NW, lds, grid, st); break;
    case 4: lq<NQ, 4, XF>(a, NW, lds, grid, st); break;
    default: lq<NQ, 0, XF>(a, NW, lds, grid, st); break;
  }
}

template <int NQ>
void lq_x(const GvArgs& a, int NW, size_t lds, unsigned grid, int bf, bool xf, hipStream_t st) {
  if (xf) lq_b<NQ, true>(a, NW, lds, grid, bf, st);
  else lq_b<NQ, false>(a, NW, lds, grid, bf, st);
}

template <int NQ, int BF>
void lb(const GvBatch& b, int NW, size_t lds, unsigned grid, hipStream_t st) {
  k_gemv_batch<NQ, BF><<<grid, NW * 64, lds, st>>>(b);
}

template <int NQ>
void lb_b(const GvBatch& b, int NW, size_t lds, unsigned grid, int bf, hipStream_t st) {
  switch (bf) {
    case 2: lb<NQ, 2>(b, NW, lds, grid, st); break;
    case 3: lb<NQ, 3>(b, NW, lds, grid, st); break;
    case 4: lb<NQ, 4>(b, NW, lds, grid, st); break;
    default: lb<NQ, 0>(b, NW, lds, grid, st); break;
  }
}

}  // namespace

hipError_t launch_gemv_batch(const GvBatch& b, int NQ, int NW, size_t lds, unsigned grid, int bf, hipStream_t st) {
  switch (NQ) {
    case 2: lb_b<2>(b, NW, lds, grid, bf, st); break;
    case 3: lb_b<3>(b, NW, lds, grid, bf, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_q(const GvArgs& a, int NQ, int NW, size_t lds, unsigned grid, int bf, bool xf, hipStream_t st) {
  switch (NQ) {
    case 1: lq_x<1>(a, NW, lds, grid, bf, xf, st); break;
    case 2: lq_x<2>(a, NW, lds, grid, bf, xf, st); break;
    case 3: lq_x<3>(a, NW, lds, grid, bf, xf, st); break;
    case 4: lq_x<4>(a, NW, lds, grid, bf, xf, st); break;
    case 5: lq_x<5>(a, NW, lds, grid, bf, xf, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qg
