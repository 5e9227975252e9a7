// k_trellis.hip -- launchers of the trellis kernels (qg_trellis.h): the M = 1
// GEMV, the banded GEMM for 2..32 rows, the x rotation, the create-time
// re-layout and the checking kernel.
#include "qg_launch.h"
#include "qg_trellis.h"

namespace qg {

hipError_t launch_trellis_gemv(const TrArgs& a, bool xl, unsigned grid, hipStream_t st) {
  if (xl) k_trellis<true><<<grid, 64 * TR_NW, 0, st>>>(a);  // a.x: the unrotated x
  else k_trellis<false><<<grid, 64 * TR_NW, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_trellis_band(const TbArgs& a, int MT, unsigned grid, hipStream_t st) {
  if (MT == 2) k_trellis_band<2><<<grid, 64 * TbShape<2>::NW, 0, st>>>(a);
  else k_trellis_band<1><<<grid, 64 * TbShape<1>::NW, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_trellis_bx(const TbArgs& a, unsigned grid, hipStream_t st) {
  k_trellis_bx<<<grid, 64 * TbShape<1>::NW, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwht(const uint16_t* x, uint16_t* xr, int M, int K, hipStream_t st) {
  const int waves = M * (K / 128);
  k_fwht<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(x, xr, M, K);
  return hipGetLastError();
}

hipError_t launch_repack_trellis(const uint16_t* tiles, const uint16_t* scales, int KT, int G, int64_t units,
                                 uint32_t* dcodes, uint16_t* dscales, hipStream_t st) {
  const int64_t threads = units * 64;
  k_repack_trellis<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(tiles, scales, KT, G, units, dcodes, dscales);
  return hipGetLastError();
}

hipError_t launch_debug_trellis(const uint32_t* codes, const uint16_t* scales, const uint16_t* cb, int K, int G,
                                int64_t units, uint16_t* states, float* w, hipStream_t st) {
  const int64_t threads = units * 64;
  k_debug_trellis<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(codes, scales, cb, K, G, units, states, w);
  return hipGetLastError();
}

}  // namespace qg
