// k_xs2.hip -- the verify GEMM for 17 to 32 rows (two 16-row tiles of x).
#include "k_xs_impl.h"

namespace qg {
hipError_t launch_gemm_xs2(const XsArgs& a, int T, bool dual, bool xsc, int NQ, int bf, bool sq, int NW, size_t lds,
                           unsigned grid, hipStream_t st) {
  return xsl::launch<2>(a, T, dual, xsc, NQ, bf, sq, NW, lds, grid, st);
}
hipError_t xs2_allow_lds() { return xsl::allow<2>(); }
}  // namespace qg
