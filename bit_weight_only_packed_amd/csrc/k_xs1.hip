// k_xs1.hip -- the verify GEMM for up to 16 rows (one 16-row tile of x).
#include "k_xs_impl.h"

namespace qg {
hipError_t launch_gemm_xs1(const XsArgs& a, int T, bool dual, bool xsc, int NQ, int bf, bool sq, int NW, size_t lds,
                           unsigned grid, hipStream_t st) {
  return xsl::launch<1>(a, T, dual, xsc, NQ, bf, sq, NW, lds, grid, st);
}
hipError_t xs1_allow_lds() { return xsl::allow<1>(); }
}  // namespace qg
