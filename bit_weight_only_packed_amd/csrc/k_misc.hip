// k_misc.hip -- launchers of the create-time, checking and measurement kernels
// (qg_misc.h) and of the fused MLP's block-exponent rounding of h.
#include <algorithm>

#include "qg_launch.h"
#include "qg_misc.h"

namespace qg {

hipError_t launch_repack_uniform(const uint32_t* canon, const int64_t* row_off, const uint16_t* scales,
                                 const int32_t* cols, int bits, int tiles, int G, int G4, int gs, uint32_t* dcodes,
                                 uint16_t* dscales, hipStream_t st) {
  const size_t nslot = (size_t)tiles * G4 * 64;
  k_repack_uniform<<<(unsigned)((nslot + 255) / 256), 256, 0, st>>>(canon, row_off, scales, cols, bits, tiles, G, G4,
                                                                   gs, dcodes, dscales);
  return hipGetLastError();
}

hipError_t launch_repack_mx_scales(const uint8_t* e8, const int32_t* cols, int tiles, int G, int G4, uint16_t* dscales,
                                   hipStream_t st) {
  const size_t nslot = (size_t)tiles * G4 * 64;
  k_repack_mx_scales<<<(unsigned)((nslot + 255) / 256), 256, 0, st>>>(e8, cols, tiles, G, G4, dscales);
  return hipGetLastError();
}

hipError_t launch_repack_mx6(const uint32_t* canon, const int32_t* cols, int tiles, int G, int G4, uint32_t* dcodes,
                             hipStream_t st) {
  const size_t nslot = (size_t)tiles * G4 * 64;
  k_repack_mx6<<<(unsigned)((nslot + 255) / 256), 256, 0, st>>>(canon, cols, tiles, G, G4, dcodes);
  return hipGetLastError();
}

hipError_t launch_debug_uniform(const SegDev& sg, const int32_t* col_map, int G, int G4, int K, int mode,
                                int32_t* codes, float* w, uint16_t* q16, hipStream_t st) {
  const int64_t n = (int64_t)sg.tiles * G * 64;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (mode == 0) k_debug_uniform<0><<<blocks, 256, 0, st>>>(sg, col_map, G, G4, K, codes, w, q16);
  else k_debug_uniform<1><<<blocks, 256, 0, st>>>(sg, col_map, G, G4, K, codes, w, q16);
  return hipGetLastError();
}

hipError_t launch_h_to_f16(const float* h, uint16_t* x16, float* xf, int M, int K, hipStream_t st) {
  const int waves = M * (K / 128);
  k_h_to_f16<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(h, x16, xf, M, K);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int cus, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  k_stream_read<<<(unsigned)(4 * cus), 512, 0, st>>>(reinterpret_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  k_fill_zero<<<(unsigned)std::min<int64_t>(1024, (n16 + 255) / 256), 256, 0, st>>>(reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace qg
