// qg_launch.h -- host-side launchers of the library's kernels.  Each kernel
// family lives in a translation unit of its own (compiled in parallel); the
// planning and C ABI code (qgemv.hip) calls only these.  Every launcher returns
// the launch's hipGetLastError().
#pragma once
#include "qg_args.h"

namespace qg {

constexpr size_t kLdsMax = 163840;  // LDS per workgroup on gfx950

// M = 1 GEMVs (k_m1q.hip, k_m1sk.hip).  bf: the single code width of the
// matrix (2, 3, 4) or 0 for several widths; xf: x is fp32.
hipError_t launch_gemv_q(const GvArgs& a, int NQ, int NW, size_t lds, unsigned grid, int bf, bool xf, hipStream_t st);
hipError_t launch_gemv_batch(const GvBatch& b, int NQ, int NW, size_t lds, unsigned grid, int bf, hipStream_t st);
hipError_t launch_gemv_sk(const SkArgs& a, bool dual, int NW, size_t lds, unsigned grid, int bf, bool xf,
                          hipStream_t st);
hipError_t m1_allow_lds();  // lets the M = 1 kernels take more than 64 KiB of dynamic LDS

// verify GEMM (k_xs1.hip: MT = 1, k_xs2.hip: MT = 2)
// sq: per-lane-quarter scales (scale groups of 64 or 32)
hipError_t launch_gemm_xs1(const XsArgs& a, int T, bool dual, bool xsc, int NQ, int bf, bool sq, int NW, size_t lds,
                           unsigned grid, hipStream_t st);
hipError_t launch_gemm_xs2(const XsArgs& a, int T, bool dual, bool xsc, int NQ, int bf, bool sq, int NW, size_t lds,
                           unsigned grid, hipStream_t st);
hipError_t xs1_allow_lds();
hipError_t xs2_allow_lds();

// trellis (k_trellis.hip)
hipError_t launch_trellis_gemv(const TrArgs& a, bool xl, unsigned grid, hipStream_t st);
hipError_t launch_trellis_band(const TbArgs& a, int MT, unsigned grid, hipStream_t st);
hipError_t launch_trellis_bx(const TbArgs& a, unsigned grid, hipStream_t st);  // 2..8 rows, x slice staged once
hipError_t launch_fwht(const uint16_t* x, uint16_t* xr, int M, int K, hipStream_t st);
hipError_t launch_repack_trellis(const uint16_t* tiles, const uint16_t* scales, int KT, int G, int64_t units,
                                 uint32_t* dcodes, uint16_t* dscales, hipStream_t st);
hipError_t launch_debug_trellis(const uint32_t* codes, const uint16_t* scales, const uint16_t* cb, int K, int G,
                                int64_t units, uint16_t* states, float* w, hipStream_t st);

// create-time, checking and measurement kernels (k_misc.hip)
hipError_t launch_repack_uniform(const uint32_t* canon, const int64_t* row_off, const uint16_t* scales,
                                 const int32_t* cols, int bits, int tiles, int G, int G4, int gs, uint32_t* dcodes,
                                 uint16_t* dscales, hipStream_t st);
// MXFP4 exponent bytes [N][K/32] -> the per-quarter scale entries (own | group max << 8)
// MXFP6 codes: canonical 6-bit stream -> the two-plane quad layout
hipError_t launch_repack_mx6(const uint32_t* canon, const int32_t* cols, int tiles, int G, int G4, uint32_t* dcodes,
                             hipStream_t st);
hipError_t launch_repack_mx_scales(const uint8_t* e8, const int32_t* cols, int tiles, int G, int G4, uint16_t* dscales,
                                   hipStream_t st);
// mode 0: the GEMV class decode; mode 1: the verify GEMM's operand decode
hipError_t launch_debug_uniform(const SegDev& sg, const int32_t* col_map, int G, int G4, int K, int mode,
                                int32_t* codes, float* w, uint16_t* q16, hipStream_t st);
hipError_t launch_h_to_f16(const float* h, uint16_t* x16, float* xf, int M, int K, hipStream_t st);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int cus, hipStream_t st);
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t st);  // bytes: a multiple of 16

// prefill route (k_prefill.hip): fp16 weights of output columns [n0, n1) from
// tiles [tl0, tl0 + ntl) of a segment into out [n - n0][K]; and the fp16 GEMM
// D (column-major rows x M, ldc) = W x^T through hipBLASLt (0, or *err set)
hipError_t launch_dequant_f16(const SegDev& sg, const int32_t* col_map, int G, int G4, int K, int tl0, int ntl, int n0,
                              int n1, uint16_t* out, hipStream_t st);
int gemm_f16_wxt(int dev, const uint16_t* w, int rows, const uint16_t* x, int M, int K, uint16_t* d, int ldc,
                 void* ws, size_t ws_bytes, hipStream_t st, const char** err);

}  // namespace qg
