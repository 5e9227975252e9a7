// qg_args.h -- kernel argument blocks, compile-time shapes and LDS sizes of the
// run kernels, shared by the kernels and by the host code that plans and
// launches them (no kernels here, so every translation unit may include it).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

constexpr int MAX_SEG = 3;

struct SegDev {
  const uint32_t* codes;   // device layout, [tiles][G4][bits][64][4] words
  const uint16_t* scales;  // fp16, [tiles][G4][16][4]; sq: [tiles][G4][4][16][4]
  int bits;                // 2, 3 or 4
  int tiles;               // 16-column tiles in this segment
  int tile0;               // index of the first tile in the handle's padded column space
  int sq;                  // scale group 64 or 32: one scale per lane quarter (32 weights) and
                           // group of 128 instead of one per column and group (qg_common.h)
  int mx;                  // MXFP4: 4-bit fields are E2M1 elements; the per-quarter scale
                           // entries hold E8M0 bytes (own exponent | group maximum << 8)
};

struct WSet {
  SegDev seg[MAX_SEG];
  int nseg;
  const int32_t* col_map;  // [16 * total tiles]: original column of each padded column, or -1
};

struct GvArgs {
  WSet w[2];               // w[1]: the up matrix of the fused gate/up pass
  const void* x;           // [K] fp16, or fp32 (the fused MLP's intermediate)
  void* y;                 // [N] fp16, or fp32 (yf32: the fused MLP's intermediate h)
  float* partial;          // [2][S][NP] fp32 when handing over through partials
  int* counters;           // one arrival counter per tile (all zero between runs)
  int K, G, G4, NP;
  int S;                   // K slices across workgroups
  int pair;                // the fused gate/up pass (w[0], w[1]), one matrix per workgroup
  unsigned long long* xw;  // per padded column word, zero between runs: the pair pass's exchange
                           // word (one K slice) or, with fx, the K slices' fixed-point sum
  int fx;                  // one matrix, K slices: meet in fixed-point words (else partials)
  int yf32;                // y holds fp32
  int ts_prefix[MAX_SEG + 1];  // prefix sums of tiles per segment
};

// several independent M = 1 products in one launch (qgemv_run_batch)
constexpr int GV_MAX_TASKS = 8;
struct GvBatch {
  GvArgs task[GV_MAX_TASKS];
  int wg0[GV_MAX_TASKS + 1];   // first workgroup of each task; wg0[n] = the grid
  int n;
};

// LDS layout (bytes): per wave its staged activations NQ*1024 and quarter
// sums NQ*64 | cross-wave partials NW*16*4 | flag 16
constexpr int M1_WAVE_LDS = 1088;  // per quad of a wave
__host__ __device__ constexpr size_t m1_lds_bytes(int NQ, int NW) {
  return (size_t)NW * NQ * M1_WAVE_LDS + (size_t)NW * 64 + 16;
}

constexpr int SK_UPW = 8;    // at most this many quads per wave
constexpr int SK_PD = 3;     // units whose loads are in flight while one is computed

struct SkArgs {
  WSet w[2];                   // w[1]: up matrix of the fused gate/up pass
  const void* x;               // [K] fp16, or fp32 (the fused MLP's intermediate)
  void* y;                     // [N] fp16, or fp32 (yf32; fused pass: h = SiLU(g) * u)
  unsigned long long* acc;     // [2][16 * total_tiles] column words, zero between launches
  int K, N, G, G4, total_tiles;
  int nch;                     // waves per tile
  int runq;                    // quads of the longest run (LDS per wave: runq * 1088 bytes)
  int yf32;                    // y holds fp32
  int64_t U;                   // total_tiles * G4
  int wg_prefix[MAX_SEG + 1];  // several widths: workgroups before each width segment
};

// LDS: per wave the staged activations of its run (at most runq quads of 512
// fp16) and their quarter sums
__host__ __device__ constexpr size_t sk_lds_bytes(int NW, int runq) { return (size_t)NW * runq * 1088; }

constexpr int XS_PD = 2;    // code buffers per wave: units in flight while one is computed, plus it
constexpr int XS_LEAD = 1;  // units whose loads are issued before the x slice is waited for

struct XsArgs {
  WSet w[2];                  // w[1]: up matrix of the fused gate/up pass
  const uint16_t* x;          // [M][K] fp16
  const float* xf;            // XSC: [M][G] factor 2^-e of each (row, group) of x
  void* y;                    // [M][ldy] fp16, or fp32 (yf32: the fused pass's h)
  int yf32;
  float* partial;             // [ND][S][M][NP] fp32 (S > 1, acc == NULL)
  int* counters;              // one per tile group, zero between launches
  unsigned long long* acc;    // [ND][M][NP] fixed-point words (S > 1), zero between launches; or NULL
  int M, K, G, G4, ldy, NP, S;
  int GPW;                    // tile groups per workgroup
  int wg_prefix[MAX_SEG + 1]; // workgroups (per slice) before each width segment
  int tg_prefix[MAX_SEG + 1]; // tile groups before each width segment
};

// LDS: the x slice as [row m][group] 256-byte rows of 128 fp16, row m at
// m * NQ KiB (a compile-time stride, so every A-fragment read is one base
// register plus an immediate offset); the 16-byte chunk p of a row sits at
// position p ^ (m & 15), so the 16 rows an A fragment reads fall on distinct
// banks.  Then the group sums as [group][16 * MT] floats, (XSC) the factors in
// the same layout, then the output column of each padded column of the
// workgroup's run (read there, not from memory, so storing a result never
// waits behind code loads).
__host__ __device__ constexpr size_t xs_x_bytes(int M, int NQ) { return (size_t)M * NQ * 1024; }
__host__ __device__ constexpr size_t xs_sum_bytes(int MT, int NQ) { return (size_t)NQ * 4 * 16 * MT * 4; }
__host__ __device__ constexpr size_t xs_col_bytes(int GPW, int T) { return ((size_t)GPW * T * 64 + 1023) / 1024 * 1024; }
__host__ __device__ constexpr size_t xs_lds_bytes(int M, int MT, int NQ, int GPW, int T, bool xsc) {
  return xs_x_bytes(M, NQ) + (xsc ? 2 : 1) * xs_sum_bytes(MT, NQ) + xs_col_bytes(GPW, T);
}

constexpr int TR_CB_BYTES = 65536 * 2;   // codebook in LDS

struct TrArgs {
  const uint32_t* codes;   // [U][64][3]
  const uint16_t* scales;  // [U][16]
  const uint16_t* cb;      // [65536] fp16
  const uint16_t* x;       // [K] fp16, rotated (XL: unrotated; the kernel rotates it)
  uint16_t* y;             // [N] fp16
  float* partial;          // [RB][maxseg][16]
  int* counters;           // [RB], zero between launches
  unsigned long long* acc; // [N] fixed-point output words (zero between launches), or NULL: partials
  int K, N, G, RB, maxseg, W;
  int64_t U;
};

// XL: the rotated x sits in LDS beside the codebook (the kernel rotates it
// itself), so a unit loads only its codes and scale
constexpr int TR_XL_BYTES = 32768;           // rotated x in LDS: K <= 16384
constexpr int TR_XL_GMAX = 8;                // groups per wave to rotate (G <= 128, 16 waves)
constexpr int TR_NW = 16;                    // waves per workgroup (four per SIMD)
constexpr int TR_PD = 2;                     // units whose loads are in flight while one is computed

template <int MT> struct TbShape {
  static constexpr int NW = MT == 2 ? 8 : 16;  // waves = row blocks per workgroup
  static constexpr int PD = MT == 2 ? 2 : 3;   // groups whose copies and code loads are in flight
  static constexpr int XB = PD + 1;            // x slots
  static constexpr int MR = 16 * MT;           // rows of an x slot
  static constexpr int XRD = MR / NW;          // 256-byte row copies per wave per group
  static constexpr int SLOT = MR * 256;        // bytes per x slot
};

// trellis GEMM for 2..8 rows with the K slice's x in LDS beside the codebook
constexpr int TBX_MAXM = 8;                           // rows
constexpr int TBX_XBYTES = 160 * 1024 - TR_CB_BYTES;  // LDS for the slice of x: 128 (group, row) pieces
constexpr int TBX_XPW = TBX_XBYTES / 256 / 16;        // pieces per wave (16 waves)
constexpr int TBX_PD = 3;                             // groups whose code loads are in flight

struct TbArgs {
  const uint32_t* codes;   // [U][64][3]
  const uint16_t* scales;  // [U][16]
  const uint16_t* cb;      // [65536] fp16
  const uint16_t* x;       // [M][K] fp16: rotated already (rot 0) or as given (rot 1)
  uint16_t* y;             // [M][N] fp16
  float* partial;          // [RB][maxseg][M][16] (S > 1, acc NULL)
  int* counters;           // [RB], zero between launches
  unsigned long long* acc; // [M][N] fixed-point output words (S > 1), zero between launches; or NULL
  int M, K, N, G, RB, maxseg, S;
  int rot;                 // rotate each group of x in the kernel (Walsh-Hadamard, 2^-3.5)
};

}  // namespace qg
