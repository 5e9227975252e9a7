/*
 * qgemv.h -- C ABI of the packed low-bit weight-only GEMV / verify GEMM library
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  y[m][n] = sum_k x[m][k] * w[n][k] for fp16 activations x
 * (M rows: 1 for a decode step, up to 32 for a speculative-decode verify batch)
 * and weights w stored as packed low-bit codes.  This is the decode GEMV of
 * "OrcaSAQ2-27B on AMD Radeon -- ROCm runtime" (intro: ~3.2 bits/weight EXL3
 * trellis weights, GEMM kernels on vector ALUs) and the batched verify of
 * "Qwen3.8-27B on a 16 GB RX 9070 XT" (section "What we added on top of
 * upstream": verifying 8 drafted tokens, verify batches up to 32 rows, a fused
 * MLP path, bit-identical output).  The weight formats:
 *
 *   QG_FMT_UNIFORM  b-bit unsigned codes c (b = 2, 3 or 4, optionally chosen
 *                   per output column), one fp16 scale s per 128 consecutive k
 *                   of a row: w = (c - (2^b - 1)/2) * s.  Block family: the
 *                   Q-series rows of the format table in "The Rock8"
 *                   (128-element blocks, fp16 per-block scale).
 *   QG_FMT_TRELLIS3 bitshift trellis, exactly 3 bits/weight: per 16x16 tile a
 *                   768-bit stream; weight i of the tile takes the cyclic
 *                   16-bit window that starts at stream bit 3*i as an index
 *                   into a 65536-entry fp16 codebook; w = codebook[state] * s.
 *                   The activations are rotated by the normalised 128-point
 *                   Walsh-Hadamard transform per 128-group before the product
 *                   (trellis family: EXL3 of the OrcaSAQ2 page).
 *
 * Canonical (input) layouts, all little-endian:
 *   x        fp16 [M][K] row-major, y fp16 [M][N] row-major.
 *   W        logical [N][K] (out x in features), y = x * W^T.
 *   codes    UNIFORM: per row n, per group g, 4*b uint32 words; in-group code
 *            j occupies stream bits [b*j, b*j+b), stream bit t = bit (t mod 32)
 *            of word t/32.  Rows are concatenated in order (with per-column
 *            widths each row has its own b).
 *            TRELLIS3: uint16 [N/16][K/16][48]; stream bit t of a tile = bit
 *            (15 - t mod 16) of word t/16; weight i = 16*r + c of tile
 *            (tn, tk) is w[16*tn + r][16*tk + c].
 *   scales   fp16 bits [N][K/128] row-major.
 *   codebook fp16 bits [65536] (TRELLIS3 only).
 *
 * Ownership.  qgemv_create copies and re-lays-out codes, scales and codebook
 * into device memory owned by the handle, synchronises the given stream and
 * returns; the caller may free its inputs afterwards.  qgemv_destroy frees
 * everything the handle owns.  qgemv_run / qmlp_run allocate nothing: they
 * enqueue kernels on the given stream and return; x, y and out stay
 * caller-owned and must stay valid until that stream work completes.
 *
 * Concurrency.  A handle is immutable after create, but it owns its split-K
 * workspace (fp32 partials, arrival counters and fixed-point column words,
 * which every run leaves re-armed) and one MLP staging buffer, so runs that
 * use the same handle must be ordered (same stream, or caller-ordered).
 * Different handles are independent.  A kernel that faulted may leave the
 * workspace un-armed: destroy and re-create the handle after a device error.
 *
 * Determinism.  Every reduction either runs in a fixed order or adds exact
 * fixed-point integers (whose sum does not depend on the order of arrival);
 * no floating-point atomics are used: for the same handle and the same
 * inputs, y is bit-identical across calls, streams and processes.
 *
 * Errors.  Every entry point returns a qg_status; on failure a message is
 * available from qg_last_error() (thread-local, valid until the next call on
 * that thread).  The library never aborts, exits or prints.  Arguments are
 * checked before any device work: a failed check leaves nothing enqueued.
 *
 * Streams are passed as void* and are hipStream_t values (NULL = the default
 * stream).  Device pointers are device (HBM) addresses; "host" marks host
 * memory.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qg_plan* qg_handle;

typedef enum {
  QG_OK = 0,
  QG_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misalignment, mismatched handles      */
  QG_ERR_UNSUPPORTED = -2,  /* no gfx950 device, or a format/size the library does not handle  */
  QG_ERR_DEVICE = -3,       /* a HIP call or kernel launch failed                                */
  QG_ERR_OOM = -4           /* device allocation failed                                          */
} qg_status;

typedef enum { QG_FMT_UNIFORM = 0, QG_FMT_TRELLIS3 = 1 } qg_format;

enum {
  QG_FLAG_X_PREROTATED = 1u << 0 /* TRELLIS3: x already rotated, skip the Walsh-Hadamard step */
};

enum { QG_GROUP = 128, QG_MAX_M = 32 };

typedef struct {
  int32_t K;                /* in-features; multiple of 128                                   */
  int32_t N;                /* out-features; multiple of 16                                   */
  int32_t group_size;       /* must be 128                                                    */
  int32_t format;           /* qg_format                                                      */
  int32_t bits;             /* UNIFORM: 2, 3 or 4 for every column, or 0 = per-column widths  */
  const uint8_t* col_bits;  /* host, N entries in {2,3,4}; read iff format UNIFORM and bits 0 */
  const void* codes;        /* device, canonical packed layout above; 16-byte aligned          */
  const uint16_t* scales;   /* device, fp16 bits [N][K/128]; 16-byte aligned                   */
  const uint16_t* codebook; /* device, fp16 bits [65536]; TRELLIS3 only                        */
  uint32_t flags;           /* QG_FLAG_*                                                       */
} qg_weight_desc;

/* Validate the descriptor, check the current device is gfx950, re-lay-out the
 * weights into handle-owned device memory and size the workspace for runs of
 * up to max_M rows (1 <= max_M <= 32).  Synchronises `stream` before it
 * returns.  On failure *out is set to NULL. */
qg_status qgemv_create(qg_handle* out, const qg_weight_desc* desc, int32_t max_M, void* stream);

/* y[M][N] = x[M][K] * W^T (TRELLIS3: rotate(x) * W^T unless pre-rotated).
 * x, y: device, fp16, 16-byte aligned; 1 <= M <= max_M.  Enqueues on stream. */
qg_status qgemv_run(qg_handle h, const uint16_t* x, int32_t M, uint16_t* y, void* stream);

/* Fused MLP: out = down( SiLU(gate(x)) * up(x) ), SiLU(z) = z / (1 + e^-z).
 * gate and up: same K (= hidden), same N (= intermediate), same per-column
 * widths; down: K = intermediate.  x: device fp16 [M][hidden]; out: device
 * fp16 [M][down N].  The intermediate h = SiLU(g)*u is kept as fp16 in the
 * gate handle's staging buffer.  UNIFORM handles only. */
qg_status qmlp_run(qg_handle gate, qg_handle up, qg_handle down, const uint16_t* x, int32_t M,
                   uint16_t* out, void* stream);

/* Free everything the handle owns (NULL is accepted). */
qg_status qgemv_destroy(qg_handle h);

/* Message of the last failure on this thread ("" if none). */
const char* qg_last_error(void);

/* Bytes the weights occupy in the canonical format (codes + scales; a
 * trellis codebook is not counted).  Host out-pointer. */
qg_status qgemv_weight_bytes(qg_handle h, int64_t* bytes);

/* Override the launch geometry used for runs with M rows in the class of
 * `M` (M = 1, or any M in 2..16, or any M in 17..32); for sweeps of launch
 * shapes.  Values <= 0 restore the built-in choice.  Meaning per kernel:
 *   M = 1, per-tile-run GEMV (the default below 256 tiles): `tiles` = waves
 *     per 16-column tile (each takes a run of at most
 *     8 quads of 512 k), `waves` = waves per workgroup (1..8), `splits` unused.
 *   M = 1, per-group GEMV: `tiles` 16-column tiles per workgroup (1), `waves`
 *     waves per workgroup splitting K (1..16), `splits` K slices across
 *     workgroups (1..16; summed in fixed-point words, exact in any order).
 *   M > 1: `tiles` tiles per wave (1, 2 or 4), `waves` waves per workgroup
 *     (1, 2, 4 or 8), `splits` K slices across workgroups (1..16).
 * Uniform-code handles only; a shape the compiled kernels cannot take fails
 * with QG_ERR_INVALID_ARG when it is run. */
qg_status qgemv_set_launch(qg_handle h, int32_t M, int32_t tiles, int32_t waves, int32_t splits);

/* ---- checking entry points (same device decode functions as the run kernels) ---- */

/* codes: device int32 [N][K], the unpacked code of every weight (UNIFORM). */
qg_status qgemv_debug_unpack(qg_handle h, int32_t* codes, void* stream);

/* w: device fp32 [N][K], exact dequantised weight (c - o_b) * s (UNIFORM) or
 * codebook[state] * s (TRELLIS3).  q16 (UNIFORM, may be NULL): device fp16
 * bits [N][K] of c - o_b. */
qg_status qgemv_debug_dequant(qg_handle h, float* w, uint16_t* q16, void* stream);

/* states: device uint16 [N][K], the trellis state of every weight (TRELLIS3). */
qg_status qgemv_debug_trellis(qg_handle h, uint16_t* states, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
