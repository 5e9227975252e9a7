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
 *                   (trellis family: EXL3 of the OrcaSAQ2 page, intro).
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
 * everything the handle owns.  The run entry points allocate nothing: they
 * enqueue kernels on the given stream and return; x, y and out stay
 * caller-owned and must stay valid until that stream work completes.
 *
 * Handles are immutable after create: every launch choice (including the
 * optional overrides and pins of the descriptor) is fixed there, and the
 * library reads no environment variable on a run.  A handle owns its split-K
 * workspace (fp32 partials, arrival counters and fixed-point column words,
 * which every run leaves re-armed) and the fused MLP's intermediate buffers, so
 * runs that use the same handle must be ordered (same stream, or
 * caller-ordered).  Different handles are independent.  A kernel that faulted
 * may leave the workspace un-armed: destroy and re-create the handle after a
 * device error.
 *
 * Determinism ("Outputs are bit-exact repeatable", results paragraph of the
 * OrcaSAQ2 page).  Every reduction either runs in a fixed order or adds exact
 * fixed-point integers (whose sum does not depend on the order of arrival);
 * no floating-point atomics are used: for the same handle and the same
 * inputs, y is bit-identical across calls, streams and processes.
 *
 * Non-finite inputs.  A NaN or infinite activation, scale or partial sum makes
 * the outputs it reaches NaN (or +-inf where a single fp32 chain carries it).
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

/* QG_FMT_MXFP4 ("The Rock8", format table, MXFP4 row: OCP microscaling, E2M1
 * elements -- sign, 2 exponent bits with bias 1, 1 mantissa bit -- nibble-
 * packed, one UE8M0 scale byte 2^(e - 127) per 32 elements along K; 255 is
 * NaN): codes in the 4-bit canonical layout below (element j of a row at bits
 * [4j, 4j + 4) of its stream), `scales` points at uint8 exponent bytes
 * [N][K/32], group_size 32, bits 0 or 4.  The verify GEMM (2..32 rows) runs
 * each 128-group at its largest exponent: the other 32-blocks' elements are
 * exact while within 2^9 of it and are rounded once to fp16 beyond that. */
/* QG_FMT_MXFP6 ("The Rock8", format table, MXFP6 row: OCP microscaling, E3M2
 * elements -- sign, 3 exponent bits with bias 3, 2 mantissa bits, no inf or
 * NaN -- four per three bytes, one UE8M0 scale byte per 32 elements along K):
 * codes in the 6-bit canonical layout below (element j of a row at bits
 * [6j, 6j + 6) of its stream, 24 words per row and group of 128), `scales`
 * points at uint8 exponent bytes [N][K/32], group_size 32, bits 0 or 6.  The
 * verify GEMM runs each 128-group at its largest exponent: the other
 * 32-blocks' elements are exact while within 2^23 of it and are rounded once to
 * fp16 beyond that.  The fused MLP and the one-launch batch take uniform codes
 * only (MX handles in qgemv_run_batch run one launch per entry). */
typedef enum { QG_FMT_UNIFORM = 0, QG_FMT_TRELLIS3 = 1, QG_FMT_MXFP4 = 2, QG_FMT_MXFP6 = 3 } qg_format;

enum {
  QG_FLAG_X_PREROTATED = 1u << 0, /* TRELLIS3: x already rotated, skip the Walsh-Hadamard step */
  /* UNIFORM only: batch-invariant rows.  Row m of a run (or qmlp_run) of M
   * rows is bit-identical to a run of that row alone, for every M in
   * [1, max_M]: every row count takes the verify GEMM with one launch plan
   * (K slices, tile grouping, hand-over) fixed at create from max_M, so no
   * row's arithmetic depends on how many rows ride along.  Speculative
   * verification then accepts exactly the tokens that one-row decoding would
   * produce ("Qwen3.8-27B on a 16 GB RX 9070 XT", "What we added on top of
   * upstream": verify batches of up to 32 rows on the fast path, with the
   * output of plain decoding).  Costs speed at M = 1 (the verify GEMM
   * instead of the GEMV); qgemv_run_batch runs such handles entry by entry.
   * Other formats: QG_ERR_UNSUPPORTED at create. */
  QG_FLAG_BATCH_INVARIANT = 1u << 1
};

/* Pins (qg_weight_desc.pins): force a kernel or hand-over that the built-in
 * choice takes only for other shapes.  For tests that cover every variant and
 * for launch sweeps; 0 keeps the built-in (measured) choice. */
enum {
  QG_PIN_M1_PERGROUP = 1u << 0, /* UNIFORM, M = 1: the per-group GEMV (default from 256 tiles up)    */
  QG_PIN_M1_RUNS = 1u << 1,     /* UNIFORM, M = 1: the per-tile-run GEMV (default below 256 tiles)  */
  QG_PIN_PARTIALS = 1u << 2,    /* K slices / trellis row blocks meet through fp32 partials summed
                                   in slice order (default: fixed-point words where they fit)       */
  QG_PIN_WORDS = 1u << 3,       /* UNIFORM, M >= 2: K slices meet through fixed-point words whenever
                                   at most 63 slices meet                                            */
  QG_PIN_XS_T1 = 1u << 4,       /* UNIFORM, M >= 2: one 16-column tile per tile group               */
  QG_PIN_XS_T2 = 1u << 5,       /* UNIFORM, M >= 2: two tiles per tile group                        */
  QG_PIN_TRELLIS_ROT_LAUNCH = 1u << 6, /* TRELLIS3, M = 1: rotate x in a launch of its own           */
  QG_PIN_TRELLIS_BAND = 1u << 7 /* TRELLIS3, 2..8 rows: the band kernel that stages x group by group
                                   behind a workgroup barrier (default: the K slice's x staged once,
                                   where it fits in LDS)                                            */
};

enum { QG_GROUP = 128, QG_MAX_M = 32 };

/* Optional launch geometry of one row class; 0 in a field keeps the built-in
 * choice.  Meaning (UNIFORM handles):
 *   M = 1, per-group GEMV: `waves` waves per workgroup splitting the K slice
 *     (1..16), `splits` K slices across workgroups; `tiles` unused.
 *   M = 1, per-tile-run GEMV: `tiles` waves per 16-column tile (each takes a
 *     run of at most 8 quads of 512 k), `waves` waves per workgroup (1..8).
 *   M >= 2: `tiles` (or `waves`) tile groups per workgroup (1..8, one per
 *     wave), `splits` K slices across workgroups.
 * A geometry the compiled kernels cannot take fails with QG_ERR_INVALID_ARG at
 * create or on the run that needs it. */
typedef struct {
  int32_t tiles, waves, splits;
} qg_launch;

typedef struct {
  int32_t K;                /* in-features; multiple of 128                                   */
  int32_t N;                /* out-features; multiple of 16                                   */
  int32_t group_size;       /* scale group: 128; UNIFORM also 64 or 32 (W4A16 g64 / g32 --
                               "The Rock8", dormant-capabilities table: int4 weight-only
                               at group 128, 64 and 32)                                       */
  int32_t format;           /* qg_format                                                      */
  int32_t bits;             /* UNIFORM: 2, 3 or 4 for every column, or 0 = per-column widths  */
  const uint8_t* col_bits;  /* host, N entries in {2,3,4}; read iff format UNIFORM and bits 0 */
  const void* codes;        /* device, canonical packed layout above; 16-byte aligned          */
  const uint16_t* scales;   /* device, fp16 bits [N][K/group_size]; 16-byte aligned. With
                               groups of 64 or 32 the verify GEMM (2..32 rows) folds each
                               scale into its fp16 operand, 2 (c - o) s rounded once, so
                               scales beyond 4096 would overflow there                        */
  const uint16_t* codebook; /* device, fp16 bits [65536]; TRELLIS3 only                        */
  uint32_t flags;           /* QG_FLAG_*                                                       */
  uint32_t pins;            /* QG_PIN_*, 0 = built-in choices                                  */
  qg_launch launch[3];      /* per row class: [0] M = 1, [1] M = 2..16, [2] M = 17..32; zeros =
                               built-in (zero-initialise the whole descriptor)                  */
} qg_weight_desc;

/* Validate the descriptor, check the current device is gfx950 (the pages'
 * kernels target RDNA and refuse other GPUs -- OrcaSAQ2 page, "Supported GPUs";
 * this library likewise runs on gfx950 only), re-lay-out the weights into
 * handle-owned device memory and size the workspace for runs of up to max_M
 * rows (1 <= max_M <= 32, the verify batch bound of the Qwen3.8-27B page, "What
 * we added on top of upstream").  Synchronises `stream` before it returns.  On
 * failure *out is set to NULL and nothing stays allocated. */
qg_status qgemv_create(qg_handle* out, const qg_weight_desc* desc, int32_t max_M, void* stream);

/* y[M][N] = x[M][K] * W^T (TRELLIS3: rotate(x) * W^T unless pre-rotated): the
 * decode GEMV at M = 1 ("The Rock8", decode-features table: a memory-bound
 * decode GEMV) and the speculative-decode verify product at M = 2..32
 * (Qwen3.8-27B page, "What we added on top of upstream": an 8-token verify,
 * batches up to 32 rows).  x, y: device, fp16, 16-byte aligned, [M][K] and
 * [M][N] row-major; 1 <= M <= max_M.  Enqueues on stream. */
qg_status qgemv_run(qg_handle h, const uint16_t* x, int32_t M, uint16_t* y, void* stream);

/* Several independent products of the same row count in one call: for i < n,
 * y_i = x_i * W_i^T with W_i the matrix of hs[i] -- the sibling projections of
 * a layer that read the same input (pass the same x pointer: "The Rock8",
 * env-var table, sibling matmuls that read the same input tensor), or a whole
 * layer's linear set at one step (OrcaSAQ2 page, intro: launch counts cut by
 * fusing).  hs, xs, ys: host arrays of n entries (1 <= n <= 8); xs[i], ys[i]:
 * device fp16 [M][K_i] and [M][N_i], 16-byte aligned; the handles must be
 * distinct (each brings its own workspace).  At M = 1 with UNIFORM handles
 * all n products run in one launch, each matrix in K slices of at most 10
 * quads that meet in fixed-point words (results within the matmul tolerance
 * of qgemv_run's, not bit-identical to them where the slicing differs, and
 * bit-identical across repeats); otherwise each entry runs as qgemv_run, in
 * order, on `stream`. */
qg_status qgemv_run_batch(int32_t n, const qg_handle* hs, const uint16_t* const* xs, uint16_t* const* ys, int32_t M,
                          void* stream);

/* Bytes of the static scratch array qgemv_run_noalloc works in (per GPU):
 * 64 KiB of arrival counters, 4 MiB of fixed-point words, the rest for fp32
 * partials and staging. */
#define QG_SCRATCH_BYTES (16 << 20)

/* For callers that cannot allocate device memory at run time (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same product as qgemv_run, by the same kernels and launch plans (so the
 * same bits), but its workspace (split-K partials, arrival counters,
 * fixed-point words, the trellis path's rotated x) lives in a file-scope
 * static device array of QG_SCRATCH_BYTES per GPU, held until the process
 * ends, instead of in the handle.  It calls no hipMalloc, hipFree or other
 * allocating routine.  A run whose workspace exceeds a region of the array
 * fails with QG_ERR_INVALID_ARG before enqueueing anything (each 27B-class
 * layer shape fits at every row count; at most about 7 MB of partials, for
 * 5120 x 17408 at 32 rows).  The first call on a GPU also
 * enqueues a kernel that clears the array; every run leaves its counters and
 * words cleared again.  All calls on one GPU share the array: calls that
 * overlap on one GPU (other streams, or other threads) race, and must be
 * ordered by the caller.  The current device must be the handle's. */
qg_status qgemv_run_noalloc(qg_handle h, const uint16_t* x, int32_t M, uint16_t* y, void* stream);

/* Fused MLP: out = down( SiLU(gate(x)) * up(x) ), SiLU(z) = z / (1 + e^-z)
 * (Qwen3.8-27B page, "What we added on top of upstream": a fused MLP path for
 * the verify batches; OrcaSAQ2 page, intro: fewer launches).  gate and up:
 * same K (= hidden), same N (= intermediate), same per-column widths; down:
 * K = intermediate.  x: device fp16 [M][hidden]; out: device fp16 [M][down N];
 * both 16-byte aligned.  gate and up run as one pass over x; the intermediate
 * h = SiLU(g)*u stays fp32 in the gate handle (for 2..32 rows it is rounded
 * once more to fp16 with a power-of-two exponent per 128 values for the
 * matrix cores).  UNIFORM handles only. */
qg_status qmlp_run(qg_handle gate, qg_handle up, qg_handle down, const uint16_t* x, int32_t M, uint16_t* out,
                   void* stream);

/* Prefill-size products (any M >= 1): y = x * W^T, with the route chosen by
 * row count as the pages describe for prompt processing ("The Rock8",
 * "Per-format hipBLASLt routes" and the route-crossover paragraph, which
 * moves with the model shape).  Above the crossover the weights are
 * dequantised to fp16 -- each w = (c - o) * s rounded once (RNE) -- and
 * multiplied by a plain fp16 GEMM with fp32 accumulation (hipBLASLt).  Up to
 * it -- measured on the 27B-class shapes, as (N, K), for uniform codes at
 * group 128 / groups of 64 or 32 / MXFP4 / MXFP6: 128 / 96 / 64 / 64 rows on
 * (17408, 5120), 224 / 160 / 128 / 96 on (5120, 17408), 64 on (5120, 5120),
 * 64 on (1024, 5120) at group 128; elsewhere 32 rows per 2048 of sqrt(N K),
 * at most 256, times 3/4 for groups of 64 or 32 and 1/2 for MX elements,
 * rounded down to a multiple of 32 (none below about 4.2 M weights) -- the
 * rows go
 * through the verify GEMM of qgemv_run, 32 at a time (max_M of at least 16
 * at a time), on the handle's own workspace and without rounding the weights.
 * x: device fp16 [M][K]; y: device fp16 [M][N]; both 16-byte aligned.
 * workspace: device, 256-byte aligned, ws_bytes long, caller-owned: its first
 * 32 MiB are the GEMM's workspace, the rest holds fp16 weight rows of a chunk
 * of output columns (the whole matrix when it fits; one width per handle can
 * be cut into chunks of 16-column multiples, several widths need the whole
 * matrix).  qgemv_prefill_workspace gives the least and the full size.
 * Enqueues on `stream` and returns; allocates no device memory.  The first
 * call on a device creates the library's hipBLASLt handle, and the first call
 * for a problem shape plans it (host work; warm a shape before capturing it).
 * The chunked rows use the handle's workspace, so calls on one handle are
 * ordered like qgemv_run's.  UNIFORM, MXFP4 and MXFP6 handles
 * (QG_ERR_UNSUPPORTED otherwise); errors of the GEMM return QG_ERR_DEVICE with hipBLASLt's
 * reason. */
qg_status qgemv_run_prefill(qg_handle h, const uint16_t* x, int32_t M, uint16_t* y, void* workspace, size_t ws_bytes,
                            void* stream);

/* Workspace sizes of qgemv_run_prefill (host out-pointers): the least it
 * accepts and the size that holds the whole matrix's fp16 weights. */
qg_status qgemv_prefill_workspace(qg_handle h, size_t* min_bytes, size_t* full_bytes);

/* Free everything the handle owns (NULL is accepted). */
qg_status qgemv_destroy(qg_handle h);

/* Message of the last failure on this thread ("" if none). */
const char* qg_last_error(void);

/* Bytes the weights occupy in the canonical format (codes + scales; a
 * trellis codebook is not counted): the algorithmic bytes a run must read.
 * Host out-pointer. */
qg_status qgemv_weight_bytes(qg_handle h, int64_t* bytes);

/* Measurement aid, not part of the product: a plain streaming read of `bytes`
 * (a multiple of 16) at device address buf (16-byte aligned) on `stream`, the
 * measured read roofline the GEMV timings are set against ("The Rock8",
 * decode-features table: a decode GEMV at 95-97 % of the measured DRAM
 * roofline).  Reads only; writes nothing. */
qg_status qg_stream_read(const void* buf, int64_t bytes, void* stream);

/* ---- checking entry points: the run kernels' own device decode functions,
 *      written back per weight so tests can compare them bit for bit ---- */

/* codes: device int32 [N][K], the unpacked code of every weight, as the M = 1
 * GEMVs decode it (UNIFORM; MXFP4 / MXFP6: the element's 4- or 6-bit code). */
qg_status qgemv_debug_unpack(qg_handle h, int32_t* codes, void* stream);

/* w: device fp32 [N][K], exact dequantised weight (c - o_b) * s (UNIFORM, as
 * the M = 1 GEMVs decode it), element * 2^(e - 127) (MXFP4 / MXFP6) or
 * codebook[state] * s (TRELLIS3).  q16 (may be NULL): device fp16 bits [N][K]
 * of c - o_b (UNIFORM) or of the element's value (MX formats). */
qg_status qgemv_debug_dequant(qg_handle h, float* w, uint16_t* q16, void* stream);

/* The verify GEMM's (M >= 2) decode of UNIFORM codes into the matrix-core
 * operand: codes (device int32 [N][K]) read back out of the operand registers,
 * b16 (device fp16 bits [N][K]) the operand element itself (c * 2^-23, i.e. the
 * integer 2c as fp16 bits), and w (device fp32 [N][K]) the dequantised weight
 * rebuilt from the operand value and the kernel's offset constant,
 * (op - o_b * 2^-23) * 2^23 * s.  Scale groups of 64 or 32: the operand is
 * 2 (c - o_b) s rounded once to fp16 and w half its value.  MXFP4: the operand
 * is element * 2^-14 * 2^-(e_max - e) (e_max the largest exponent of the
 * 128-group), rounded once, and w = op * 2^(e_max - 113); MXFP6: element *
 * 2^(3 - (e_max - e)), w = op * 2^(e_max - 130).  Each pointer may be NULL,
 * not all three. */
qg_status qgemv_debug_operand(qg_handle h, int32_t* codes, uint16_t* b16, float* w, void* stream);

/* states: device uint16 [N][K], the trellis state of every weight (TRELLIS3). */
qg_status qgemv_debug_trellis(qg_handle h, uint16_t* states, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
