// qgemv.hip -- host side of the C ABI declared in include/qgemv.h: descriptor
// validation, device check, weight re-layout into handle-owned memory, launch
// planning per (shape, row count) and dispatch onto the caller's stream.  The
// kernels are launched through qg_launch.h (one translation unit per kernel
// family).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/qgemv.h"
#include "qg_launch.h"

using namespace qg;

namespace {

thread_local std::string g_err;

qg_status fail(qg_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define QG_HIP(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) return fail(QG_ERR_DEVICE, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

struct Launch {
  int T = 0, NW = 0, S = 0;  // 0 = built-in choice
};

// Device workspace of a run: fp32 split-K partials, arrival counters and
// fixed-point output words (counters and words zero between runs: every
// kernel re-arms what it used), and the trellis path's rotated activations.
struct Work {
  float* partial = nullptr;
  size_t partial_floats = 0;
  int* counters = nullptr;
  size_t ncounters = 0;
  unsigned long long* acc64 = nullptr;
  size_t acc64_words = 0;
  uint16_t* xrot = nullptr;
  size_t xrot_halves = 0;
};

struct HostSeg {
  int bits, tiles, tile0, ncols;
  int sq = 0;  // scale group 64 or 32 (per-lane-quarter scale layout)
  int mx = 0;  // 1: MXFP4 elements; 2: MXFP6 elements (bits 6, the two-plane layout)
  uint32_t* codes = nullptr;
  uint16_t* scales = nullptr;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int mclass(int M) { return M <= 1 ? 0 : (M <= 16 ? 1 : 2); }

}  // namespace

struct qg_plan {
  int K = 0, N = 0, G = 0, G4 = 0, format = 0, max_M = 0;
  int group_size = QG_GROUP;      // scale group: 128, or 64 / 32 (uniform codes)
  uint32_t flags = 0, pins = 0;
  bool debug_sync = false;        // QG_DEBUG_SYNC set at create: synchronise and check after each run
  int device = 0;
  int cus = 0;                    // compute units of the device
  Launch over[3];
  std::vector<HostSeg> segs;
  std::vector<uint8_t> col_bits;  // host copy (uniform: per column)
  int total_tiles = 0;
  int32_t* col_map = nullptr;     // device [16*total_tiles]
  int64_t weight_bytes = 0;
  Work ws;                        // the handle's own workspace (allocated at create)
  // the fused MLP's intermediate (in the gate handle): fp32 h [max_M][N], and
  // for 2..32 rows its block-exponent fp16 form [max_M][N] with the factors
  // [max_M][N/128]
  float* h32 = nullptr;
  uint16_t* h16 = nullptr;
  float* hf = nullptr;
  // trellis
  uint32_t* tcodes = nullptr;     // device layout of trellis tiles
  uint16_t* tscales = nullptr;    // [N/16 tiles][G][16]
  uint16_t* codebook = nullptr;   // device copy, 65536 fp16
  int64_t tr_units = 0;           // (N/16) * G
  int tr_grid = 0, tr_maxseg = 0;
  bool tr_fx = false;             // M = 1 trellis GEMV hands row blocks on through fixed-point words (acc64)
};

namespace {

qg_status after_launch(const qg_plan* h, hipError_t e, hipStream_t st) {
  if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  if (h->debug_sync) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel failed: %s", hipGetErrorString(e));
  }
  return QG_OK;
}

WSet wset_of(const qg_plan* h) {
  WSet w{};
  w.nseg = (int)h->segs.size();
  for (int i = 0; i < w.nseg; ++i) {
    const HostSeg& s = h->segs[i];
    w.seg[i] = SegDev{s.codes, s.scales, s.bits, s.tiles, s.tile0, s.sq, s.mx};
  }
  w.col_map = h->col_map;
  return w;
}

// the kernels' width argument: the single code width, 0 for several, 5 for
// MXFP4, 6 for MXFP6
int single_bits(const qg_plan* h) {
  if (h->format == QG_FMT_MXFP4) return 5;
  if (h->format == QG_FMT_MXFP6) return 6;
  return h->segs.size() == 1 ? h->segs[0].bits : 0;
}
// uniform codes and the MX formats share the tile layout and the GEMV / verify GEMM
bool mxfmt(int f) { return f == QG_FMT_MXFP4 || f == QG_FMT_MXFP6; }
bool coded(const qg_plan* h) { return h->format == QG_FMT_UNIFORM || mxfmt(h->format); }

// ---- M = 1 plans -------------------------------------------------------------
// quads-per-wave counts the per-group GEMV is compiled for
constexpr int kNQ[] = {1, 2, 3, 4, 5};
int nq_round_up(int nq) {
  for (int v : kNQ)
    if (v >= nq) return v;
  return 0;
}

struct M1Plan {
  int S = 1, NW = 1, NQ = 0;
};

// Per-group GEMV: one tile per workgroup; NW waves of NQ quads each split the
// K slice.  Measured on the decode shapes: 2 quads per wave is fastest, then
// 3, then 1 (more quads per wave lengthen the serial load-to-use chain, fewer
// add per-wave fixed cost); take the first of that order that fits in 16 waves
// with <= 1/8 dead quads (the fused gate/up pass: at most 2 quads per wave
// on this path).
// K slices (one matrix; measured): up to K = 8192 and 1024 tiles, of about 2
// quads (a one-wave workgroup per slice: q/o 6.4 us against 7.0 in one slice,
// q|k|v stacked 7.1 against 7.2; wider matrices gain nothing: gate/up
// 10.4-10.9 either way, gate|up stacked 16.7 in one slice against 16.9-18.8);
// beyond K = 8192 of about 7 quads (down: 10.6-10.8 against 14.7 in one slice;
// with 2- and 3-bit columns 11.8 against 12.9 in 4).
// Several widths beyond K = 8192 (the fused MLP's down pass), and the fused
// gate/up pass, take 3 quads per wave (measured, same-box A/B in palindrome
// order, the MLP 5120 -> 17408 -> 5120 at one row: with mixed widths 36.0 ->
// 32.0 us from the gate/up pass, 31.3 us with the down pass in slices of 12
// quads; with one width 29.1 -> 28.2 us from the gate/up pass, while the
// one-width down pass is faster as it was).
M1Plan m1_plan(const qg_plan* h, bool dual) {
  const Launch& L = h->over[0];
  M1Plan p;
  const int G4 = h->G4;
  const bool several = h->segs.size() > 1;
  p.S = L.S > 0 ? L.S
                : (dual ? 1
                        : (G4 > 16 ? (several ? (G4 + 11) / 12 : (G4 + 6) / 8)
                                   : (h->total_tiles <= 1024 ? (G4 + 1) / 2 : 1)));
  p.S = std::min(p.S, G4);
  const int g4s = (G4 + p.S - 1) / p.S;
  if (L.NW <= 0 && (dual || (several && G4 > 16)) && g4s >= 9 && (g4s + 2) / 3 <= 16) {
    p.NQ = 3;
    p.NW = (g4s + 2) / 3;
  } else if (L.NW <= 0) {
    static const int order[] = {2, 3, 1, 4, 5};
    int best_nw = std::min(16, g4s), best_nq = (g4s + best_nw - 1) / best_nw;
    for (int nq : order) {
      if (dual && nq > 2) continue;
      const int nw = (g4s + nq - 1) / nq;
      if (nw > 16) continue;
      const int dead = nw * nq - g4s;
      if (dead * 8 > std::max(g4s, 8)) continue;
      best_nq = nq;
      best_nw = nw;
      break;
    }
    p.NW = best_nw;
    p.NQ = nq_round_up(best_nq);
    // more 2-quad waves than the chip holds at once (seven per SIMD): 3 quads
    // per wave instead, as the batched launch measured (a stacked gate|up
    // handle, 2,176 tiles: one and a half rounds of 5-wave workgroups)
    const int64_t waves = (int64_t)h->total_tiles * p.S * p.NW;
    if (p.NQ == 2 && waves > (int64_t)7 * 4 * std::max(1, h->cus) && g4s >= 9 && (g4s + 2) / 3 <= 16) {
      p.NQ = 3;
      p.NW = (g4s + 2) / 3;
    }
  } else {
    p.NW = L.NW;
    p.NQ = nq_round_up((g4s + L.NW - 1) / L.NW);
  }
  return p;
}

bool sk_fits(const qg_plan* h) { return h->G4 <= 63 * SK_UPW; }

// M = 1 kernel choice, measured on the decode shapes: the per-group kernel
// from 256 tiles up, the per-tile-run kernel for narrower matrices.
bool use_sk(const qg_plan* h) {
  if (!sk_fits(h) || mxfmt(h->format)) return false;  // MX formats: the per-group GEMV only
  if (h->pins & QG_PIN_M1_PERGROUP) return false;
  if (h->pins & QG_PIN_M1_RUNS) return true;
  return h->total_tiles < 256;
}

struct SkPlan {
  int NW = 4, nch = 1, runq = 1;
  unsigned grid = 0;
  int wg_prefix[MAX_SEG + 1] = {};
};

// measured on the decode shapes: 4 waves per workgroup (8 for K >= 16384), and
// enough waves per tile for about 25 / 16 waves per SIMD over the whole chip
SkPlan sk_plan(const qg_plan* h) {
  const Launch& L = h->over[0];
  SkPlan p;
  p.NW = L.NW > 0 ? std::min(L.NW, 8) : (h->G4 >= 32 ? 8 : 4);
  const int nch_min = (h->G4 + SK_UPW - 1) / SK_UPW;
  const int nch_want = L.T > 0 ? L.T : (int)((25LL * h->cus / 4 + h->total_tiles - 1) / h->total_tiles);
  p.nch = std::max(nch_min, std::min(nch_want, std::min(h->G4, 63)));
  p.runq = (h->G4 + p.nch - 1) / p.nch;  // run ch covers quads [ch G4 / nch, (ch + 1) G4 / nch)
  // one segment per workgroup: each segment's waves are rounded up to whole workgroups
  int wgs = 0;
  for (int i = 0; i < (int)h->segs.size(); ++i) {
    p.wg_prefix[i] = wgs;
    wgs += (int)(((int64_t)h->segs[i].tiles * p.nch + p.NW - 1) / p.NW);
  }
  for (int i = (int)h->segs.size(); i <= MAX_SEG; ++i) p.wg_prefix[i] = wgs;
  p.grid = (unsigned)wgs;
  return p;
}

// ---- verify GEMM plans ---------------------------------------------------------
constexpr int kXsNQs[] = {4, 5, 8};  // slice lengths (quads) the verify GEMM is compiled for

int xs_nq_compiled(int nq) {
  for (int v : kXsNQs)
    if (v >= nq) return v;
  return 0;
}

// Plan of the verify GEMM (k_gemm_xs): K slices S (as few as let the slice of
// x fit LDS), T tiles per group and GPW tile groups per workgroup, one per wave,
// at most 8 (about one workgroup per LDS slot of the chip).
struct XsPlan {
  int MT = 1, T = 2, S = 1, nq = 1, NQ = 4, GPW = 1, NW = 1;
  bool fx = false;  // K slices meet in fixed-point words (else fp32 partials)
  size_t lds = 0;
  unsigned grid = 0;
  int wg_prefix[MAX_SEG + 1] = {};
  int tg_prefix[MAX_SEG + 1] = {};
};

// Launch shapes of the verify GEMM measured best on MI355X (sweeps over tile
// groups per workgroup GPW and K slices S) for the 27B-class layer shapes; the
// generic rule in xs_plan covers other shapes.
struct XsTuned {
  int N, K, mcls, GPW, S, T;  // T: tiles per tile group (1 or 2)
};
constexpr XsTuned kXsTuned[] = {
    {5120, 5120, 1, 8, 6, 1},  {5120, 5120, 2, 8, 4, 1},    // q, o
    {1024, 5120, 1, 4, 10, 1}, {1024, 5120, 2, 4, 10, 1},   // k, v
    {17408, 5120, 1, 8, 3, 1}, {17408, 5120, 2, 8, 3, 2},   // gate, up
    {5120, 17408, 1, 8, 6, 1}, {5120, 17408, 2, 8, 9, 2},   // down
    {7168, 5120, 1, 8, 4, 1},  {7168, 5120, 2, 8, 4, 1},    // q | k | v stacked
    {34816, 5120, 1, 8, 3, 1}, {34816, 5120, 2, 8, 3, 2},   // gate | up stacked
};

bool invariant(const qg_plan* h) { return (h->flags & QG_FLAG_BATCH_INVARIANT) != 0; }

// Batch-invariant handles plan every row count as max_M rows (at least 2):
// the K slices, tile grouping, workgroup split and hand-over are then the same
// for every M, and only the row tiles actually computed (MT) and the LDS taken
// follow M.  Each output element's arithmetic -- its MFMA chains over the
// slice's groups in order, its scale products and the slices' hand-over --
// does not depend on the other rows.
XsPlan xs_plan(const qg_plan* h, int M, bool dual, bool xsc) {
  XsPlan p;
  const int Mp = invariant(h) ? std::max(2, h->max_M) : M;  // the row count the plan is made for
  Launch L = h->over[mclass(Mp)];
  // one-tile groups (twice the waves) measured faster except for wide
  // matrices at more than 16 rows
  int tuned_T = (Mp <= 16 || h->total_tiles <= 512) ? 1 : 2;
  if (!dual)
    for (const XsTuned& t : kXsTuned)
      if (t.N == h->N && t.K == h->K && t.mcls == mclass(Mp)) {
        tuned_T = t.T;
        if (L.T <= 0 && L.NW <= 0 && L.S <= 0) {
          L.T = t.GPW;
          L.S = t.S;
        }
      }
  p.MT = M <= 16 ? 1 : 2;
  const int MTp = Mp <= 16 ? 1 : 2;
  // tiles per tile group: 1 for the fused gate/up pair; else the tuned count
  p.T = dual ? 1 : tuned_T;
  if (!dual && (h->pins & QG_PIN_XS_T1)) p.T = 1;
  if (!dual && (h->pins & QG_PIN_XS_T2)) p.T = 2;
  const size_t col_cap = 4096;  // room for the run's column map
  const size_t nsum = xsc ? 2 : 1;
  // fewest K slices whose x slice fits LDS (at the compiled slice length)
  p.S = std::max(1, std::min(h->G4, L.S > 0 ? L.S : 1));
  for (;; ++p.S) {
    p.nq = (h->G4 + p.S - 1) / p.S;
    p.NQ = xs_nq_compiled(p.nq);
    if (p.NQ > 0 && xs_x_bytes(Mp, p.NQ) + nsum * xs_sum_bytes(MTp, p.NQ) + col_cap <= kLdsMax) break;
    if (p.S >= h->G4) break;
  }
  int tg = 0;
  for (const auto& sg : h->segs) tg += (sg.tiles + p.T - 1) / p.T;
  const size_t lds0 = xs_x_bytes(Mp, p.NQ) + nsum * xs_sum_bytes(MTp, p.NQ) + 1024;
  const int per_cu = std::max(1, (int)(kLdsMax / lds0));
  const int64_t want = (int64_t)std::max(1, h->cus) * per_cu;  // workgroups that fit at once
  if (L.T > 0) p.GPW = L.T;
  else if (L.NW > 0) p.GPW = L.NW;
  else p.GPW = (int)std::max<int64_t>(1, ((int64_t)tg * p.S + want - 1) / want);
  p.GPW = std::max(1, std::min(p.GPW, 8));  // one tile group per wave
  p.NW = p.GPW;
  int wgs = 0, tgs = 0;
  for (int i = 0; i < (int)h->segs.size(); ++i) {
    const int ng = (h->segs[i].tiles + p.T - 1) / p.T;
    p.wg_prefix[i] = wgs;
    p.tg_prefix[i] = tgs;
    wgs += (ng + p.GPW - 1) / p.GPW;
    tgs += ng;
  }
  for (int i = (int)h->segs.size(); i <= MAX_SEG; ++i) {
    p.wg_prefix[i] = wgs;
    p.tg_prefix[i] = tgs;
  }
  p.grid = (unsigned)wgs * (unsigned)p.S;
  p.lds = xs_lds_bytes(M, p.MT, p.NQ, p.GPW, p.T, xsc);
  // fixed-point words when the atomics are few (measured: they win at 8 and 16
  // rows on every decode shape, the partial blocks at 32 rows on gate/up and
  // down -- down at 32 rows 22.9 -> 20.6 us with 9 slices)
  const int64_t atomics = (int64_t)Mp * 16 * h->total_tiles * p.S;
  p.fx = p.S > 1 && p.S <= 63 && atomics <= (int64_t)1 << 20;
  if (h->pins & QG_PIN_PARTIALS) p.fx = false;
  if (h->pins & QG_PIN_WORDS) p.fx = p.S > 1 && p.S <= 63;
  return p;
}

size_t partial_need(const qg_plan* h, int S, int M, int nd) {
  return S <= 1 ? 0 : (size_t)nd * S * M * (size_t)(16 * h->total_tiles);
}

// the verify GEMM's partials: per (tile group, slice, matrix) a block of T * MT
// quarter tiles of 64 lanes x 4 fp32
size_t xs_partial_need(const XsPlan& p, int nd) {
  return p.S <= 1 ? 0 : (size_t)nd * p.S * (size_t)p.tg_prefix[MAX_SEG] * p.T * p.MT * 256;
}

// M = 1 K slices of one matrix meet in fixed-point words unless pinned to partials
bool m1_fx(const qg_plan* h, int S) { return S > 1 && S <= 63 && !(h->pins & QG_PIN_PARTIALS); }

// Workspace for every plan the handle can run (sized once, at create).
qg_status size_workspace(qg_plan* h, size_t* floats) {
  size_t need = 0;
  if (!use_sk(h)) {
    const M1Plan p1 = m1_plan(h, false);
    if (!m1_fx(h, p1.S)) need = std::max(need, partial_need(h, p1.S, 1, 1));
    const M1Plan p2 = m1_plan(h, true);  // the fused gate/up pass: both matrices' slices
    need = std::max(need, (size_t)2 * std::max(p2.S, 1) * (size_t)(16 * h->total_tiles));
  }
  for (int M = invariant(h) ? 1 : 2; M <= h->max_M; ++M)
    for (int v = 0; v < 3; ++v) {
      const bool dual = v == 1, xsc = v == 2;
      const XsPlan p = xs_plan(h, M, dual, xsc);
      if (p.NQ == 0 || p.lds > kLdsMax)
        return fail(QG_ERR_INVALID_ARG, "verify GEMM: an x slice of %d quads at M=%d does not fit LDS", p.nq, M);
      if (!p.fx) need = std::max(need, xs_partial_need(p, dual ? 2 : 1));
    }
  *floats = need;
  return QG_OK;
}

qg_status check_device(int* dev) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) return fail(QG_ERR_UNSUPPORTED, "no HIP device available");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, d) != hipSuccess) return fail(QG_ERR_UNSUPPORTED, "cannot query HIP device");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(QG_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", d, prop.gcnArchName);
  *dev = d;
  return QG_OK;
}

void free_plan(qg_plan* h) {
  if (!h) return;
  for (auto& s : h->segs) {
    if (s.codes) hipFree(s.codes);
    if (s.scales) hipFree(s.scales);
  }
  void* bufs[] = {h->col_map, h->ws.partial, h->ws.counters, h->ws.acc64, h->h32,     h->h16,
                  h->hf,      h->tcodes,     h->tscales,     h->codebook, h->ws.xrot};
  for (void* p : bufs)
    if (p) hipFree(p);
  delete h;
}

// ---- trellis -----------------------------------------------------------------
// stream-K plan of the M = 1 GEMV: W = grid * NW waves share the U = (N/16) * G
// units; maxseg is the largest number of waves any row block is split over (the
// device kernel finds the same first and last wave of a row block with tr_wave_of)
int tr_wave_of_host(int64_t x, int64_t U, int W) {
  int w = (int)(x * W / U);
  while (w + 1 < W && ((int64_t)(w + 1) * U) / W <= x) ++w;
  while (w > 0 && ((int64_t)w * U) / W > x) --w;
  return w;
}

int tr_maxseg_of(int RB, int G, int64_t U, int W) {
  int mx = 1;
  for (int rb = 0; rb < RB; ++rb) {
    const int w0 = tr_wave_of_host((int64_t)rb * G, U, W);
    const int w1 = tr_wave_of_host((int64_t)rb * G + G - 1, U, W);
    mx = std::max(mx, w1 - w0 + 1);
  }
  return mx;
}

// Banded trellis GEMM: K slices so that the bands x slices workgroups (one per
// compute unit: the codebook fills its LDS) cover the chip in one round.
int tb_slices(const qg_plan* h, int nw) {
  const int RB = h->N / 16, bands = (RB + nw - 1) / nw;
  return std::max(1, std::min(h->G, std::max(1, h->cus) / bands));
}

int tr_waves(const qg_plan* h) { return (int)std::min<int64_t>((int64_t)h->tr_grid * TR_NW, h->tr_units); }

qg_status create_trellis(qg_plan* h, const qg_weight_desc* d, hipStream_t st) {
  const int N = d->N, K = d->K, G = K / QG_GROUP, RB = N / 16;
  h->total_tiles = RB;
  h->tr_units = (int64_t)RB * G;
  h->weight_bytes = (int64_t)N * K * 3 / 8 + (int64_t)N * G * 2;
  // one workgroup per compute unit (the codebook fills its LDS) of 16 waves;
  // the codebook gathers bound the kernel, so small matrices still spread over
  // as many compute units as they have 16 units for
  h->tr_grid = (int)std::max<int64_t>(1, std::min<int64_t>(h->cus, (h->tr_units + 15) / 16));
  const int mseg = tr_maxseg_of(RB, G, h->tr_units, tr_waves(h));
  // the M = 1 GEMV's row blocks meet in fixed-point words (one round trip)
  // where at most 63 waves share one (the words count arrivals in 6 bits)
  h->tr_fx = mseg <= 63 && !(h->pins & QG_PIN_PARTIALS);
  h->tr_maxseg = std::max({mseg, tb_slices(h, TbShape<1>::NW), tb_slices(h, TbShape<2>::NW)});
  const size_t ncode = (size_t)h->tr_units * 64 * 3;
  QG_HIP(hipMalloc(&h->tcodes, ncode * sizeof(uint32_t)));
  QG_HIP(hipMalloc(&h->tscales, (size_t)h->tr_units * 16 * sizeof(uint16_t)));
  QG_HIP(hipMalloc(&h->codebook, 65536 * sizeof(uint16_t)));
  if (!(d->flags & QG_FLAG_X_PREROTATED)) {
    h->ws.xrot_halves = (size_t)h->max_M * K;
    QG_HIP(hipMalloc(&h->ws.xrot, h->ws.xrot_halves * sizeof(uint16_t)));
  }
  const size_t nf = (size_t)RB * h->tr_maxseg * h->max_M * 16;
  QG_HIP(hipMalloc(&h->ws.partial, nf * sizeof(float)));
  h->ws.partial_floats = nf;
  // fixed-point output words [max_M][N] of the M = 1 GEMV and the banded GEMM, zero between runs
  h->ws.acc64_words = (size_t)h->max_M * N;
  QG_HIP(hipMalloc(&h->ws.acc64, h->ws.acc64_words * sizeof(unsigned long long)));
  QG_HIP(hipMemsetAsync(h->ws.acc64, 0, h->ws.acc64_words * sizeof(unsigned long long), st));
  QG_HIP(hipMemcpyAsync(h->codebook, d->codebook, 65536 * sizeof(uint16_t), hipMemcpyDeviceToDevice, st));
  QG_HIP(launch_repack_trellis((const uint16_t*)d->codes, d->scales, K / 16, G, h->tr_units, h->tcodes, h->tscales, st));
  return QG_OK;
}

// 2..8 rows: the banded GEMM that stages its K slice's x once (and rotates
// it there) where M x (groups per slice) pieces of 256 bytes fit beside the
// codebook; the band kernel's K slices, so the workspace is the same
bool trellis_bx(const qg_plan* h, int M) {
  if (M < 2 || M > TBX_MAXM || (h->pins & QG_PIN_TRELLIS_BAND)) return false;
  const int S = tb_slices(h, TbShape<1>::NW);
  return (int64_t)M * ((h->G + S - 1) / S) <= TBX_XBYTES / 256;
}

// M = 1 GEMV that rotates x itself into LDS (no separate rotation launch):
// room for the rotated x beside the codebook up to K = 16384
// x rotated inside the run kernel.  2..32 rows: each band workgroup rotates the
// groups of its K slice as it stages them, so every group is rotated once per
// band; measured (same-box A/B, 8 rows): k/v (160 band-groups) 13.2 -> 11.8 us,
// q/o (800) 19.0 -> 18.5, but gate/up and down (2,720) 39.5 -> 41.1 and
// 35.1 -> 35.9, where one rotation launch is cheaper.  One row: where the
// rotated x fits the GEMV's LDS.
bool trellis_xl(const qg_plan* h, int M) {
  if (trellis_bx(h, M)) return !(h->flags & QG_FLAG_X_PREROTATED);
  if (M > 1) {
    const int nw = M > 16 ? TbShape<2>::NW : TbShape<1>::NW;
    const int64_t bands = (h->N / 16 + nw - 1) / nw;
    return !(h->flags & QG_FLAG_X_PREROTATED) && bands * h->G <= 2000;
  }
  if (h->pins & QG_PIN_TRELLIS_ROT_LAUNCH) return false;
  return !(h->flags & QG_FLAG_X_PREROTATED) && (size_t)h->K * 2 <= (size_t)TR_XL_BYTES &&
         h->G <= TR_XL_GMAX * TR_NW;
}

qg_status run_trellis(const qg_plan* h, const Work& w, const uint16_t* x, int M, uint16_t* y, hipStream_t st) {
  const uint16_t* xr = x;
  const bool xl = trellis_xl(h, M);
  if (!(h->flags & QG_FLAG_X_PREROTATED) && !xl) {
    const hipError_t e = launch_fwht(x, w.xrot, M, h->K, st);
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "rotation launch failed: %s", hipGetErrorString(e));
    xr = w.xrot;
  }
  if (M > 1) {
    const int MT = M > 16 ? 2 : 1;
    const int nw = MT == 2 ? TbShape<2>::NW : TbShape<1>::NW;
    TbArgs b{};
    b.codes = h->tcodes;
    b.scales = h->tscales;
    b.cb = h->codebook;
    b.x = xr;
    b.rot = xl ? 1 : 0;
    b.y = y;
    b.partial = w.partial;
    b.counters = w.counters;
    b.M = M;
    b.K = h->K;
    b.N = h->N;
    b.G = h->G;
    b.RB = h->N / 16;
    b.maxseg = h->tr_maxseg;
    b.S = tb_slices(h, nw);
    if (b.S > h->tr_maxseg) return fail(QG_ERR_INVALID_ARG, "%d K slices exceed the workspace's %d", b.S, h->tr_maxseg);
    // K slices meet in fixed-point words where the atomics are few (and the
    // words' 6-bit count holds S)
    const bool fx = b.S > 1 && b.S <= 63 && (int64_t)M * h->N * b.S <= (1 << 20) && !(h->pins & QG_PIN_PARTIALS);
    b.acc = fx ? w.acc64 : nullptr;
    const unsigned grid = (unsigned)(((b.RB + nw - 1) / nw) * b.S);
    if (trellis_bx(h, M)) return after_launch(h, launch_trellis_bx(b, grid, st), st);
    return after_launch(h, launch_trellis_band(b, MT, grid, st), st);
  }
  TrArgs a{};
  a.codes = h->tcodes;
  a.scales = h->tscales;
  a.cb = h->codebook;
  a.x = xr;
  a.y = y;
  a.partial = w.partial;
  a.counters = w.counters;
  a.acc = h->tr_fx ? w.acc64 : nullptr;
  a.K = h->K;
  a.N = h->N;
  a.G = h->G;
  a.RB = h->N / 16;
  a.maxseg = h->tr_maxseg;
  a.W = tr_waves(h);  // every wave's range non-empty
  a.U = h->tr_units;
  return after_launch(h, launch_trellis_gemv(a, xl, (unsigned)h->tr_grid, st), st);
}

// ---- uniform create -----------------------------------------------------------
qg_status create_uniform(qg_plan* h, const qg_weight_desc* d, hipStream_t st) {
  const int N = d->N, K = d->K, G = K / QG_GROUP, G4 = (G + 3) / 4;
  h->col_bits.resize(N);
  const bool mx = mxfmt(d->format), mx6 = d->format == QG_FMT_MXFP6;
  if (mx) {
    // E2M1 elements in 4-bit fields, E3M2 elements in 6-bit fields
    std::fill(h->col_bits.begin(), h->col_bits.end(), (uint8_t)(mx6 ? 6 : 4));
  } else if (d->bits == 0) {
    if (!d->col_bits) return fail(QG_ERR_INVALID_ARG, "bits == 0 needs col_bits (host, N entries)");
    for (int n = 0; n < N; ++n) {
      const int b = d->col_bits[n];
      if (b < 2 || b > 4) return fail(QG_ERR_INVALID_ARG, "col_bits[%d] = %d is not in {2,3,4}", n, b);
      h->col_bits[n] = (uint8_t)b;
    }
  } else {
    if (d->bits < 2 || d->bits > 4) return fail(QG_ERR_INVALID_ARG, "bits = %d is not in {0,2,3,4}", d->bits);
    std::fill(h->col_bits.begin(), h->col_bits.end(), (uint8_t)d->bits);
  }
  // segments: columns grouped by width (ascending column order inside each)
  std::vector<int32_t> cmap;
  std::vector<int64_t> row_off(N);
  int64_t acc = 0;
  for (int n = 0; n < N; ++n) {
    row_off[n] = acc;
    acc += (int64_t)h->col_bits[n] * K / 32;
  }
  const int gs = d->group_size, sq = gs < QG_GROUP ? 1 : 0;
  h->group_size = gs;
  h->weight_bytes = acc * 4 + (int64_t)N * (K / gs) * (mx ? 1 : 2);  // MX: one exponent byte per block
  // widest codes first: their workgroups (the longest) are dispatched first,
  // so the tail of a launch is the lighter widths'
  int tile0 = 0;
  for (int b = 6; b >= 2; --b) {
    std::vector<int32_t> cols;
    for (int n = 0; n < N; ++n)
      if (h->col_bits[n] == b) cols.push_back(n);
    if (cols.empty()) continue;
    HostSeg s;
    s.bits = b;
    s.sq = sq;
    s.mx = mx ? (mx6 ? 2 : 1) : 0;
    s.ncols = (int)cols.size();
    s.tiles = (s.ncols + 15) / 16;
    s.tile0 = tile0;
    tile0 += s.tiles;
    cols.resize((size_t)16 * s.tiles, -1);
    cmap.insert(cmap.end(), cols.begin(), cols.end());
    h->segs.push_back(s);
  }
  h->total_tiles = tile0;
  QG_HIP(hipMalloc(&h->col_map, cmap.size() * sizeof(int32_t)));
  QG_HIP(hipMemcpyAsync(h->col_map, cmap.data(), cmap.size() * sizeof(int32_t), hipMemcpyHostToDevice, st));
  int64_t* d_off = nullptr;
  QG_HIP(hipMalloc(&d_off, N * sizeof(int64_t)));
  hipError_t e = hipMemcpyAsync(d_off, row_off.data(), N * sizeof(int64_t), hipMemcpyHostToDevice, st);
  for (auto& s : h->segs) {
    if (e != hipSuccess) break;
    const size_t nslot = (size_t)s.tiles * G4 * 64;
    if (hipMalloc(&s.codes, nslot * s.bits * 4 * sizeof(uint32_t)) != hipSuccess ||
        hipMalloc(&s.scales, nslot * (sq ? 4 : 1) * sizeof(uint16_t)) != hipSuccess) {
      hipStreamSynchronize(st);
      hipFree(d_off);
      return fail(QG_ERR_OOM, "device allocation for the weight layout failed");
    }
    if (mx6)
      e = launch_repack_mx6((const uint32_t*)d->codes, h->col_map + 16 * s.tile0, s.tiles, G, G4, s.codes, st);
    else
      e = launch_repack_uniform((const uint32_t*)d->codes, d_off, d->scales, h->col_map + 16 * s.tile0, s.bits, s.tiles,
                                G, G4, gs, s.codes, mx ? nullptr : s.scales, st);
    if (e == hipSuccess && mx)
      e = launch_repack_mx_scales(reinterpret_cast<const uint8_t*>(d->scales), h->col_map + 16 * s.tile0, s.tiles, G,
                                  G4, s.scales, st);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  hipFree(d_off);
  if (e != hipSuccess) return fail(QG_ERR_DEVICE, "weight re-layout failed: %s", hipGetErrorString(e));
  // workspace, sized for every plan this handle can run
  size_t nf = 0;
  const qg_status s = size_workspace(h, &nf);
  if (s != QG_OK) return s;
  if (nf > 0) {
    if (hipMalloc(&h->ws.partial, nf * sizeof(float)) != hipSuccess)
      return fail(QG_ERR_OOM, "workspace allocation of %zu bytes failed", nf * sizeof(float));
    h->ws.partial_floats = nf;
  }
  // fixed-point output words [2][max_M][16 * total_tiles]: the M = 1 GEMVs use
  // the first 2 * 16 * total_tiles (the fused gate/up pass the first
  // 16 * total_tiles as exchange words), the verify GEMM [matrix][row][column]
  h->ws.acc64_words = (size_t)2 * h->max_M * 16 * h->total_tiles;
  QG_HIP(hipMalloc(&h->ws.acc64, h->ws.acc64_words * sizeof(unsigned long long)));
  QG_HIP(hipMemsetAsync(h->ws.acc64, 0, h->ws.acc64_words * sizeof(unsigned long long), st));
  // the fused MLP's intermediate, when this handle is an MLP's gate
  QG_HIP(hipMalloc(&h->h32, (size_t)h->max_M * N * sizeof(float)));
  if (h->max_M > 1) {
    QG_HIP(hipMalloc(&h->h16, (size_t)h->max_M * N * sizeof(uint16_t)));
    QG_HIP(hipMalloc(&h->hf, (size_t)h->max_M * (N / 128 + 1) * sizeof(float)));
  }
  return QG_OK;
}

// ---- dispatch ------------------------------------------------------------------
// One M = 1 GEMV over a uniform handle, or the fused gate + up pair when h2 !=
// NULL (h = SiLU(g) * u into y).  xf32: x is fp32; yf32: y receives fp32.
qg_status run_m1(const qg_plan* h, const Work& w, const qg_plan* h2, const void* x, bool xf32, void* y, bool yf32,
                 hipStream_t st) {
  const bool dual = h2 != nullptr;
  const int bf = single_bits(h);
  if (use_sk(h)) {
    const SkPlan p = sk_plan(h);
    SkArgs a{};
    a.w[0] = wset_of(h);
    if (h2) a.w[1] = wset_of(h2);
    a.x = x;
    a.y = y;
    a.yf32 = yf32 ? 1 : 0;
    a.acc = w.acc64;
    a.K = h->K;
    a.N = h->N;
    a.G = h->G;
    a.G4 = h->G4;
    a.total_tiles = h->total_tiles;
    a.U = (int64_t)h->total_tiles * h->G4;
    a.nch = p.nch;
    a.runq = p.runq;
    for (int i = 0; i <= MAX_SEG; ++i) a.wg_prefix[i] = p.wg_prefix[i];
    return after_launch(h, launch_gemv_sk(a, dual, p.NW, sk_lds_bytes(p.NW, p.runq), p.grid, bf, xf32, st), st);
  }
  const M1Plan p = m1_plan(h, dual);
  const int nqs = (h->G4 + p.S - 1) / p.S;
  if (p.NQ <= 0 || (int64_t)p.NQ * p.NW < nqs)
    return fail(QG_ERR_INVALID_ARG, "%d waves cannot cover %d quads per slice with the compiled quad counts", p.NW, nqs);
  if (p.NW > 16) return fail(QG_ERR_INVALID_ARG, "at most 16 waves per workgroup");
  const size_t lds = m1_lds_bytes(p.NQ, p.NW);
  if (lds > 65536) return fail(QG_ERR_INVALID_ARG, "K slice of %d quads does not fit LDS: use more splits", nqs);
  GvArgs a{};
  a.w[0] = wset_of(h);
  if (h2) a.w[1] = wset_of(h2);
  a.x = x;
  a.y = y;
  a.yf32 = yf32 ? 1 : 0;
  a.partial = w.partial;
  a.counters = w.counters;
  a.K = h->K;
  a.G = h->G;
  a.G4 = h->G4;
  a.NP = 16 * h->total_tiles;
  a.S = p.S;
  a.pair = dual ? 1 : 0;
  a.xw = w.acc64;
  a.fx = (!dual && m1_fx(h, p.S)) ? 1 : 0;
  int pre = 0;
  for (int i = 0; i < (int)h->segs.size(); ++i) {
    a.ts_prefix[i] = pre;
    pre += h->segs[i].tiles;
  }
  for (int i = (int)h->segs.size(); i <= MAX_SEG; ++i) a.ts_prefix[i] = pre;
  const size_t need = dual ? (size_t)2 * p.S * a.NP : (a.fx ? 0 : partial_need(h, p.S, 1, 1));
  if (need > w.partial_floats) return fail(QG_ERR_INVALID_ARG, "workspace too small for %d K slices", p.S);
  const unsigned grid = (unsigned)pre * (unsigned)p.S * (dual ? 2u : 1u);
  return after_launch(h, launch_gemv_q(a, p.NQ, p.NW, lds, grid, bf, xf32, st), st);
}

// One verify GEMM (2..32 rows) over a uniform handle, or the fused gate + up
// pair when h2 != NULL.  xf: (the MLP's down pass) per (row, group) factors
// of x, [M][G]; yf32: y receives fp32.
qg_status run_xs(const qg_plan* h, const Work& w, const qg_plan* h2, const uint16_t* x, const float* xf, int M, void* y,
                 bool yf32, int ldy, hipStream_t st) {
  const bool dual = h2 != nullptr;
  const bool xsc = xf != nullptr;
  const XsPlan p = xs_plan(h, M, dual, xsc);
  if (p.NQ == 0 || p.lds > kLdsMax)
    return fail(QG_ERR_INVALID_ARG, "x slice of %d quads at M=%d does not fit LDS", p.nq, M);
  if (!p.fx && xs_partial_need(p, dual ? 2 : 1) > w.partial_floats)
    return fail(QG_ERR_INVALID_ARG, "workspace too small for %d K-slices at M=%d", p.S, M);
  if ((size_t)p.tg_prefix[MAX_SEG] > w.ncounters) return fail(QG_ERR_INVALID_ARG, "more tile groups than counters");
  XsArgs a{};
  a.w[0] = wset_of(h);
  if (h2) a.w[1] = wset_of(h2);
  a.x = x;
  a.xf = xf;
  a.y = y;
  a.yf32 = yf32 ? 1 : 0;
  a.partial = w.partial;
  a.counters = w.counters;
  a.acc = p.fx ? w.acc64 : nullptr;
  a.M = M;
  a.K = h->K;
  a.G = h->G;
  a.G4 = h->G4;
  a.ldy = ldy;
  a.NP = 16 * h->total_tiles;
  a.S = p.S;
  a.GPW = p.GPW;
  for (int i = 0; i <= MAX_SEG; ++i) {
    a.wg_prefix[i] = p.wg_prefix[i];
    a.tg_prefix[i] = p.tg_prefix[i];
  }
  const int bf = single_bits(h);
  const bool sq = h->group_size < QG_GROUP;
  const hipError_t e = p.MT == 1 ? launch_gemm_xs1(a, p.T, dual, xsc, p.NQ, bf, sq, p.NW, p.lds, p.grid, st)
                                 : launch_gemm_xs2(a, p.T, dual, xsc, p.NQ, bf, sq, p.NW, p.lds, p.grid, st);
  return after_launch(h, e, st);
}

// Several independent M = 1 products (uniform handles, distinct) in one
// launch of the per-group GEMV: one plan shape for all (NQ quads per wave, NW
// waves per workgroup covering the longest K slice), each matrix cut into as
// many K slices as that takes, slices meeting in fixed-point words (or, with
// the partials pinned, in the handle's partials when they fit).  Measured
// (same-box A/B, palindrome order): 2 quads per wave in slices of at most 10
// quads (5 waves) for narrow batches (q,k,v: 448 tiles, 7.0 us against 7.5
// with 3 quads); 3 quads per wave in slices of at most 12 (4 waves) from 1024
// tiles and 9 quads up (gate,up: 2,176 tiles, 18.95 us against 19.74).
qg_status run_batch_m1(int n, const qg_plan* const* hs, const uint16_t* const* xs, uint16_t* const* ys, hipStream_t st) {
  int maxg4 = 1, bf = single_bits(hs[0]), tiles = 0;
  for (int i = 0; i < n; ++i) {
    maxg4 = std::max(maxg4, hs[i]->G4);
    tiles += hs[i]->total_tiles;
    if (single_bits(hs[i]) != bf) bf = 0;
  }
  const int NQ = (tiles >= 1024 && maxg4 >= 9) ? 3 : 2;
  const int NW = (std::min(NQ == 3 ? 12 : 10, maxg4) + NQ - 1) / NQ;
  GvBatch b{};
  b.n = n;
  int wg = 0;
  for (int i = 0; i < n; ++i) {
    const qg_plan* h = hs[i];
    GvArgs& a = b.task[i];
    const int S = (h->G4 + NW * NQ - 1) / (NW * NQ);
    a.w[0] = wset_of(h);
    a.x = xs[i];
    a.y = ys[i];
    a.partial = h->ws.partial;
    a.counters = h->ws.counters;
    a.K = h->K;
    a.G = h->G;
    a.G4 = h->G4;
    a.NP = 16 * h->total_tiles;
    a.S = S;
    a.xw = h->ws.acc64;
    a.fx = m1_fx(h, S) ? 1 : 0;
    if (S > 1 && !a.fx && partial_need(h, S, 1, 1) > h->ws.partial_floats)
      return fail(QG_ERR_INVALID_ARG, "batch entry %d: %d K slices need more partials than its handle holds", i, S);
    if (S > 63) return fail(QG_ERR_UNSUPPORTED, "batch entry %d: K = %d is too long for one launch", i, h->K);
    int pre = 0;
    for (int k = 0; k < (int)h->segs.size(); ++k) {
      a.ts_prefix[k] = pre;
      pre += h->segs[k].tiles;
    }
    for (int k = (int)h->segs.size(); k <= MAX_SEG; ++k) a.ts_prefix[k] = pre;
    b.wg0[i] = wg;
    wg += pre * S;
  }
  b.wg0[n] = wg;
  for (int i = n + 1; i <= GV_MAX_TASKS; ++i) b.wg0[i] = wg;
  return after_launch(hs[0], launch_gemv_batch(b, NQ, NW, m1_lds_bytes(NQ, NW), (unsigned)wg, bf, st), st);
}

// The workspace one qgemv_run of M rows takes (sizes in elements; the
// allocation-free entry point carves it out of its static array).
Work run_need(const qg_plan* h, int M) {
  Work n;
  n.ncounters = (size_t)std::max(1, h->total_tiles);
  const size_t NP = (size_t)16 * h->total_tiles;
  if (h->format == QG_FMT_TRELLIS3) {
    const int RB = h->N / 16;
    if (!(h->flags & QG_FLAG_X_PREROTATED) && !trellis_xl(h, M)) n.xrot_halves = (size_t)M * h->K;
    if (M > 1) {
      const int S = tb_slices(h, M > 16 ? TbShape<2>::NW : TbShape<1>::NW);
      const bool fx = S > 1 && S <= 63 && (int64_t)M * h->N * S <= (1 << 20) && !(h->pins & QG_PIN_PARTIALS);
      if (fx) n.acc64_words = (size_t)M * h->N;
      else if (S > 1) n.partial_floats = (size_t)RB * h->tr_maxseg * M * 16;
    } else {
      if (h->tr_fx) n.acc64_words = (size_t)h->N;
      else n.partial_floats = (size_t)RB * h->tr_maxseg * 16;
    }
    return n;
  }
  if (M == 1 && !invariant(h)) {
    if (use_sk(h)) {
      n.acc64_words = NP;
    } else {
      const M1Plan p = m1_plan(h, false);
      if (m1_fx(h, p.S)) n.acc64_words = NP;
      else n.partial_floats = partial_need(h, p.S, 1, 1);
    }
    return n;
  }
  const XsPlan p = xs_plan(h, M, false, false);
  if (p.fx) n.acc64_words = (size_t)M * NP;
  else n.partial_floats = xs_partial_need(p, 1);
  return n;
}

qg_status check_launch_overrides(const qg_weight_desc* d) {
  for (int c = 0; c < 3; ++c) {
    const qg_launch& L = d->launch[c];
    if (L.tiles < 0 || L.waves < 0 || L.splits < 0)
      return fail(QG_ERR_INVALID_ARG, "launch[%d]: negative field", c);
    if (L.splits > 63) return fail(QG_ERR_INVALID_ARG, "launch[%d]: at most 63 K slices", c);
    if (c == 0 && (L.waves > 16 || L.tiles > 63))
      return fail(QG_ERR_INVALID_ARG, "launch[0]: at most 16 waves per workgroup and 63 waves per tile");
    if (c > 0 && (L.tiles > 8 || L.waves > 8))
      return fail(QG_ERR_INVALID_ARG, "launch[%d]: at most 8 tile groups per workgroup", c);
  }
  return QG_OK;
}

}  // namespace

// ---- the allocation-free entry point's workspace -----------------------------------
// A file-scope device array (each GPU the library runs on holds its own copy
// until the process ends).  In host code its name is a host-side stand-in, not
// a device address: the device address of each GPU's copy comes from
// hipGetSymbolAddress, once per device, and only that address is ever handed
// to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[QG_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of the current device's copy of `scratch`; the first call on
// a device also clears it (a fill kernel on `st`, in order before the caller's
// work), so counters and fixed-point words start at zero there
qg_status scratch_of(int dev, hipStream_t st, unsigned char** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(QG_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(QG_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    QG_HIP(launch_fill_zero(p, QG_SCRATCH_BYTES, st));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<unsigned char*>(g_scratch_ptr[dev]);
  return QG_OK;
}

// The scratch array's fixed regions: arrival counters and fixed-point words
// (which must read zero when a run starts: every run re-arms what it used, and
// no run ever writes anything else there), then partials and the rotated x
// (written before they are read).  Fixed, so that no run's partials can land
// where a later run expects zeros.
constexpr size_t kScrCounters = 64 << 10;
constexpr size_t kScrWords = 4 << 20;
constexpr size_t kScrRest = (size_t)QG_SCRATCH_BYTES - kScrCounters - kScrWords;
static_assert(QG_SCRATCH_BYTES > kScrCounters + kScrWords, "scratch regions");

// the run's workspace in the scratch array at `base`; false (and a message)
// when a region is too small for it
bool carve(const Work& need, uintptr_t base, Work* w) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const size_t cb = need.ncounters * sizeof(int), wb = need.acc64_words * sizeof(unsigned long long);
  const size_t pb = up(need.partial_floats * sizeof(float)), xb = need.xrot_halves * sizeof(uint16_t);
  if (cb > kScrCounters || wb > kScrWords || pb + xb > kScrRest) {
    fail(QG_ERR_INVALID_ARG,
         "this run needs %zu B of counters, %zu B of words and %zu B of partials and staging; the static scratch "
         "array holds %zu, %zu and %zu",
         cb, wb, pb + xb, kScrCounters, kScrWords, kScrRest);
    return false;
  }
  *w = need;
  w->counters = reinterpret_cast<int*>(base);
  w->acc64 = reinterpret_cast<unsigned long long*>(base + kScrCounters);
  w->partial = reinterpret_cast<float*>(base + kScrCounters + kScrWords);
  w->xrot = reinterpret_cast<uint16_t*>(base + kScrCounters + kScrWords + pb);
  return true;
}

}  // namespace

// =================================================================================
// C ABI
// =================================================================================
extern "C" {

const char* qg_last_error(void) { return g_err.c_str(); }

qg_status qgemv_create(qg_handle* out, const qg_weight_desc* d, int32_t max_M, void* stream) {
  g_err.clear();
  if (!out) return fail(QG_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!d) return fail(QG_ERR_INVALID_ARG, "desc is NULL");
  if (d->format == QG_FMT_MXFP4) {
    if (d->group_size != 32) return fail(QG_ERR_INVALID_ARG, "MXFP4: group_size must be 32 (got %d)", d->group_size);
    if (d->bits != 0 && d->bits != 4) return fail(QG_ERR_INVALID_ARG, "MXFP4: bits must be 0 or 4 (got %d)", d->bits);
  } else if (d->format == QG_FMT_MXFP6) {
    if (d->group_size != 32) return fail(QG_ERR_INVALID_ARG, "MXFP6: group_size must be 32 (got %d)", d->group_size);
    if (d->bits != 0 && d->bits != 6) return fail(QG_ERR_INVALID_ARG, "MXFP6: bits must be 0 or 6 (got %d)", d->bits);
  } else if (d->group_size != QG_GROUP &&
             !(d->format == QG_FMT_UNIFORM && (d->group_size == 64 || d->group_size == 32))) {
    return fail(QG_ERR_INVALID_ARG, "group_size must be 128 (uniform codes: 128, 64 or 32; got %d)", d->group_size);
  }
  if (d->K <= 0 || d->K % QG_GROUP) return fail(QG_ERR_INVALID_ARG, "K = %d is not a positive multiple of 128", d->K);
  if (d->N <= 0 || d->N % 16) return fail(QG_ERR_INVALID_ARG, "N = %d is not a positive multiple of 16", d->N);
  if (max_M < 1 || max_M > QG_MAX_M) return fail(QG_ERR_INVALID_ARG, "max_M = %d is not in [1, 32]", max_M);
  if (!d->codes || !d->scales) return fail(QG_ERR_INVALID_ARG, "codes and scales must be device pointers");
  if (!aligned16(d->codes) || !aligned16(d->scales)) return fail(QG_ERR_INVALID_ARG, "codes/scales must be 16-byte aligned");
  if (d->format != QG_FMT_UNIFORM && d->format != QG_FMT_TRELLIS3 && !mxfmt(d->format))
    return fail(QG_ERR_INVALID_ARG, "unknown format %d", d->format);
  if (d->format == QG_FMT_TRELLIS3) {
    if (!d->codebook || !aligned16(d->codebook)) return fail(QG_ERR_INVALID_ARG, "trellis needs a 16-byte aligned codebook");
  }
  if ((d->flags & QG_FLAG_BATCH_INVARIANT) && d->format == QG_FMT_TRELLIS3)
    return fail(QG_ERR_UNSUPPORTED, "batch-invariant rows are built for uniform-code handles only");
  if ((d->pins & QG_PIN_M1_PERGROUP) && (d->pins & QG_PIN_M1_RUNS))
    return fail(QG_ERR_INVALID_ARG, "pins: one M = 1 kernel at a time");
  if ((d->pins & QG_PIN_XS_T1) && (d->pins & QG_PIN_XS_T2))
    return fail(QG_ERR_INVALID_ARG, "pins: one tile-group size at a time");
  if ((d->pins & QG_PIN_PARTIALS) && (d->pins & QG_PIN_WORDS))
    return fail(QG_ERR_INVALID_ARG, "pins: one hand-over at a time");
  qg_status s = check_launch_overrides(d);
  if (s != QG_OK) return s;
  int dev = 0;
  s = check_device(&dev);
  if (s != QG_OK) return s;
  qg_plan* h = new (std::nothrow) qg_plan();
  if (!h) return fail(QG_ERR_OOM, "host allocation failed");
  h->K = d->K;
  h->N = d->N;
  h->G = d->K / QG_GROUP;
  h->G4 = (h->G + 3) / 4;
  h->format = d->format;
  h->max_M = max_M;
  h->flags = d->flags;
  h->pins = d->pins;
  h->device = dev;
  h->debug_sync = getenv("QG_DEBUG_SYNC") != nullptr;
  for (int c = 0; c < 3; ++c) {
    h->over[c].T = d->launch[c].tiles;
    h->over[c].NW = d->launch[c].waves;
    h->over[c].S = d->launch[c].splits;
  }
  if (hipDeviceGetAttribute(&h->cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || h->cus < 1) {
    delete h;
    return fail(QG_ERR_DEVICE, "cannot query the compute-unit count");
  }
  hipStream_t st = (hipStream_t)stream;
  s = d->format == QG_FMT_TRELLIS3 ? create_trellis(h, d, st) : create_uniform(h, d, st);
  if (s == QG_OK) {
    const int nc = std::max(1, h->total_tiles);
    h->ws.ncounters = (size_t)nc;
    if (hipMalloc(&h->ws.counters, nc * sizeof(int)) != hipSuccess) s = fail(QG_ERR_OOM, "counter allocation failed");
    else if (hipMemsetAsync(h->ws.counters, 0, nc * sizeof(int), st) != hipSuccess)
      s = fail(QG_ERR_DEVICE, "counter initialisation failed");
  }
  if (s == QG_OK && coded(h)) {
    if (m1_allow_lds() != hipSuccess || xs1_allow_lds() != hipSuccess || xs2_allow_lds() != hipSuccess)
      s = fail(QG_ERR_DEVICE, "cannot raise the LDS limit of the kernels");
  }
  if (hipStreamSynchronize(st) != hipSuccess && s == QG_OK) s = fail(QG_ERR_DEVICE, "stream synchronisation failed");
  if (s != QG_OK) {
    free_plan(h);
    return s;
  }
  *out = h;
  return QG_OK;
}

qg_status qgemv_destroy(qg_handle h) {
  g_err.clear();
  free_plan(h);
  return QG_OK;
}

qg_status qgemv_weight_bytes(qg_handle h, int64_t* bytes) {
  g_err.clear();
  if (!h || !bytes) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  *bytes = h->weight_bytes;
  return QG_OK;
}

qg_status qgemv_run(qg_handle h, const uint16_t* x, int32_t M, uint16_t* y, void* stream) {
  g_err.clear();
  if (!h || !x || !y) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (M < 1 || M > h->max_M) return fail(QG_ERR_INVALID_ARG, "M = %d is not in [1, %d]", M, h->max_M);
  if (!aligned16(x) || !aligned16(y)) return fail(QG_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (h->format == QG_FMT_TRELLIS3) return run_trellis(h, h->ws, x, M, y, st);
  if (M == 1 && !invariant(h)) return run_m1(h, h->ws, nullptr, x, false, y, false, st);
  return run_xs(h, h->ws, nullptr, x, nullptr, M, y, false, h->N, st);
}

qg_status qgemv_run_noalloc(qg_handle h, const uint16_t* x, int32_t M, uint16_t* y, void* stream) {
  g_err.clear();
  if (!h || !x || !y) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (M < 1 || M > h->max_M) return fail(QG_ERR_INVALID_ARG, "M = %d is not in [1, %d]", M, h->max_M);
  if (!aligned16(x) || !aligned16(y)) return fail(QG_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  int dev = -1;
  QG_HIP(hipGetDevice(&dev));
  if (dev != h->device) return fail(QG_ERR_INVALID_ARG, "the handle lives on device %d, the current one is %d", h->device, dev);
  hipStream_t st = (hipStream_t)stream;
  Work w;
  const Work need = run_need(h, M);
  if (!carve(need, 0, &w)) return QG_ERR_INVALID_ARG;  // sizes only: nothing enqueued when the run does not fit
  unsigned char* base = nullptr;
  const qg_status s = scratch_of(dev, st, &base);
  if (s != QG_OK) return s;
  carve(need, reinterpret_cast<uintptr_t>(base), &w);
  if (h->format == QG_FMT_TRELLIS3) return run_trellis(h, w, x, M, y, st);
  if (M == 1 && !invariant(h)) return run_m1(h, w, nullptr, x, false, y, false, st);
  return run_xs(h, w, nullptr, x, nullptr, M, y, false, h->N, st);
}

qg_status qgemv_run_batch(int32_t n, const qg_handle* hs, const uint16_t* const* xs, uint16_t* const* ys, int32_t M,
                          void* stream) {
  g_err.clear();
  if (n < 1 || n > GV_MAX_TASKS) return fail(QG_ERR_INVALID_ARG, "n = %d is not in [1, %d]", n, GV_MAX_TASKS);
  if (!hs || !xs || !ys) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  bool one_launch = M == 1;
  for (int i = 0; i < n; ++i) {
    if (!hs[i] || !xs[i] || !ys[i]) return fail(QG_ERR_INVALID_ARG, "NULL entry %d", i);
    if (M < 1 || M > hs[i]->max_M) return fail(QG_ERR_INVALID_ARG, "M = %d is not in [1, %d] for entry %d", M, hs[i]->max_M, i);
    if (!aligned16(xs[i]) || !aligned16(ys[i])) return fail(QG_ERR_INVALID_ARG, "x and y of entry %d must be 16-byte aligned", i);
    for (int k = 0; k < i; ++k)
      if (hs[k] == hs[i]) return fail(QG_ERR_INVALID_ARG, "entries %d and %d share a handle (and its workspace)", k, i);
    if (hs[i]->format != QG_FMT_UNIFORM || hs[i]->device != hs[0]->device || invariant(hs[i])) one_launch = false;
    // (MX-format and trellis handles run entry by entry)
  }
  hipStream_t st = (hipStream_t)stream;
  if (one_launch) return run_batch_m1(n, hs, xs, ys, st);
  for (int i = 0; i < n; ++i) {  // other formats and row counts: one launch per entry, in order
    const qg_status s = qgemv_run(hs[i], xs[i], M, ys[i], stream);
    if (s != QG_OK) return s;
  }
  return QG_OK;
}

qg_status qmlp_run(qg_handle gate, qg_handle up, qg_handle down, const uint16_t* x, int32_t M, uint16_t* out,
                   void* stream) {
  g_err.clear();
  if (!gate || !up || !down || !x || !out) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (gate->format != QG_FMT_UNIFORM || up->format != QG_FMT_UNIFORM || down->format != QG_FMT_UNIFORM)
    return fail(QG_ERR_UNSUPPORTED, "the fused MLP takes uniform-code handles");
  if (gate->K != up->K || gate->N != up->N) return fail(QG_ERR_INVALID_ARG, "gate and up shapes differ");
  if (gate->col_bits != up->col_bits) return fail(QG_ERR_INVALID_ARG, "gate and up need the same per-column widths");
  if (gate->group_size != up->group_size) return fail(QG_ERR_INVALID_ARG, "gate and up need the same scale group size");
  if (down->K != gate->N) return fail(QG_ERR_INVALID_ARG, "down K (%d) != gate N (%d)", down->K, gate->N);
  if (M < 1 || M > gate->max_M || M > down->max_M) return fail(QG_ERR_INVALID_ARG, "M = %d out of range", M);
  if (!aligned16(x) || !aligned16(out)) return fail(QG_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
  if (invariant(gate) != invariant(up) || invariant(gate) != invariant(down))
    return fail(QG_ERR_INVALID_ARG, "gate, up and down must agree on QG_FLAG_BATCH_INVARIANT");
  hipStream_t st = (hipStream_t)stream;
  if (M == 1 && !invariant(gate)) {
    const qg_status s = run_m1(gate, gate->ws, up, x, false, gate->h32, true, st);
    if (s != QG_OK) return s;
    return run_m1(down, down->ws, nullptr, gate->h32, true, out, false, st);
  }
  qg_status s = run_xs(gate, gate->ws, up, x, nullptr, M, gate->h32, true, gate->N, st);
  if (s != QG_OK) return s;
  s = after_launch(gate, launch_h_to_f16(gate->h32, gate->h16, gate->hf, M, gate->N, st), st);
  if (s != QG_OK) return s;
  return run_xs(down, down->ws, nullptr, gate->h16, gate->hf, M, out, false, down->N, st);
}

// ---- prefill route: dequantise to fp16 in column chunks, then hipBLASLt ----------
namespace {
constexpr size_t kPrefillGemmWs = (size_t)32 << 20;  // hipBLASLt workspace at the front of the caller's
}

// Rows up to which qgemv_run_prefill runs the verify GEMM in chunks of up to
// 32 rows instead of dequantising the matrix.  Measured on MI355X (both sides
// graph-timed over weight copies of 1 GiB), as (N, K) and per format class
// (uniform codes at group 128 of any width / groups of 64 or 32 / MXFP4 /
// MXFP6): the chunks win up to 128 / 96 / 64 / 64 rows on (17408, 5120),
// 224 / 160 / 128 / 96 on (5120, 17408), 64 on (5120, 5120) in every class,
// and 64 on (1024, 5120) at group 128.  A chunk costs about its codes'
// decode, dearer for the scale groups and MX elements; the route a
// dequantisation that grows with N K plus a GEMM that hipBLASLt runs slower
// on a deep K than on a wide N, so shapes of one N K cross at different row
// counts.  Elsewhere: 32 rows per 2048 of sqrt(N K), at most 256, times 3/4
// for groups of 64 or 32 and 1/2 for MX elements, rounded down to 32 rows
// (0: the route from one row).
namespace {
struct PrefillTuned {
  int N, K;
  int rows[4];  // per format class; -1: not measured (the rule above)
};
constexpr PrefillTuned kPrefillTuned[] = {{17408, 5120, {128, 96, 64, 64}},
                                          {5120, 17408, {224, 160, 128, 96}},
                                          {5120, 5120, {64, 64, 64, 64}},
                                          {1024, 5120, {64, -1, -1, -1}}};
}  // namespace

static int prefill_chunk_rows(const qg_plan* h) {
  const int f = h->format == QG_FMT_MXFP4 ? 2 : h->format == QG_FMT_MXFP6 ? 3 : (h->group_size < QG_GROUP ? 1 : 0);
  for (const PrefillTuned& t : kPrefillTuned)
    if (t.N == h->N && t.K == h->K && t.rows[f] >= 0) return t.rows[f];
  const int c = std::min(8, (int)(std::sqrt((double)h->N * (double)h->K) / 2048.0));
  const int quarters = c * (f == 0 ? 4 : f == 1 ? 3 : 2);  // in quarters of 32 rows
  return 32 * (quarters / 4);
}

qg_status qgemv_prefill_workspace(qg_handle h, size_t* min_bytes, size_t* full_bytes) {
  g_err.clear();
  if (!h || !min_bytes || !full_bytes) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (!coded(h)) return fail(QG_ERR_UNSUPPORTED, "the prefill route takes uniform-code and MX-format handles");
  const size_t row = (size_t)h->K * sizeof(uint16_t);
  *full_bytes = kPrefillGemmWs + (size_t)h->N * row;
  *min_bytes = h->segs.size() == 1 ? kPrefillGemmWs + 16 * row : *full_bytes;
  return QG_OK;
}

qg_status qgemv_run_prefill(qg_handle h, const uint16_t* x, int32_t M, uint16_t* y, void* workspace, size_t ws_bytes,
                            void* stream) {
  g_err.clear();
  if (!h || !x || !y || !workspace) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (M < 1) return fail(QG_ERR_INVALID_ARG, "M = %d is not positive", M);
  if (!aligned16(x) || !aligned16(y)) return fail(QG_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(QG_ERR_INVALID_ARG, "the workspace must be 256-byte aligned");
  size_t min_b = 0, full_b = 0;
  qg_status s = qgemv_prefill_workspace(h, &min_b, &full_b);
  if (s != QG_OK) return s;
  if (ws_bytes < min_b)
    return fail(QG_ERR_INVALID_ARG, "the prefill workspace needs at least %zu bytes (got %zu)", min_b, ws_bytes);
  int dev = -1;
  QG_HIP(hipGetDevice(&dev));
  if (dev != h->device) return fail(QG_ERR_INVALID_ARG, "the handle lives on device %d, the current one is %d", h->device, dev);
  hipStream_t st = (hipStream_t)stream;
  // below the crossover: the verify GEMM, 32 rows (or the handle's max_M of at
  // least 16) at a time, on the handle's own workspace; the caller's is unused
  const int cm = std::min(32, h->max_M);
  if (cm >= 16 && M <= prefill_chunk_rows(h)) {
    for (int r0 = 0; r0 < M; r0 += cm) {
      const int m = std::min(cm, M - r0);
      const uint16_t* xr = x + (size_t)r0 * h->K;
      uint16_t* yr = y + (size_t)r0 * h->N;
      const qg_status r = (m == 1 && !invariant(h)) ? run_m1(h, h->ws, nullptr, xr, false, yr, false, st)
                                                   : run_xs(h, h->ws, nullptr, xr, nullptr, m, yr, false, h->N, st);
      if (r != QG_OK) return r;
    }
    return QG_OK;
  }
  const size_t row = (size_t)h->K * sizeof(uint16_t);
  const int nc = (int)std::min<size_t>((size_t)h->N, (ws_bytes - kPrefillGemmWs) / row) / 16 * 16;
  uint16_t* wbuf = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + kPrefillGemmWs);
  for (int n0 = 0; n0 < h->N; n0 += nc) {
    const int n1 = std::min(h->N, n0 + nc);
    if (h->segs.size() == 1) {  // one width: column n is tile n / 16, lane n % 16
      const HostSeg& g = h->segs[0];
      const SegDev sd{g.codes, g.scales, g.bits, g.tiles, g.tile0, g.sq, g.mx};
      QG_HIP(launch_dequant_f16(sd, h->col_map, h->G, h->G4, h->K, n0 / 16, (n1 - n0) / 16, n0, n1, wbuf, st));
    } else {  // several widths (one chunk): every segment's columns land at their own rows
      for (const auto& g : h->segs) {
        const SegDev sd{g.codes, g.scales, g.bits, g.tiles, g.tile0, g.sq, g.mx};
        QG_HIP(launch_dequant_f16(sd, h->col_map, h->G, h->G4, h->K, 0, g.tiles, n0, n1, wbuf, st));
      }
    }
    const char* err = nullptr;
    if (gemm_f16_wxt(dev, wbuf, n1 - n0, x, M, h->K, y + n0, h->N, workspace, kPrefillGemmWs, st, &err) != 0)
      return fail(QG_ERR_DEVICE, "prefill GEMM (%d x %d x %d): %s", M, n1 - n0, h->K, err);
  }
  if (h->debug_sync) {
    const hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "prefill failed: %s", hipGetErrorString(e));
  }
  return QG_OK;
}

qg_status qg_stream_read(const void* buf, int64_t bytes, void* stream) {
  g_err.clear();
  if (!buf || bytes <= 0 || bytes % 16 || !aligned16(buf))
    return fail(QG_ERR_INVALID_ARG, "stream read needs a 16-byte aligned buffer and a positive multiple of 16 bytes");
  int dev = 0, cus = 0;
  QG_HIP(hipGetDevice(&dev));
  QG_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  QG_HIP(launch_stream_read(buf, bytes, nullptr, std::max(cus, 1), (hipStream_t)stream));
  return QG_OK;
}

qg_status qgemv_debug_unpack(qg_handle h, int32_t* codes, void* stream) {
  g_err.clear();
  if (!h || !codes) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (!coded(h)) return fail(QG_ERR_INVALID_ARG, "debug_unpack takes a uniform-code or MX-format handle");
  for (const auto& s : h->segs) {
    const SegDev sd{s.codes, s.scales, s.bits, s.tiles, s.tile0, s.sq, s.mx};
    QG_HIP(launch_debug_uniform(sd, h->col_map, h->G, h->G4, h->K, 0, codes, nullptr, nullptr, (hipStream_t)stream));
  }
  return QG_OK;
}

qg_status qgemv_debug_dequant(qg_handle h, float* w, uint16_t* q16, void* stream) {
  g_err.clear();
  if (!h || !w) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  hipStream_t st = (hipStream_t)stream;
  if (h->format == QG_FMT_TRELLIS3) {
    QG_HIP(launch_debug_trellis(h->tcodes, h->tscales, h->codebook, h->K, h->G, h->tr_units, nullptr, w, st));
    return QG_OK;
  }
  for (const auto& s : h->segs) {
    const SegDev sd{s.codes, s.scales, s.bits, s.tiles, s.tile0, s.sq, s.mx};
    QG_HIP(launch_debug_uniform(sd, h->col_map, h->G, h->G4, h->K, 0, nullptr, w, q16, st));
  }
  return QG_OK;
}

qg_status qgemv_debug_operand(qg_handle h, int32_t* codes, uint16_t* b16, float* w, void* stream) {
  g_err.clear();
  if (!h || (!codes && !b16 && !w)) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (!coded(h)) return fail(QG_ERR_INVALID_ARG, "debug_operand takes a uniform-code or MX-format handle");
  for (const auto& s : h->segs) {
    const SegDev sd{s.codes, s.scales, s.bits, s.tiles, s.tile0, s.sq, s.mx};
    QG_HIP(launch_debug_uniform(sd, h->col_map, h->G, h->G4, h->K, 1, codes, w, b16, (hipStream_t)stream));
  }
  return QG_OK;
}

qg_status qgemv_debug_trellis(qg_handle h, uint16_t* states, void* stream) {
  g_err.clear();
  if (!h || !states) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (h->format != QG_FMT_TRELLIS3) return fail(QG_ERR_INVALID_ARG, "debug_trellis takes a trellis handle");
  QG_HIP(launch_debug_trellis(h->tcodes, h->tscales, h->codebook, h->K, h->G, h->tr_units, states, nullptr,
                              (hipStream_t)stream));
  return QG_OK;
}

}  // extern "C"
