// qgemv.hip -- host side of the C ABI declared in include/qgemv.h: descriptor
// validation, device check, weight re-layout into handle-owned memory, launch
// planning per (shape, row count) and dispatch onto the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/qgemv.h"
#include "qg_kernels.h"
#include "qg_trellis.h"
#include "qg_stream.h"
#include "qg_gemm.h"
#include "qg_xs.h"

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
  int NQ = 0;                // M = 1: quads per wave (derived)
};

// quads-per-wave counts the M = 1 kernel is compiled for
constexpr int kNQ[] = {1, 2, 3, 4, 5};
int nq_round_up(int nq) {
  for (int v : kNQ)
    if (v >= nq) return v;
  return 0;
}

struct HostSeg {
  int bits, tiles, tile0, ncols;
  uint32_t* codes = nullptr;
  uint16_t* scales = nullptr;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int mclass(int M) { return M <= 1 ? 0 : (M <= 16 ? 1 : 2); }

}  // namespace

struct qg_plan {
  int K = 0, N = 0, G = 0, G4 = 0, format = 0, max_M = 0;
  uint32_t flags = 0;
  int device = 0;
  std::vector<HostSeg> segs;
  std::vector<uint8_t> col_bits;  // host copy (uniform: per column)
  int total_tiles = 0;
  int32_t* col_map = nullptr;     // device [16*total_tiles]
  int64_t weight_bytes = 0;
  float* partial = nullptr;       // device workspace
  size_t partial_floats = 0;
  int* counters = nullptr;        // device [total_tiles] split-K arrival counters, zero between runs
  uint16_t* hbuf = nullptr;       // device [max_M][N] fp16, MLP intermediate
  unsigned long long* acc64 = nullptr;  // device [2][max_M][16*total_tiles] fixed-point output words, zero between runs
  int cus = 0;                    // compute units of the device
  Launch over[3];
  // trellis
  uint32_t* tcodes = nullptr;     // device layout of trellis tiles
  uint16_t* tscales = nullptr;    // [N/16 tiles][G][16]
  uint16_t* codebook = nullptr;   // device copy, 65536 fp16
  uint16_t* xrot = nullptr;       // device [max_M][K] fp16, rotated activations
  int64_t tr_units = 0;           // (N/16) * G
  int tr_grid = 0, tr_maxseg = 0;
  bool tr_fx = false;             // M = 1 trellis GEMV hands row blocks on through fixed-point words (acc64)
};

namespace {

// ---- launch planning --------------------------------------------------------
// verify GEMM kernels: the per-wave-K-split kernel (k_gemm_mfma), the shared-x
// kernel (k_gemm_v2) and the x-in-LDS streaming kernel (k_gemm_xs).
// QG_GEMM=mfma (or v1)|v2|xs forces one.
enum { GEMM_MFMA = 0, GEMM_V2 = 1, GEMM_XS = 2 };
int gemm_forced() {
  const char* f = getenv("QG_GEMM");
  if (f && (!strcmp(f, "mfma") || !strcmp(f, "v1"))) return GEMM_MFMA;
  if (f && !strcmp(f, "v2")) return GEMM_V2;
  if (f && !strcmp(f, "xs")) return GEMM_XS;
  return -1;
}
bool gemm_v2_on() { return gemm_forced() == GEMM_V2; }

// Launch shapes of the per-wave-K-split GEMM measured best on MI355X (sweeps
// over tiles per wave T, waves per workgroup NW and K slices S) for the
// 27B-class layer shapes; other shapes use the generic rule in choose().
struct TunedLaunch {
  int N, K, mcls, T, NW, S;
};
constexpr TunedLaunch kTuned[] = {
    {5120, 5120, 1, 2, 4, 1},  {5120, 5120, 2, 2, 4, 1},   // q, o
    {1024, 5120, 1, 1, 4, 1},  {1024, 5120, 2, 2, 8, 5},   // k, v
    {17408, 5120, 1, 2, 2, 1}, {17408, 5120, 2, 4, 4, 1},  // gate, up
    {5120, 17408, 1, 2, 8, 1}, {5120, 17408, 2, 4, 4, 3},  // down
};

Launch choose(const qg_plan* h, int M, bool dual = false, int force_v2 = -1) {
  Launch L = h->over[mclass(M)];
  const int G = h->G;
  if (h->format == QG_FMT_TRELLIS3) {
    if (L.T <= 0) L.T = 1;
    if (L.NW <= 0) L.NW = 4;
    if (L.S <= 0) L.S = 1;
    return L;
  }
  // waves per workgroup split K; pick the most that keep every workgroup of the
  // grid resident at once (no second round) and give each wave >= 2 groups
  auto pick_nw = [&](int tilesets, int budget) {
    int nw = 8;
    while (nw > 1 && ((int64_t)tilesets * nw > budget || G / nw < 2)) nw /= 2;
    return nw;
  };
  if (M == 1) {
    // one tile per workgroup; NW waves of NQ quads each split the K slice.  Measured
    // on the decode shapes: 2 quads per wave is fastest, then 3, then 1 (more quads
    // per wave lengthen the serial load-to-use chain, fewer add per-wave fixed
    // cost); take the first of that order that fits in 16 waves with <= 1/8 dead
    // quads (fused gate/up: at most 2 quads per wave for register room)
    L.T = 1;
    const int G4 = h->G4;
    // K slices (one matrix; measured): up to K = 8192 and 1024 tiles, of
    // about 2 quads (a one-wave workgroup per slice: q/o 6.4 us against 7.0 in
    // one slice, q|k|v stacked 7.1 against 7.2; wider matrices gain nothing:
    // gate/up 10.4-10.9 either way, gate|up stacked 16.7 in one slice against
    // 16.9-18.8); beyond K = 8192 of about 7 quads (down: 10.6-10.8 against
    // 14.7 in one slice; with 2- and 3-bit columns 11.8 against 12.9 in 4)
    if (L.S <= 0) L.S = dual ? 1 : (G4 > 16 ? (G4 + 6) / 8 : (h->total_tiles <= 1024 ? (G4 + 1) / 2 : 1));
    L.S = std::min(L.S, G4);
    const int g4s = (G4 + L.S - 1) / L.S;
    if (L.NW <= 0) {
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
      L.NW = best_nw;
      L.NQ = nq_round_up(best_nq);
    } else {
      L.NQ = nq_round_up((g4s + L.NW - 1) / L.NW);
    }
    return L;
  } else if (force_v2 < 0 ? gemm_v2_on() : force_v2 != 0) {
    // verify GEMM: K slices of at most QMAX quads; T tiles per wave and NW
    // waves per workgroup as wide as keeps >= 2 workgroups per compute unit
    const int qmax = M <= 16 ? 4 : 2;
    const int smin = (h->G4 + qmax - 1) / qmax;
    L.S = std::min(std::max(L.S, smin), h->G4);
    const int want = std::max(1, h->cus);
    auto wgs = [&](int T, int NW) {
      int n = 0;
      for (const auto& sg : h->segs) n += (sg.tiles + T * NW - 1) / (T * NW);
      return (int64_t)n * L.S;
    };
    if (L.T <= 0) {
      L.T = 2;
      if (wgs(2, 8) < want) L.T = 1;
    }
    L.T = L.T >= 4 ? 4 : (L.T >= 2 ? 2 : 1);
    L.T = std::min(L.T, M <= 16 ? (dual ? 1 : 2) : (dual ? 2 : 4));  // compiled tile counts
    if (L.NW <= 0) L.NW = 8;
    L.NW = L.NW >= 8 ? 8 : 4;  // the x staging takes at least 4 waves
    return L;
  } else {
    if (L.T <= 0 && L.NW <= 0 && L.S <= 0 && !dual) {
      for (const TunedLaunch& t : kTuned)
        if (t.N == h->N && t.K == h->K && t.mcls == mclass(M)) {
          L.T = t.T;
          L.NW = t.NW;
          L.S = t.S;
        }
    }
    if (L.T <= 0) L.T = 2;
    const int tilesets = (h->total_tiles + L.T - 1) / L.T;
    if (L.NW <= 0) L.NW = pick_nw(tilesets, 1800);
    if (L.S <= 0) L.S = 1;
  }
  L.S = std::min(L.S, G);
  return L;
}

constexpr size_t kLdsMax = 163840;  // LDS per workgroup on gfx950
constexpr int kXsNQ = 8;            // longest K slice of the x-in-LDS GEMM, in quads
// slice lengths the x-in-LDS GEMM is compiled for (the smallest >= the longest slice runs)
constexpr int kXsNQs[] = {4, 5, 8};

// Plan of the x-in-LDS GEMM (k_gemm_xs): K slices S (as few as let the slice of
// x fit LDS), T tiles per group (2; 1 gate + 1 up tile in the fused pass) and
// GPW tile groups per workgroup, one per wave, at most 8 (about one workgroup
// per LDS slot of the chip).  Overrides for M > 1 (qgemv_set_launch): tiles (or
// waves) = tile groups per workgroup, splits = K slices (at least as many as
// the LDS needs).
struct XsPlan {
  int MT = 1, T = 2, S = 1, nq = 1, NQ = 4, GPW = 1, NW = 1;
  bool fx = false;  // K slices meet in fixed-point words (else fp32 partials)
  size_t lds = 0;
  unsigned grid = 0;
  int wg_prefix[MAX_SEG + 1] = {};
  int tg_prefix[MAX_SEG + 1] = {};
};

int xs_nq_compiled(int nq) {
  for (int v : kXsNQs)
    if (v >= nq) return v;
  return 0;
}

// Launch shapes of the x-in-LDS GEMM measured best on MI355X (sweeps over tile
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

// Verify GEMM kind: the x-in-LDS kernel (measured fastest on every decode
// shape once its tile groups may hold one tile); QG_GEMM forces one.
int gemm_kind(const qg_plan* h, int M) {
  (void)h;
  (void)M;
  const int f = gemm_forced();
  if (f >= 0) return f;
  return GEMM_XS;
}

XsPlan xs_plan(const qg_plan* h, int M, bool dual) {
  XsPlan p;
  Launch L = h->over[mclass(M)];
  // one-tile groups (twice the waves) measured faster except for wide
  // matrices at more than 16 rows
  int tuned_T = (M <= 16 || h->total_tiles <= 512) ? 1 : 2;
  if (!dual)
    for (const XsTuned& t : kXsTuned)
      if (t.N == h->N && t.K == h->K && t.mcls == mclass(M)) {
        tuned_T = t.T;
        if (L.T <= 0 && L.NW <= 0 && L.S <= 0) {
          L.T = t.GPW;
          L.S = t.S;
        }
      }
  p.MT = M <= 16 ? 1 : 2;
  // tiles per tile group: 1 for the fused gate/up pair; else the tuned count
  // (QG_XS_T=1|2 forces one)
  p.T = dual ? 1 : tuned_T;
  if (!dual) {
    const char* ft = getenv("QG_XS_T");
    if (ft && (atoi(ft) == 1 || atoi(ft) == 2)) p.T = atoi(ft);
  }
  const size_t col_cap = 4096;  // room for the run's column map
  // fewest K slices whose x slice fits LDS (at the compiled slice length)
  p.S = std::max(1, std::min(h->G4, L.S > 0 ? L.S : 1));
  for (;; ++p.S) {
    p.nq = (h->G4 + p.S - 1) / p.S;
    p.NQ = xs_nq_compiled(p.nq);
    if (p.NQ > 0 && xs_x_bytes(M, p.NQ) + xs_sum_bytes(p.MT, p.NQ) + col_cap <= kLdsMax) break;
    if (p.S >= h->G4) break;
  }
  int tg = 0;
  for (const auto& sg : h->segs) tg += (sg.tiles + p.T - 1) / p.T;
  const size_t lds0 = xs_x_bytes(M, p.NQ) + xs_sum_bytes(p.MT, p.NQ) + 1024;
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
  p.lds = xs_lds_bytes(M, p.MT, p.NQ, p.GPW, p.T);
  // fixed-point words while the atomics stay few (measured: they win at 8 rows
  // on every decode shape, the partials at 32 rows on the widest); <= 63 slices
  // fixed-point words when the atomics are few, or when many slices would make
  // the last one read its partials in several round trips (measured: down at
  // 24-32 rows, 9 slices, gains; gate/up, 3 slices, loses)
  const int64_t atomics = (int64_t)M * 16 * h->total_tiles * p.S;
  p.fx = p.S > 1 && p.S <= 63 && (atomics <= (int64_t)1 << 20 || (p.S >= 6 && atomics <= (int64_t)1 << 22));
  const char* fh = getenv("QG_XS_HANDOVER");  // =partials | =words forces one
  if (fh && !strcmp(fh, "partials")) p.fx = false;
  if (fh && !strcmp(fh, "words")) p.fx = p.S > 1 && p.S <= 63;
  return p;
}

size_t partial_need(const qg_plan* h, int S, int M) {
  return S <= 1 ? 0 : (size_t)2 * S * M * (size_t)(16 * h->total_tiles);
}

// M = 1 fused gate/up pass with one matrix per workgroup (partials of both
// matrices, even with one K slice); QG_M1_PAIR=0 keeps both matrices in each
// workgroup
bool m1_pair_on() {
  const char* f = getenv("QG_M1_PAIR");
  return !(f && !strcmp(f, "0"));
}
size_t pair_need(const qg_plan* h, int S) { return (size_t)2 * std::max(S, 1) * (size_t)(16 * h->total_tiles); }

qg_status ensure_workspace(qg_plan* h) {
  size_t need = 0;
  for (int c = 0; c < 3; ++c) {
    const int Mc = c == 0 ? 1 : (c == 1 ? 16 : 32);
    if (Mc > h->max_M && c > 0 && (c == 1 ? 2 : 17) > h->max_M) continue;
    const int Mm = std::min(Mc, h->max_M);
    if (c == 0) need = std::max(need, pair_need(h, choose(h, 1, true).S));
    // any verify GEMM may be selected at run time: size for all
    for (int v2 = 0; v2 < 2; ++v2) {
      need = std::max(need, partial_need(h, choose(h, Mm, false, v2).S, Mm));
      need = std::max(need, partial_need(h, choose(h, Mm, true, v2).S, Mm));
    }
    for (int Mx = 2; Mx <= Mm; ++Mx) {
      need = std::max(need, partial_need(h, xs_plan(h, Mx, false).S, Mx));
      need = std::max(need, partial_need(h, xs_plan(h, Mx, true).S, Mx));
    }
  }
  if (need > h->partial_floats) {
    if (h->partial) hipFree(h->partial);
    h->partial = nullptr;
    h->partial_floats = 0;
    if (hipMalloc(&h->partial, need * sizeof(float)) != hipSuccess)
      return fail(QG_ERR_OOM, "workspace allocation of %zu bytes failed", need * sizeof(float));
    h->partial_floats = need;
  }
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
  if (h->col_map) hipFree(h->col_map);
  if (h->partial) hipFree(h->partial);
  if (h->counters) hipFree(h->counters);
  if (h->hbuf) hipFree(h->hbuf);
  if (h->acc64) hipFree(h->acc64);
  if (h->tcodes) hipFree(h->tcodes);
  if (h->tscales) hipFree(h->tscales);
  if (h->codebook) hipFree(h->codebook);
  if (h->xrot) hipFree(h->xrot);
  delete h;
}

WSet wset_of(const qg_plan* h) {
  WSet w{};
  w.nseg = (int)h->segs.size();
  for (int i = 0; i < w.nseg; ++i) {
    const HostSeg& s = h->segs[i];
    w.seg[i] = SegDev{s.codes, s.scales, s.bits, s.tiles, s.tile0};
  }
  w.col_map = h->col_map;
  return w;
}


// ---- trellis ---------------------------------------------------------------------
// stream-K plan: W = grid * NW waves share the U = (N/16) * G units; maxseg is
// the largest number of waves any row block is split over (the device kernel
// finds the same first and last wave of a row block with tr_wave_of)
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

bool trellis_banded_on(int M) {
  const char* f = getenv("QG_TRELLIS");
  if (f && !strcmp(f, "stream")) return false;
  return M > 1;
}

qg_status create_trellis(qg_plan* h, const qg_weight_desc* d, hipStream_t st) {
  const int N = d->N, K = d->K, G = K / QG_GROUP, RB = N / 16;
  int cus = 0;
  QG_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device));
  h->total_tiles = RB;
  h->tr_units = (int64_t)RB * G;
  h->weight_bytes = (int64_t)N * K * 3 / 8 + (int64_t)N * G * 2;
  // one workgroup per compute unit (the codebook fills its LDS) of 16 waves (8
  // for more than 16 rows); the codebook gathers bound the kernel, so small
  // matrices still spread over as many compute units as they have 16 units for
  h->tr_grid = (int)std::max<int64_t>(1, std::min<int64_t>(cus, (h->tr_units + 15) / 16));
  h->tr_maxseg = 1;
  for (int nw : {8, 16}) {
    const int W = (int)std::min<int64_t>((int64_t)h->tr_grid * nw, h->tr_units);
    h->tr_maxseg = std::max(h->tr_maxseg, tr_maxseg_of(RB, G, h->tr_units, W));
  }
  // the M = 1 GEMV's row blocks meet in fixed-point words (one round trip)
  // where at most 63 waves share one (the words count arrivals in 6 bits)
  h->tr_fx = tr_maxseg_of(RB, G, h->tr_units, (int)std::min<int64_t>((int64_t)h->tr_grid * 16, h->tr_units)) <= 63;
  h->tr_maxseg = std::max({h->tr_maxseg, tb_slices(h, TbShape<1>::NW), tb_slices(h, TbShape<2>::NW)});
  const size_t ncode = (size_t)h->tr_units * 64 * 3;
  QG_HIP(hipMalloc(&h->tcodes, ncode * sizeof(uint32_t)));
  QG_HIP(hipMalloc(&h->tscales, (size_t)h->tr_units * 16 * sizeof(uint16_t)));
  QG_HIP(hipMalloc(&h->codebook, 65536 * sizeof(uint16_t)));
  if (!(d->flags & QG_FLAG_X_PREROTATED)) QG_HIP(hipMalloc(&h->xrot, (size_t)h->max_M * K * sizeof(uint16_t)));
  const size_t nf = (size_t)RB * h->tr_maxseg * h->max_M * 16;
  QG_HIP(hipMalloc(&h->partial, nf * sizeof(float)));
  h->partial_floats = nf;
  // fixed-point output words [max_M][N] of the M = 1 GEMV and the banded GEMM, zero between runs
  QG_HIP(hipMalloc(&h->acc64, (size_t)h->max_M * N * sizeof(unsigned long long)));
  QG_HIP(hipMemsetAsync(h->acc64, 0, (size_t)h->max_M * N * sizeof(unsigned long long), st));
  QG_HIP(hipMemcpyAsync(h->codebook, d->codebook, 65536 * sizeof(uint16_t), hipMemcpyDeviceToDevice, st));
  const int64_t threads = h->tr_units * 64;
  k_repack_trellis<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>((const uint16_t*)d->codes, d->scales, K / 16, G,
                                                                      h->tr_units, h->tcodes, h->tscales);
  QG_HIP(hipGetLastError());
  QG_HIP(hipStreamSynchronize(st));
  return QG_OK;
}

// M = 1 GEMV that rotates x itself into LDS (no separate rotation launch):
// room for the rotated x beside the codebook up to K = 16384
bool trellis_xl(const qg_plan* h, int M) {
  const char* f = getenv("QG_TRELLIS_ROT");  // =launch: the separate rotation kernel
  if (f && !strcmp(f, "launch")) return false;
  return M == 1 && !(h->flags & QG_FLAG_X_PREROTATED) && (size_t)h->K * 2 <= (size_t)TR_XL_BYTES &&
         h->G <= TR_XL_GMAX * TrShape<0>::NWMAX;
}

qg_status run_trellis(const qg_plan* h, const uint16_t* x, int M, uint16_t* y, hipStream_t st) {
  const uint16_t* xr = x;
  const bool xl = trellis_xl(h, M);
  if (!(h->flags & QG_FLAG_X_PREROTATED) && !xl) {
    const int waves = M * h->G;
    k_fwht<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(x, h->xrot, M, h->K);
    xr = h->xrot;
  }
  if (trellis_banded_on(M)) {
    const bool m32 = M > 16;
    const int nw = m32 ? TbShape<2>::NW : TbShape<1>::NW;
    TbArgs b{};
    b.codes = h->tcodes;
    b.scales = h->tscales;
    b.cb = h->codebook;
    b.x = xr;
    b.y = y;
    b.partial = h->partial;
    b.counters = h->counters;
    b.M = M;
    b.K = h->K;
    b.N = h->N;
    b.G = h->G;
    b.RB = h->N / 16;
    b.maxseg = h->tr_maxseg;
    b.S = tb_slices(h, nw);
    if (b.S > h->tr_maxseg) return fail(QG_ERR_INVALID_ARG, "%d K slices exceed the workspace's %d", b.S, h->tr_maxseg);
    // K slices meet in fixed-point words where the atomics are few (and the
    // words' 6-bit count holds S); QG_TRELLIS_HANDOVER=partials forces the partials
    const char* fh = getenv("QG_TRELLIS_HANDOVER");
    const bool fx = b.S > 1 && b.S <= 63 && (int64_t)M * h->N * b.S <= (1 << 20) && !(fh && !strcmp(fh, "partials"));
    b.acc = fx ? h->acc64 : nullptr;
    const unsigned grid = (unsigned)(((b.RB + nw - 1) / nw) * b.S);
    if (m32) k_trellis_band<2><<<grid, 64 * nw, 0, st>>>(b);
    else k_trellis_band<1><<<grid, 64 * nw, 0, st>>>(b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    if (getenv("QG_DEBUG_SYNC")) {
      e = hipStreamSynchronize(st);
      if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel failed: %s", hipGetErrorString(e));
    }
    return QG_OK;
  }
  TrArgs a{};
  a.codes = h->tcodes;
  a.scales = h->tscales;
  a.cb = h->codebook;
  a.x = xr;
  a.y = y;
  a.partial = h->partial;
  a.counters = h->counters;
  a.M = M;
  a.K = h->K;
  a.N = h->N;
  a.G = h->G;
  a.RB = h->N / 16;
  a.maxseg = h->tr_maxseg;
  const int nw = M > 16 ? TrShape<2>::NWMAX : TrShape<0>::NWMAX;
  a.W = (int)std::min<int64_t>((int64_t)h->tr_grid * nw, h->tr_units);  // every wave's range non-empty
  a.U = h->tr_units;
  const dim3 grid((unsigned)h->tr_grid), block((unsigned)(64 * nw));
  if (M == 1) {
    const char* f = getenv("QG_TRELLIS_HANDOVER");  // =partials: the hand-over through partials and a count
    a.acc = h->tr_fx && !(f && !strcmp(f, "partials")) ? h->acc64 : nullptr;
    if (xl) k_trellis<0, true><<<grid, block, 0, st>>>(a);  // a.x: the unrotated x
    else k_trellis<0><<<grid, block, 0, st>>>(a);
  } else if (M <= 16) {
    k_trellis<1><<<grid, block, 0, st>>>(a);
  } else {
    k_trellis<2><<<grid, block, 0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  if (getenv("QG_DEBUG_SYNC")) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel failed: %s", hipGetErrorString(e));
  }
  return QG_OK;
}

qg_status debug_trellis(const qg_plan* h, uint16_t* states, float* w, hipStream_t st) {
  const int64_t threads = h->tr_units * 64;
  k_debug_trellis<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(h->tcodes, h->tscales, h->codebook, h->K, h->G,
                                                                     h->tr_units, states, w);
  QG_HIP(hipGetLastError());
  return QG_OK;
}

// ---- uniform create -----------------------------------------------------------
qg_status create_uniform(qg_plan* h, const qg_weight_desc* d, hipStream_t st) {
  const int N = d->N, K = d->K, G = K / QG_GROUP, G4 = (G + 3) / 4;
  h->col_bits.resize(N);
  if (d->bits == 0) {
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
  h->weight_bytes = acc * 4 + (int64_t)N * G * 2;
  // widest codes first: their workgroups (the longest) are dispatched first,
  // so the tail of a launch is the lighter widths'
  int tile0 = 0;
  for (int b = 4; b >= 2; --b) {
    std::vector<int32_t> cols;
    for (int n = 0; n < N; ++n)
      if (h->col_bits[n] == b) cols.push_back(n);
    if (cols.empty()) continue;
    HostSeg s;
    s.bits = b;
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
        hipMalloc(&s.scales, nslot * sizeof(uint16_t)) != hipSuccess) {
      hipFree(d_off);
      return fail(QG_ERR_OOM, "device allocation for the weight layout failed");
    }
    const int threads = 256;
    const unsigned blocks = (unsigned)((nslot + threads - 1) / threads);
    k_repack_uniform<<<blocks, threads, 0, st>>>((const uint32_t*)d->codes, d_off, d->scales,
                                                 h->col_map + 16 * s.tile0, s.bits, s.tiles, G, G4, s.codes,
                                                 s.scales);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  hipFree(d_off);
  if (e != hipSuccess) return fail(QG_ERR_DEVICE, "weight re-layout failed: %s", hipGetErrorString(e));
  return QG_OK;
}

// ---- dispatch ------------------------------------------------------------------
// BF = the single code width of the handle (kernels compiled for it alone) or 0
// (per-column widths: the kernel branches per segment).
template <int NQ, int BF>
void launch_q_b(const RunArgs& a, int NW, size_t lds, unsigned grid, bool dual, hipStream_t st) {
  if constexpr (NQ <= 2) {
    if (dual) {
      k_gemv_q<NQ, true, BF><<<grid, NW * 64, lds, st>>>(a);
      return;
    }
  }
  k_gemv_q<NQ, false, BF><<<grid, NW * 64, lds, st>>>(a);
}

template <int NQ>
void launch_q(const RunArgs& a, int NW, size_t lds, unsigned grid, bool dual, int bf, hipStream_t st) {
  switch (bf) {
    case 2: launch_q_b<NQ, 2>(a, NW, lds, grid, dual, st); break;
    case 3: launch_q_b<NQ, 3>(a, NW, lds, grid, dual, st); break;
    case 4: launch_q_b<NQ, 4>(a, NW, lds, grid, dual, st); break;
    default: launch_q_b<NQ, 0>(a, NW, lds, grid, dual, st); break;
  }
}

template <int T, int MT, int BF>
void launch_mfma_b(const RunArgs& a, int NW, size_t lds, unsigned grid, bool dual, hipStream_t st) {
  if constexpr (T <= 2) {
    if (dual) {
      k_gemm_mfma<T, MT, true, BF><<<grid, NW * 64, lds, st>>>(a);
      return;
    }
  }
  k_gemm_mfma<T, MT, false, BF><<<grid, NW * 64, lds, st>>>(a);
}

template <int T, int MT>
void launch_mfma_t(const RunArgs& a, int NW, size_t lds, unsigned grid, bool dual, int bf, hipStream_t st) {
  switch (bf) {
    case 2: launch_mfma_b<T, MT, 2>(a, NW, lds, grid, dual, st); break;
    case 3: launch_mfma_b<T, MT, 3>(a, NW, lds, grid, dual, st); break;
    case 4: launch_mfma_b<T, MT, 4>(a, NW, lds, grid, dual, st); break;
    default: launch_mfma_b<T, MT, 0>(a, NW, lds, grid, dual, st); break;
  }
}

template <int MT>
void launch_mfma(const RunArgs& a, int T, int NW, size_t lds, unsigned grid, bool dual, int bf, hipStream_t st) {
  switch (T) {
    case 1: launch_mfma_t<1, MT>(a, NW, lds, grid, dual, bf, st); break;
    case 2: launch_mfma_t<2, MT>(a, NW, lds, grid, dual, bf, st); break;
    default: launch_mfma_t<4, MT>(a, NW, lds, grid, dual, bf, st); break;
  }
}

// M = 1 stream-K GEMV.  Launch knobs (M = 1 overrides): NW waves per workgroup
// (default 8), S workgroups per compute unit (default 2).
bool sk_fits(const qg_plan* h) { return h->G4 <= 63 && sk_lds_bytes(h->G4) <= kLdsMax; }

template <int BF, int ND>
hipError_t sk_allow_lds() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_sk<BF, ND>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
}

// let the stream-K GEMV take more than 64 KiB of dynamic LDS (wide x, several widths)
hipError_t sk_allow_lds_all() {
  hipError_t e = hipSuccess;
  const hipError_t r[] = {sk_allow_lds<0, 1>(), sk_allow_lds<0, 2>(), sk_allow_lds<2, 1>(), sk_allow_lds<2, 2>(),
                          sk_allow_lds<3, 1>(), sk_allow_lds<3, 2>(), sk_allow_lds<4, 1>(), sk_allow_lds<4, 2>()};
  for (hipError_t x : r)
    if (x != hipSuccess) e = x;
  return e;
}

template <int BF>
void launch_sk_b(const SkArgs& a, bool dual, unsigned grid, int NW, size_t lds, hipStream_t st) {
  if (dual) k_gemv_sk<BF, 2><<<grid, NW * 64, lds, st>>>(a);
  else k_gemv_sk<BF, 1><<<grid, NW * 64, lds, st>>>(a);
}

qg_status run_sk(const qg_plan* h, const qg_plan* h2, const uint16_t* x, uint16_t* y, hipStream_t st) {
  const Launch& L = h->over[0];
  // measured on the decode shapes: 4 waves per workgroup (8 for K >= 16384), and
  // enough waves per tile for about 25 / 16 waves per SIMD over the whole chip
  const int NW = std::max(L.NW > 0 ? std::min(L.NW, 8) : (h->G4 >= 32 ? 8 : 4), (h->G4 + SK_XR - 1) / SK_XR);
  const int nch_min = (h->G4 + SK_UPW - 1) / SK_UPW;
  const int nch_want = L.T > 0 ? L.T : (int)((25LL * h->cus / 4 + h->total_tiles - 1) / h->total_tiles);
  const int nch = std::max(nch_min, std::min(nch_want, std::min(h->G4, 63)));
  SkArgs a{};
  a.w[0] = wset_of(h);
  if (h2) a.w[1] = wset_of(h2);
  a.x = x;
  a.y = y;
  a.acc = h->acc64;
  a.K = h->K;
  a.N = h->N;
  a.G = h->G;
  a.G4 = h->G4;
  a.total_tiles = h->total_tiles;
  a.U = (int64_t)h->total_tiles * h->G4;
  a.nch = nch;  // waves per tile
  // one segment per workgroup: each segment's waves are rounded up to whole workgroups
  int wgs = 0;
  for (int i = 0; i < (int)h->segs.size(); ++i) {
    a.wg_prefix[i] = wgs;
    wgs += (int)(((int64_t)h->segs[i].tiles * nch + NW - 1) / NW);
  }
  for (int i = (int)h->segs.size(); i <= MAX_SEG; ++i) a.wg_prefix[i] = wgs;
  const unsigned grid = (unsigned)wgs;
  const size_t lds = sk_lds_bytes(h->G4);
  const int bf = h->segs.size() == 1 ? h->segs[0].bits : 0;
  switch (bf) {
    case 2: launch_sk_b<2>(a, h2 != nullptr, grid, NW, lds, st); break;
    case 3: launch_sk_b<3>(a, h2 != nullptr, grid, NW, lds, st); break;
    case 4: launch_sk_b<4>(a, h2 != nullptr, grid, NW, lds, st); break;
    default: launch_sk_b<0>(a, h2 != nullptr, grid, NW, lds, st); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  if (getenv("QG_DEBUG_SYNC")) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel failed: %s", hipGetErrorString(e));
  }
  return QG_OK;
}

// M = 1 kernel choice, measured on the decode shapes: the per-group kernel
// (k_gemv_q, in K slices that meet in fixed-point words) from 256 tiles up,
// the per-tile-run kernel (run_sk) for narrower matrices.
// QG_M1_KERNEL=pergroup|runs forces one.
bool use_sk(const qg_plan* h) {
  if (!sk_fits(h)) return false;
  const char* f = getenv("QG_M1_KERNEL");
  if (f && !strcmp(f, "pergroup")) return false;
  if (f && !strcmp(f, "runs")) return true;
  return h->total_tiles < 256;
}

template <int T, int MT, int QMAX, bool DUAL>
void launch_v2_b(const GmArgs& a, int bf, unsigned grid, size_t lds, hipStream_t st) {
  switch (bf) {
    case 2: k_gemm_v2<T, MT, QMAX, DUAL, 2><<<grid, a.NW * 64, lds, st>>>(a); break;
    case 3: k_gemm_v2<T, MT, QMAX, DUAL, 3><<<grid, a.NW * 64, lds, st>>>(a); break;
    case 4: k_gemm_v2<T, MT, QMAX, DUAL, 4><<<grid, a.NW * 64, lds, st>>>(a); break;
    default: k_gemm_v2<T, MT, QMAX, DUAL, 0><<<grid, a.NW * 64, lds, st>>>(a); break;
  }
}

// compiled tile counts per wave: (MT, QMAX) = (1, 4): T <= 2, fused pair T = 1;
// (2, 2): T <= 4, fused pair T <= 2 (register room for all of a slice's codes)
constexpr int v2_tmax(int MT, bool dual) { return MT == 1 ? (dual ? 1 : 2) : (dual ? 2 : 4); }

template <int MT, int QMAX>
void launch_v2(const GmArgs& a, int T, bool dual, int bf, unsigned grid, size_t lds, hipStream_t st) {
  if (dual) {
    if (T == 1 || v2_tmax(MT, true) < 2) launch_v2_b<1, MT, QMAX, true>(a, bf, grid, lds, st);
    else if constexpr (v2_tmax(MT, true) >= 2) launch_v2_b<2, MT, QMAX, true>(a, bf, grid, lds, st);
  } else {
    if (T == 1) launch_v2_b<1, MT, QMAX, false>(a, bf, grid, lds, st);
    else if (T == 2 || v2_tmax(MT, false) < 4) launch_v2_b<2, MT, QMAX, false>(a, bf, grid, lds, st);
    else if constexpr (v2_tmax(MT, false) >= 4) launch_v2_b<4, MT, QMAX, false>(a, bf, grid, lds, st);
  }
}

qg_status run_gemm_v2(const qg_plan* h, const qg_plan* h2, const uint16_t* x, int M, uint16_t* y, int ldy,
                      hipStream_t st) {
  const bool dual = h2 != nullptr;
  const Launch L = choose(h, M, dual);
  GmArgs a{};
  a.w[0] = wset_of(h);
  if (h2) a.w[1] = wset_of(h2);
  a.x = x;
  a.y = y;
  a.partial = h->partial;
  a.counters = h->counters;
  a.M = M;
  a.K = h->K;
  a.G = h->G;
  a.G4 = h->G4;
  a.ldy = ldy;
  a.NP = 16 * h->total_tiles;
  a.S = L.S;
  a.NW = L.NW;
  int pre = 0;
  for (int i = 0; i < (int)h->segs.size(); ++i) {
    a.ts_prefix[i] = pre;
    pre += (h->segs[i].tiles + L.T * L.NW - 1) / (L.T * L.NW);
  }
  for (int i = (int)h->segs.size(); i <= MAX_SEG; ++i) a.ts_prefix[i] = pre;
  if (L.S > 1 && partial_need(h, L.S, M) > h->partial_floats)
    return fail(QG_ERR_INVALID_ARG, "workspace too small for %d K-slices at M=%d", L.S, M);
  if (pre > h->total_tiles) return fail(QG_ERR_INVALID_ARG, "more tile sets than counters");
  const unsigned grid = (unsigned)pre * (unsigned)L.S;
  const int bf = h->segs.size() == 1 ? h->segs[0].bits : 0;
  if (M <= 16) launch_v2<1, 4>(a, L.T, dual, bf, grid, gm_lds_bytes(1, 4), st);
  else launch_v2<2, 2>(a, L.T, dual, bf, grid, gm_lds_bytes(2, 2), st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  if (getenv("QG_DEBUG_SYNC")) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel failed: %s", hipGetErrorString(e));
  }
  return QG_OK;
}

template <int T, int MT, bool DUAL, int BF>
hipError_t xs_allow_lds() {
  hipError_t e = hipSuccess;
  const hipError_t r[] = {
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_xs<T, MT, DUAL, BF, 4>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax),
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_xs<T, MT, DUAL, BF, 5>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax),
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_xs<T, MT, DUAL, BF, 8>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax)};
  for (hipError_t x : r)
    if (x != hipSuccess) e = x;
  return e;
}

template <int BF>
hipError_t xs_allow_lds_b() {
  hipError_t e = hipSuccess;
  const hipError_t r[] = {xs_allow_lds<2, 1, false, BF>(), xs_allow_lds<2, 2, false, BF>(),
                          xs_allow_lds<1, 1, false, BF>(), xs_allow_lds<1, 2, false, BF>(),
                          xs_allow_lds<1, 1, true, BF>(), xs_allow_lds<1, 2, true, BF>()};
  for (hipError_t x : r)
    if (x != hipSuccess) e = x;
  return e;
}

// let the x-in-LDS GEMM take up to the whole LDS of a compute unit
hipError_t xs_allow_lds_all() {
  hipError_t e = hipSuccess;
  const hipError_t r[] = {xs_allow_lds_b<0>(), xs_allow_lds_b<2>(), xs_allow_lds_b<3>(), xs_allow_lds_b<4>()};
  for (hipError_t x : r)
    if (x != hipSuccess) e = x;
  return e;
}

template <int T, int MT, bool DUAL, int NQ>
void launch_xs_t(const XsArgs& a, const XsPlan& p, int bf, hipStream_t st) {
  switch (bf) {
    case 2: k_gemm_xs<T, MT, DUAL, 2, NQ><<<p.grid, p.NW * 64, p.lds, st>>>(a); break;
    case 3: k_gemm_xs<T, MT, DUAL, 3, NQ><<<p.grid, p.NW * 64, p.lds, st>>>(a); break;
    case 4: k_gemm_xs<T, MT, DUAL, 4, NQ><<<p.grid, p.NW * 64, p.lds, st>>>(a); break;
    default: k_gemm_xs<T, MT, DUAL, 0, NQ><<<p.grid, p.NW * 64, p.lds, st>>>(a); break;
  }
}

template <int MT, bool DUAL, int NQ>
void launch_xs_q(const XsArgs& a, const XsPlan& p, int bf, hipStream_t st) {
  if constexpr (DUAL) launch_xs_t<1, MT, true, NQ>(a, p, bf, st);
  else if (p.T == 1) launch_xs_t<1, MT, false, NQ>(a, p, bf, st);
  else launch_xs_t<2, MT, false, NQ>(a, p, bf, st);
}

template <int MT, bool DUAL>
void launch_xs_b(const XsArgs& a, const XsPlan& p, int bf, hipStream_t st) {
  if (p.NQ == 4) launch_xs_q<MT, DUAL, 4>(a, p, bf, st);
  else if (p.NQ == 5) launch_xs_q<MT, DUAL, 5>(a, p, bf, st);
  else launch_xs_q<MT, DUAL, 8>(a, p, bf, st);
}

qg_status run_gemm_xs(const qg_plan* h, const qg_plan* h2, const uint16_t* x, int M, uint16_t* y, int ldy,
                      hipStream_t st) {
  const bool dual = h2 != nullptr;
  const XsPlan p = xs_plan(h, M, dual);
  if (p.NQ == 0 || p.lds > kLdsMax)
    return fail(QG_ERR_INVALID_ARG, "x slice of %d quads at M=%d does not fit LDS", p.nq, M);
  if (p.S > 1 && partial_need(h, p.S, M) > h->partial_floats)
    return fail(QG_ERR_INVALID_ARG, "workspace too small for %d K-slices at M=%d", p.S, M);
  if (p.tg_prefix[MAX_SEG] > std::max(1, h->total_tiles)) return fail(QG_ERR_INVALID_ARG, "more tile groups than counters");
  XsArgs a{};
  a.w[0] = wset_of(h);
  if (h2) a.w[1] = wset_of(h2);
  a.x = x;
  a.y = y;
  a.partial = h->partial;
  a.counters = h->counters;
  a.acc = p.fx ? h->acc64 : nullptr;
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
  const int bf = h->segs.size() == 1 ? h->segs[0].bits : 0;
  if (p.MT == 1) {
    if (dual) launch_xs_b<1, true>(a, p, bf, st);
    else launch_xs_b<1, false>(a, p, bf, st);
  } else {
    if (dual) launch_xs_b<2, true>(a, p, bf, st);
    else launch_xs_b<2, false>(a, p, bf, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  if (getenv("QG_DEBUG_SYNC")) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel failed: %s", hipGetErrorString(e));
  }
  return QG_OK;
}

// one GEMV/GEMM over a uniform handle (or the fused gate+up pair when h2 != NULL)
qg_status run_uniform(const qg_plan* h, const qg_plan* h2, const uint16_t* x, int M, uint16_t* y, int ldy,
                      hipStream_t st) {
  const bool dual = h2 != nullptr;
  if (M == 1 && use_sk(h)) return run_sk(h, h2, x, y, st);
  if (M > 1 && gemm_kind(h, M) == GEMM_XS) return run_gemm_xs(h, h2, x, M, y, ldy, st);
  if (M > 1 && gemm_v2_on()) return run_gemm_v2(h, h2, x, M, y, ldy, st);
  Launch L = choose(h, M, dual);
  int T = L.T;
  if (M == 1) T = 1;
  else T = (T >= 4) ? 4 : (T >= 2 ? 2 : 1);
  int NW = std::max(1, std::min(L.NW, M == 1 ? 16 : 8));
  if (M > 1) NW = NW >= 8 ? 8 : (NW >= 4 ? 4 : (NW >= 2 ? 2 : 1));
  const int S = L.S;
  const int bf = h->segs.size() == 1 ? h->segs[0].bits : 0;
  if (dual && M > 1 && T > 2) T = 2;  // the fused gate/up MFMA pass is built for <= 2 tiles
  if (M > 1) {
    const int MT = M <= 16 ? 1 : 2;
    while ((dual ? 2 : 1) * NW * T * MT * 1024 + 16 > 65536) {
      if (T > 1) T /= 2;
      else NW /= 2;
    }
  }
  RunArgs a{};
  a.w[0] = wset_of(h);
  if (h2) a.w[1] = wset_of(h2);
  a.x = x;
  a.y = y;
  a.partial = h->partial;
  a.counters = h->counters;
  a.M = M;
  a.K = h->K;
  a.G = h->G;
  a.G4 = h->G4;
  a.ldy = ldy;
  a.NP = 16 * h->total_tiles;
  a.T = T;
  a.S = S;
  const bool pair = M == 1 && dual && m1_pair_on();
  a.pair = pair ? 1 : 0;
  a.xw = h->acc64;
  if (pair && S == 1 && !h->acc64) return fail(QG_ERR_INVALID_ARG, "no hand-over words for the paired gate/up pass");
  {
    // M = 1, one matrix, K slices: fixed-point words (QG_M1_HANDOVER=partials forces the partials)
    const char* fh = getenv("QG_M1_HANDOVER");
    a.fx = (M == 1 && !dual && S > 1 && S <= 63 && h->acc64 && !(fh && !strcmp(fh, "partials"))) ? 1 : 0;
  }
  int pre = 0;
  for (int i = 0; i < (int)h->segs.size(); ++i) {
    a.ts_prefix[i] = pre;
    pre += (h->segs[i].tiles + T - 1) / T;
  }
  for (int i = (int)h->segs.size(); i <= MAX_SEG; ++i) a.ts_prefix[i] = pre;
  if (S > 1 && partial_need(h, S, M) > h->partial_floats)
    return fail(QG_ERR_INVALID_ARG, "workspace too small for %d K-slices at M=%d", S, M);
  if (pair && pair_need(h, S) > h->partial_floats)
    return fail(QG_ERR_INVALID_ARG, "workspace too small for the paired gate/up pass");
  const unsigned grid = (unsigned)pre * (unsigned)S * (pair ? 2u : 1u);
  if (M == 1) {
    const int nqs = (h->G4 + S - 1) / S;
    const int NQ = L.NQ;
    if (NQ <= 0 || (int64_t)NQ * NW < nqs)
      return fail(QG_ERR_INVALID_ARG, "%d waves cannot cover %d quads per slice with the compiled quad counts", NW, nqs);
    if (dual && !pair && NQ > 2) return fail(QG_ERR_INVALID_ARG, "fused gate/up needs at most 2 quads per wave");
    const bool kd = dual && !pair;  // both matrices in each workgroup
    const size_t lds = m1_lds_bytes(nqs, kd ? 2 : 1, NW);
    if (lds > 65536) return fail(QG_ERR_INVALID_ARG, "K slice of %d quads does not fit LDS: use more splits", nqs);
    switch (NQ) {
      case 1: launch_q<1>(a, NW, lds, grid, kd, bf, st); break;
      case 2: launch_q<2>(a, NW, lds, grid, kd, bf, st); break;
      case 3: launch_q<3>(a, NW, lds, grid, kd, bf, st); break;
      case 4: launch_q<4>(a, NW, lds, grid, kd, bf, st); break;
      case 5: launch_q<5>(a, NW, lds, grid, kd, bf, st); break;
      default: launch_q<5>(a, NW, lds, grid, kd, bf, st); break;
    }
  } else {
    const int MT = M <= 16 ? 1 : 2;
    const size_t lds = (size_t)(dual ? 2 : 1) * NW * T * MT * 4 * 64 * sizeof(float) + 16;
    if (lds > 65536) return fail(QG_ERR_INVALID_ARG, "launch needs %zu B of LDS (max 65536): fewer tiles or waves", lds);
    if (MT == 1) launch_mfma<1>(a, T, NW, lds, grid, dual, bf, st);
    else launch_mfma<2>(a, T, NW, lds, grid, dual, bf, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  if (getenv("QG_DEBUG_SYNC")) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(QG_ERR_DEVICE, "kernel failed: %s", hipGetErrorString(e));
  }
  return QG_OK;
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
  if (d->group_size != QG_GROUP) return fail(QG_ERR_INVALID_ARG, "group_size must be 128 (got %d)", d->group_size);
  if (d->K <= 0 || d->K % QG_GROUP) return fail(QG_ERR_INVALID_ARG, "K = %d is not a positive multiple of 128", d->K);
  if (d->N <= 0 || d->N % 16) return fail(QG_ERR_INVALID_ARG, "N = %d is not a positive multiple of 16", d->N);
  if (max_M < 1 || max_M > QG_MAX_M) return fail(QG_ERR_INVALID_ARG, "max_M = %d is not in [1, 32]", max_M);
  if (!d->codes || !d->scales) return fail(QG_ERR_INVALID_ARG, "codes and scales must be device pointers");
  if (!aligned16(d->codes) || !aligned16(d->scales)) return fail(QG_ERR_INVALID_ARG, "codes/scales must be 16-byte aligned");
  if (d->format != QG_FMT_UNIFORM && d->format != QG_FMT_TRELLIS3)
    return fail(QG_ERR_INVALID_ARG, "unknown format %d", d->format);
  if (d->format == QG_FMT_TRELLIS3) {
    if (!d->codebook || !aligned16(d->codebook)) return fail(QG_ERR_INVALID_ARG, "trellis needs a 16-byte aligned codebook");
  }
  int dev = 0;
  qg_status s = check_device(&dev);
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
  h->device = dev;
  if (hipDeviceGetAttribute(&h->cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || h->cus < 1) {
    delete h;
    return fail(QG_ERR_DEVICE, "cannot query the compute-unit count");
  }
  hipStream_t st = (hipStream_t)stream;
  s = d->format == QG_FMT_UNIFORM ? create_uniform(h, d, st) : create_trellis(h, d, st);
  if (s == QG_OK && h->format == QG_FMT_UNIFORM) s = ensure_workspace(h);
  if (s == QG_OK) {
    const int nc = std::max(1, h->total_tiles);
    if (hipMalloc(&h->counters, nc * sizeof(int)) != hipSuccess) s = fail(QG_ERR_OOM, "counter allocation failed");
    else if (hipMemsetAsync(h->counters, 0, nc * sizeof(int), st) != hipSuccess)
      s = fail(QG_ERR_DEVICE, "counter initialisation failed");
  }
  if (s == QG_OK && hipMalloc(&h->hbuf, (size_t)max_M * d->N * sizeof(uint16_t)) != hipSuccess)
    s = fail(QG_ERR_OOM, "staging allocation failed");
  if (s == QG_OK && h->format == QG_FMT_UNIFORM && sk_allow_lds_all() != hipSuccess)
    s = fail(QG_ERR_DEVICE, "cannot raise the LDS limit of the M = 1 kernels");
  if (s == QG_OK && h->format == QG_FMT_UNIFORM && xs_allow_lds_all() != hipSuccess)
    s = fail(QG_ERR_DEVICE, "cannot raise the LDS limit of the verify GEMM");
  if (s == QG_OK && h->format == QG_FMT_UNIFORM) {
    // fixed-point output words [2][max_M][16 * total_tiles]: the M = 1 GEMV uses
    // the first 2 * 16 * total_tiles (the paired gate/up pass the first
    // 16 * total_tiles as hand-over words), the x-in-LDS GEMM rows 0 .. M - 1
    const size_t nw = (size_t)2 * h->max_M * 16 * h->total_tiles;
    if (hipMalloc(&h->acc64, nw * sizeof(unsigned long long)) != hipSuccess)
      s = fail(QG_ERR_OOM, "column-word allocation failed");
    else if (hipMemsetAsync(h->acc64, 0, nw * sizeof(unsigned long long), st) != hipSuccess)
      s = fail(QG_ERR_DEVICE, "column-word initialisation failed");
  }
  if (s == QG_OK && hipStreamSynchronize(st) != hipSuccess) s = fail(QG_ERR_DEVICE, "stream synchronisation failed");
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

qg_status qgemv_set_launch(qg_handle h, int32_t M, int32_t tiles, int32_t waves, int32_t splits) {
  g_err.clear();
  if (!h) return fail(QG_ERR_INVALID_ARG, "NULL handle");
  if (h->format != QG_FMT_UNIFORM) return fail(QG_ERR_INVALID_ARG, "launch overrides apply to uniform-code handles");
  if (M < 1 || M > QG_MAX_M) return fail(QG_ERR_INVALID_ARG, "M = %d is not in [1, 32]", M);
  if (M == 1 ? (waves > 16) : (waves > 0 && waves != 1 && waves != 2 && waves != 4 && waves != 8))
    return fail(QG_ERR_INVALID_ARG, "waves must be 1..16 for M = 1, else 1, 2, 4 or 8");
  if (splits > 16) return fail(QG_ERR_INVALID_ARG, "splits must be <= 16");
  Launch& L = h->over[mclass(M)];
  L.T = tiles;
  L.NW = waves;
  L.S = splits;
  return ensure_workspace(h);
}

qg_status qgemv_run(qg_handle h, const uint16_t* x, int32_t M, uint16_t* y, void* stream) {
  g_err.clear();
  if (!h || !x || !y) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (M < 1 || M > h->max_M) return fail(QG_ERR_INVALID_ARG, "M = %d is not in [1, %d]", M, h->max_M);
  if (!aligned16(x) || !aligned16(y)) return fail(QG_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (h->format == QG_FMT_TRELLIS3) return run_trellis(h, x, M, y, st);
  return run_uniform(h, nullptr, x, M, y, h->N, st);
}

qg_status qmlp_run(qg_handle gate, qg_handle up, qg_handle down, const uint16_t* x, int32_t M, uint16_t* out,
                   void* stream) {
  g_err.clear();
  if (!gate || !up || !down || !x || !out) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (gate->format != QG_FMT_UNIFORM || up->format != QG_FMT_UNIFORM || down->format != QG_FMT_UNIFORM)
    return fail(QG_ERR_UNSUPPORTED, "the fused MLP takes uniform-code handles");
  if (gate->K != up->K || gate->N != up->N) return fail(QG_ERR_INVALID_ARG, "gate and up shapes differ");
  if (gate->col_bits != up->col_bits) return fail(QG_ERR_INVALID_ARG, "gate and up need the same per-column widths");
  if (down->K != gate->N) return fail(QG_ERR_INVALID_ARG, "down K (%d) != gate N (%d)", down->K, gate->N);
  if (M < 1 || M > gate->max_M || M > down->max_M) return fail(QG_ERR_INVALID_ARG, "M = %d out of range", M);
  if (!aligned16(x) || !aligned16(out)) return fail(QG_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  qg_status s = run_uniform(gate, up, x, M, gate->hbuf, gate->N, st);
  if (s != QG_OK) return s;
  return run_uniform(down, nullptr, gate->hbuf, M, out, down->N, st);
}

qg_status qgemv_debug_unpack(qg_handle h, int32_t* codes, void* stream) {
  g_err.clear();
  if (!h || !codes) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (h->format != QG_FMT_UNIFORM) return fail(QG_ERR_INVALID_ARG, "debug_unpack takes a uniform-code handle");
  hipStream_t st = (hipStream_t)stream;
  for (const auto& s : h->segs) {
    SegDev sd{s.codes, s.scales, s.bits, s.tiles, s.tile0};
    const int64_t n = (int64_t)s.tiles * h->G * 64;
    k_debug_uniform<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(sd, h->col_map, h->G, h->G4, h->K, codes, nullptr,
                                                                 nullptr);
  }
  QG_HIP(hipGetLastError());
  return QG_OK;
}

qg_status qgemv_debug_dequant(qg_handle h, float* w, uint16_t* q16, void* stream) {
  g_err.clear();
  if (!h || !w) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  hipStream_t st = (hipStream_t)stream;
  if (h->format == QG_FMT_TRELLIS3) return debug_trellis(h, nullptr, w, st);
  for (const auto& s : h->segs) {
    SegDev sd{s.codes, s.scales, s.bits, s.tiles, s.tile0};
    const int64_t n = (int64_t)s.tiles * h->G * 64;
    k_debug_uniform<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(sd, h->col_map, h->G, h->G4, h->K, nullptr, w, q16);
  }
  QG_HIP(hipGetLastError());
  return QG_OK;
}

qg_status qgemv_debug_trellis(qg_handle h, uint16_t* states, void* stream) {
  g_err.clear();
  if (!h || !states) return fail(QG_ERR_INVALID_ARG, "NULL argument");
  if (h->format != QG_FMT_TRELLIS3) return fail(QG_ERR_INVALID_ARG, "debug_trellis takes a trellis handle");
  return debug_trellis(h, states, nullptr, (hipStream_t)stream);
}

}  // extern "C"
