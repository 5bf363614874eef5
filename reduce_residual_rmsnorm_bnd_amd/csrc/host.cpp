// host.cpp -- the C ABI of libboundary: stream state machine, validation,
// launch-shape choice and dispatch (declared in include/boundary.h).
//
// The stream follows the state table of the SGLang guide "Layer boundaries"
// (section "Residual stream"): Initial -> the read enters; Written -> the
// read applies no update; Pending -> complete the owed work, fold it into the
// residual, read. Owed tokens play the part of the guide's OwedOutput
// handles: a read must present the token of the stream's current
// publication, so a stale or foreign handle is refused instead of applying
// the wrong pending work. Every check runs before any launch, so a refused
// call leaves outputs and state untouched (section "Fusion providers and
// output decisions": a candidate refuses before modifying its inputs).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>

#include "../../include/boundary.h"
#include "launch.h"

using bnd::Launch;
using bnd::RowArgs;
using bnd::Source;

struct bnd_stream {
  uint64_t serial;
  uint32_t epoch;
  int64_t T, H, row_begin, rows;
  uint16_t* residual;
  int64_t ld_res;
  bnd_state state;
  bnd_norm_form norm_form;
  bool has_residual;
  bnd_kind kind;
  bnd_owed owed;
  // partials (global rows): element (t, h) at src[p] + (t - src_origin) * ld_src + h
  const uint16_t* src[BND_MAX_SOURCES];
  int nsrc;
  int64_t ld_src;
  int64_t src_origin;
  // deferred MoE finalize
  const uint16_t* experts;
  int64_t n_expert_rows;
  int64_t ld_e;
  const int32_t* idx;
  const float* gate;
  int k;
};

namespace {

thread_local std::string g_last_error;
std::atomic<uint64_t> g_serial{1};
std::atomic<int> g_fused_unavailable{-1};  // -1: read BND_DISABLE_FUSED on first use
std::atomic<int> g_threads_override{0};
std::atomic<int> g_vpt_override{0};
std::atomic<int> g_one_wave_mode{BND_ONE_WAVEFRONT_AUTO};
std::atomic<int> g_depth_override{0};
thread_local hipEvent_t g_time_start = nullptr;  // consumed by the thread's next launch
thread_local hipEvent_t g_time_stop = nullptr;
thread_local Launch g_chosen;       // the shape of the launch being prepared
thread_local Launch g_last_launch;  // the shape of the thread's last launch

bnd_status fail(bnd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(bnd_status_str(st)) + ": " + buf;
  return st;
}

bnd_status ok() {
  g_last_error.clear();
  return BND_OK;
}

bool fused_unavailable() {
  int v = g_fused_unavailable.load();
  if (v < 0) {
    const char* e = getenv("BND_DISABLE_FUSED");
    v = (e && e[0] == '1') ? 1 : 0;
    int expected = -1;
    g_fused_unavailable.compare_exchange_strong(expected, v);
    v = g_fused_unavailable.load();
  }
  return v == 1;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bnd_owed make_owed(const bnd_stream* s) { return (s->serial << 24) | (s->epoch & 0xFFFFFFu); }

// Byte range [lo, hi) touched by rows [0, rows) of a row tensor.
struct Range {
  uintptr_t lo = 0, hi = 0;
};

// Unsigned arithmetic: with rows, ld <= 2^31 - 1 and elem <= 4 the extent stays below 2^64.
Range rows_range(const void* base, int64_t rows, int64_t ld, int64_t width, int64_t elem) {
  Range r;
  if (!base || rows <= 0 || width <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(base);
  r.hi = r.lo + ((uintptr_t)(rows - 1) * (uintptr_t)ld + (uintptr_t)width) * (uintptr_t)elem;
  return r;
}

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bnd_status check_hidden(int64_t H) {
  if (H < 8 || H > BND_MAX_HIDDEN || H % 8 != 0)
    return fail(BND_ERR_NO_PATH, "hidden size %lld: need a multiple of 8 in [8, %d]", (long long)H,
                BND_MAX_HIDDEN);
  return BND_OK;
}

bnd_status check_rows_tensor(const char* what, const void* p, int64_t ld, int64_t H, bool needed) {
  if (!needed) return BND_OK;
  if (!p) return fail(BND_ERR_INVALID_ARG, "%s is NULL", what);
  if (!aligned(p, 16)) return fail(BND_ERR_INVALID_ARG, "%s is not 16-byte aligned", what);
  if (ld < H || ld % 8 != 0 || ld > BND_MAX_LD)
    return fail(BND_ERR_INVALID_ARG, "%s leading dimension %lld: need a multiple of 8 in [H = %lld, %lld]",
                what, (long long)ld, (long long)H, (long long)BND_MAX_LD);
  return BND_OK;
}

bnd_status check_weight(const float* w, float eps, bool needed) {
  if (!(eps >= 0.0f) || eps != eps || eps > 3.4e38f)
    return fail(BND_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!needed) return BND_OK;
  if (!w) return fail(BND_ERR_INVALID_ARG, "weight is NULL");
  if (!aligned(w, 16)) return fail(BND_ERR_INVALID_ARG, "weight is not 16-byte aligned");
  return BND_OK;
}

// Compute units of the current device (256 on MI355X), read once.
int compute_units() {
  static std::atomic<int> cus{0};
  int n = cus.load();
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
    cus.store(n);
  }
  return n;
}

// ---------------------------------------------------------------------------
// Launch shape. One workgroup per row, in one of two kernel families:
//  - one wavefront per row: 64 lanes x `width` vectors of 8 elements, width the
//    narrowest even count that covers the row (2 .. 14 for the reads, 16 for the
//    completes), only for calls that take owed partials or MoE picks;
//  - several wavefronts per row: `threads` x `vpt` vectors (vpt 1, 2 or 4).
// The automatic choice is the data below, from launch-shape sweeps on MI355X.
// A "round" is the rows the chip holds at once with a kernel: its occupancy
// in rows per CU (the HIP runtime's answer for the kernel, which its VGPRs
// set) times the CUs.
// ---------------------------------------------------------------------------

// The one-wavefront kernel of a width is taken when the row is long enough for
// it (its lanes more than 3/4 full at the widths of 2 and 4; a row that needs
// a wider width always is), the call may take it (width 2: owed partials only,
// the MoE finalize measured slower there at every row count), and either
//  - the launch has deep_from <= rows per CU < deep_below and fits in one
//    round of the kernel with the deep ring (every vector of a source in
//    flight), which replaces two loads in flight where too few rows per CU
//    would leave the memory idle; or
//  - the launch has at least min_rows_per_cu rows per CU and fits in one
//    round, or its last round is full enough (WaveFit::last_num / last_den).
// Measured against the multi-wave shapes: 5-12% faster at 2048 rows for every
// such call at H = 4096 and 7168 and 1-13% at H = 2048 .. 6144; from 10%
// slower to 5% faster at 6 rows per CU; 17-87% slower at 4 rows per CU and
// below with two loads in flight; with a last round a sixth to a half full,
// 5-14% slower for the reads (the completes still 4-11% faster from a third).
struct WaveRule {
  int min_vectors;        // shortest row, in 16-byte vectors, that takes the width
  bool partials_only;     // only calls on owed partials take it
  int min_rows_per_cu;    // two loads in flight: from this many rows per CU
  int deep_from, deep_below;  // the deep ring: rows per CU in [deep_from, deep_below)
};

constexpr WaveRule kWaveRules[bnd::kWaveWidths] = {
    //  vectors  partials  rows/CU  deep ring
    {97, true, 12, 0, 0},    // width 2: H = 776 .. 1024
    {193, false, 6, 6, 8},   // width 4: H = 1544 .. 2048
    {193, false, 6, 6, 8},   // width 6
    {193, false, 6, 4, 8},   // width 8: H = 3080 .. 4096
    {193, false, 6, 0, 0},   // width 10
    {193, false, 6, 0, 0},   // width 12
    {193, false, 6, 0, 0},   // width 14
    {193, false, 6, 0, 0},   // width 16 (the completes)
};
static_assert(bnd::kWaveWidths == 8 && bnd::wave_slot(16) == 7, "one rule per width");

// The multi-wave shapes: one vector per thread while the row has at most 256
// vectors, or at most 1024 and every row of the launch is resident at once
// (rows x waves per row <= the CU's wave slots x CUs): more waves per row
// hide more latency, 5-11% faster for 128..1024 rows. Otherwise two vectors
// per thread up to 2048 vectors (with P = 8 about 60 VGPRs: eight 4-wave rows
// per CU keep a 2048-row batch resident; 8-wave rows need two rounds, 4%
// slower), four beyond. Workgroups of 256 threads or more are whole
// multiples of 256, so every SIMD of the CU gets the same number of waves
// (7- or 5-wave workgroups measured 3-6% slower).
constexpr int kWaveSlotsPerCu = 32;
// Reads with one vector per thread on fewer rows than CUs (decode boundaries)
// take the kernels with non-temporal stores: 3% faster per boundary; launches
// that give every CU a row or more keep sc1 stores (non-temporal: the 256-row
// MoE share 3% and the 2048-row calls 3.6% slower). The completes always
// store with sc1.
constexpr int kOneVectorAlways = 256;
constexpr int kOneVectorResident = 1024;
constexpr int kTwoVectors = 2048;

int round_threads(int need) {
  const int unit = need >= 256 ? 4 * bnd::kWave : bnd::kWave;
  return ((need + unit - 1) / unit) * unit;
}

// The call's one-wavefront kernels: whether it has them, whether it takes owed
// partials, the widest, how full a launch's last round must be, and each
// kernel's rows per CU.
struct WaveFit {
  bool ok = false;
  bool partials = false;
  int max_vpt = 0;
  int last_num = 1;  // reads: 3/4 of a round; completes: 1/3
  int last_den = 1;
  int rows_per_cu[bnd::kWaveWidths] = {};
  int deep_rows_per_cu[bnd::kWaveDeepWidths] = {};  // the deep-ring kernels (widths 4 .. 8)
};

WaveFit wave_fit_read(bnd::Source src, bool fp8) {
  WaveFit f;
  f.ok = true;
  f.partials = src == Source::Partials;
  f.max_vpt = bnd::kWaveReadVptMax;
  f.last_num = 3;
  f.last_den = 4;
  for (int v = bnd::kWaveVptMin; v <= bnd::kWaveVptMax; v += 2)
    f.rows_per_cu[bnd::wave_slot(v)] = bnd::wave_read_rows_per_cu(src, fp8, v);
  for (int v = bnd::kWaveDeepMin; v <= bnd::kWaveDeepMax; v += 2)
    f.deep_rows_per_cu[bnd::deep_slot(v)] = bnd::wave_read_rows_per_cu(src, fp8, v, true);
  return f;
}

WaveFit wave_fit_complete(bnd::Source src, bnd::Tail tail) {
  WaveFit f;
  f.ok = true;
  f.partials = src == Source::Partials;
  f.max_vpt = bnd::kWaveVptMax;
  f.last_num = 1;
  f.last_den = 3;
  for (int v = bnd::kWaveVptMin; v <= bnd::kWaveVptMax; v += 2)
    f.rows_per_cu[bnd::wave_slot(v)] = bnd::wave_complete_rows_per_cu(src, tail, v);
  for (int v = bnd::kWaveDeepMin; v <= bnd::kWaveDeepMax; v += 2)
    f.deep_rows_per_cu[bnd::deep_slot(v)] = bnd::wave_complete_rows_per_cu(src, tail, v, true);
  return f;
}

// The device queries the launch heuristic needs (CU count, the one-wavefront
// kernels' occupancy), made once per process when the first stream is created,
// so that no hot call asks the runtime anything but to launch (a hot call may
// run under HIP graph capture).
void warm_launch_queries() {
  static std::once_flag once;
  std::call_once(once, [] {
    compute_units();
    for (Source src : {Source::Partials, Source::Moe}) {
      for (bool fp8 : {false, true}) (void)wave_fit_read(src, fp8);
      for (bnd::Tail t : {bnd::Tail::None, bnd::Tail::Extra, bnd::Tail::Residual}) (void)wave_fit_complete(src, t);
    }
  });
}

// Whether a launch of `rows` rows fills its rounds of `per_round` resident
// rows well enough: one round always, more when the last one is at least
// num / den full.
bool rounds_fill(int64_t rows, int64_t per_round, int num, int den) {
  if (per_round <= 0) return false;
  if (rows <= per_round) return true;
  const int64_t last = rows - (rows - 1) / per_round * per_round;  // rows of the last round, 1..per_round
  return last * den >= per_round * num;
}

// The automatic one-wavefront choice for a row of nvec vectors (kWaveRules);
// *deep tells whether it takes the deep ring. `ring_two` is a forced ring of two.
bool auto_one_wave(int nvec, int64_t rows, int64_t cus, const WaveFit& wave, bool ring_two, bool* deep) {
  const int width = bnd::wave_width(nvec);
  const int w = bnd::wave_slot(width);
  if (!wave.ok || w < 0 || width > wave.max_vpt) return false;
  const WaveRule& r = kWaveRules[w];
  if (nvec < r.min_vectors || (r.partials_only && !wave.partials)) return false;
  const int d = bnd::deep_slot(width);
  if (d >= 0 && !ring_two && rows >= r.deep_from * cus && rows < r.deep_below * cus &&
      rows <= (int64_t)wave.deep_rows_per_cu[d] * cus) {
    *deep = true;
    return true;
  }
  return rows >= r.min_rows_per_cu * cus &&
         rounds_fill(rows, (int64_t)wave.rows_per_cu[w] * cus, wave.last_num, wave.last_den);
}

bnd_status choose_launch(int64_t H, int64_t rows, const WaveFit& wave, Launch* l) {
  const int nvec = (int)(H / 8);
  int vpt = g_vpt_override.load();
  int threads = g_threads_override.load();
  const int one_wave_mode = g_one_wave_mode.load();
  const int depth = g_depth_override.load();
  const int64_t cus = compute_units();
  const bool forced = vpt != 0;
  // A forced count of 6 .. 16 is one wavefront per row; under ALWAYS every
  // forced count is (2 and 4 included); under NEVER none may be.
  bool one_wave = forced && (vpt > 4 || one_wave_mode == BND_ONE_WAVEFRONT_ALWAYS);
  bool deep = false;
  if (one_wave && one_wave_mode == BND_ONE_WAVEFRONT_NEVER)
    return fail(BND_ERR_NO_PATH, "%d vectors per thread is one wavefront per row, which is switched off", vpt);
  if (!forced && one_wave_mode == BND_ONE_WAVEFRONT_ALWAYS) {
    one_wave = true;
    vpt = bnd::wave_width(nvec);
  } else if (!forced) {
    if (one_wave_mode == BND_ONE_WAVEFRONT_AUTO && auto_one_wave(nvec, rows, cus, wave, depth == 2, &deep)) {
      one_wave = true;
      vpt = bnd::wave_width(nvec);
    } else if (nvec <= kOneVectorAlways ||
               (nvec <= kOneVectorResident &&
                rows * (int64_t)(round_threads(nvec) / bnd::kWave) <= cus * kWaveSlotsPerCu)) {
      vpt = 1;
    } else {
      vpt = nvec <= kTwoVectors ? 2 : 4;
    }
  }
  if (one_wave) {
    if (!wave.ok)
      return fail(BND_ERR_NO_PATH,
                  "%d vectors per lane (one wavefront per row) only takes the owed partials or MoE picks", vpt);
    if (bnd::wave_slot(vpt) < 0 || vpt > wave.max_vpt)
      return forced ? fail(BND_ERR_NO_PATH, "one wavefront per row takes %d .. %d (even) vectors per lane, not %d",
                           bnd::kWaveVptMin, wave.max_vpt, vpt)
                    : fail(BND_ERR_NO_PATH, "one wavefront per row covers H <= %d, not H = %lld",
                           wave.max_vpt * bnd::kWave * 8, (long long)H);
    if (nvec > vpt * bnd::kWave)
      return fail(BND_ERR_NO_PATH, "%d vectors per lane (one wavefront per row) needs H <= %d", vpt,
                  vpt * bnd::kWave * 8);
    if (threads != 0 && threads != bnd::kWave)
      return fail(BND_ERR_NO_PATH, "%d vectors per lane (one wavefront per row) needs 64 threads, not %d", vpt,
                  threads);
    threads = bnd::kWave;
    if (depth > 2) {
      if (vpt != depth)
        return fail(BND_ERR_NO_PATH, "the deep ring of %d is built for %d vectors per lane, not %d", depth, depth, vpt);
      deep = true;
    }
  } else if (depth > 2) {
    return fail(BND_ERR_NO_PATH, "the deep ring is for one wavefront per row; this launch has %d threads per row",
                threads != 0 ? threads : round_threads((nvec + vpt - 1) / vpt));
  }
  if (threads == 0) threads = round_threads((nvec + vpt - 1) / vpt);
  if (!one_wave && vpt != 1 && vpt != 2 && vpt != 4)
    return fail(BND_ERR_NO_PATH, "vectors per thread %d: need 1, 2 or 4, or 6 .. 16 (even) for one wavefront "
                "per row", vpt);
  if (threads < bnd::kWave || threads > bnd::kMaxThreads || threads % bnd::kWave != 0)
    return fail(BND_ERR_NO_PATH, "threads per row %d: need a multiple of 64 in [64, 1024]", threads);
  if ((int64_t)threads * vpt < nvec)
    return fail(BND_ERR_NO_PATH, "launch shape %d threads x %d vectors cannot cover H = %lld", threads,
                vpt, (long long)H);
  if (rows > 0x7fffffff) return fail(BND_ERR_NO_PATH, "too many rows for one grid");
  // a dispatch packet counts its grid in work-items, in 32 bits
  if ((uint64_t)rows * (uint64_t)threads > 0xffffffffull)
    return fail(BND_ERR_NO_PATH, "%lld rows of %d threads exceed one dispatch's 2^32 - 1 work-items", (long long)rows,
                threads);
  l->rows = (int)rows;
  l->threads = threads;
  l->vpt = vpt;
  l->one_wave = one_wave;
  l->deep = deep;
  l->nt_stores = !one_wave && vpt == 1 && rows < cus;
  l->start = g_time_start;
  l->stop = g_time_stop;
  g_chosen = *l;
  return BND_OK;
}

RowArgs base_args(const bnd_stream* s) {
  RowArgs a;
  memset(&a, 0, sizeof a);
  a.H = (int)s->H;
  a.nvec = (int)(s->H / 8);
  a.res = s->residual;
  a.ld_res = s->ld_res;
  a.has_residual = s->has_residual ? 1 : 0;
  a.gemma = s->norm_form == BND_NORM_GEMMA ? 1 : 0;
  return a;
}

// Fill the owed-work part of the arguments for the stream's slice.
void pending_args(const bnd_stream* s, RowArgs* a) {
  if (s->kind == BND_KIND_PARTIALS) {
    for (int p = 0; p < s->nsrc; ++p) a->src[p] = s->src[p] + (s->row_begin - s->src_origin) * s->ld_src;
    a->ld_src = s->ld_src;
  } else if (s->kind == BND_KIND_MOE) {
    a->experts = s->experts;
    a->ld_e = s->ld_e;
    a->n_expert_rows = s->n_expert_rows;
    a->idx = s->idx + s->row_begin * s->k;
    a->gate = s->gate + s->row_begin * s->k;
  }
}

// Input byte ranges of the pending work restricted to the slice.
int pending_ranges(const bnd_stream* s, Range* out) {
  int n = 0;
  if (s->rows <= 0) return 0;
  if (s->kind == BND_KIND_PARTIALS) {
    for (int p = 0; p < s->nsrc; ++p)
      out[n++] = rows_range(s->src[p] + (s->row_begin - s->src_origin) * s->ld_src, s->rows, s->ld_src,
                            s->H, 2);
  } else if (s->kind == BND_KIND_MOE) {
    out[n++] = rows_range(s->experts, s->n_expert_rows, s->ld_e, s->H, 2);
    out[n++] = rows_range(s->idx + s->row_begin * s->k, s->rows, s->k, s->k, 4);
    out[n++] = rows_range(s->gate + s->row_begin * s->k, s->rows, s->k, s->k, 4);
  }
  return n;
}

bnd_status check_output_disjoint(const bnd_stream* s, const char* what, const Range& out, bool with_residual,
                                 const Range* extra = nullptr, int n_extra = 0) {
  Range in[BND_MAX_SOURCES + 4];
  int n = pending_ranges(s, in);
  if (with_residual) in[n++] = rows_range(s->residual, s->rows, s->ld_res, s->H, 2);
  for (int i = 0; i < n; ++i)
    if (overlap(out, in[i])) return fail(BND_ERR_INVALID_ARG, "%s overlaps the residual or an input", what);
  for (int i = 0; i < n_extra; ++i)
    if (overlap(out, extra[i])) return fail(BND_ERR_INVALID_ARG, "%s overlaps another output", what);
  return BND_OK;
}

bnd_status launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BND_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  g_time_start = nullptr;
  g_time_stop = nullptr;
  g_last_launch = g_chosen;
  return BND_OK;
}

// The shared state checks of a read that folds owed work (fold_norm,
// fold_norm_quant_fp8, moe_finalize_fold_norm). `kind` is the owed-work kind
// the call completes. On BND_OK, *fold tells whether there is work to fold.
bnd_status check_fold_state(const bnd_stream* s, bnd_owed owed, bnd_kind kind, bool* fold) {
  if (!s) return fail(BND_ERR_INVALID_ARG, "stream is NULL");
  if (s->state == BND_INITIAL)
    return fail(BND_ERR_NOT_STARTED, "the stream has neither a residual nor a contribution; enter first");
  if (s->state == BND_WRITTEN) {
    if (owed != BND_OWED_NONE) return fail(BND_ERR_FOREIGN_OUTPUT, "the stream owes nothing; the handle is foreign");
    *fold = false;
    return BND_OK;
  }
  if (s->kind != kind)
    return fail(BND_ERR_WRONG_KIND, "the pending contribution is a %s, this call completes a %s",
                s->kind == BND_KIND_MOE ? "MoE finalize handoff" : "set of partials",
                kind == BND_KIND_MOE ? "MoE finalize handoff" : "set of partials");
  if (owed != s->owed) return fail(BND_ERR_FOREIGN_OUTPUT, "the handle does not belong to this stream's pending output");
  if (fused_unavailable() && (kind == BND_KIND_MOE || s->nsrc > 1))
    return fail(BND_ERR_UNAVAILABLE, "fused completion is switched off; complete_only then a one-source fold");
  *fold = true;
  return BND_OK;
}

void become_written(bnd_stream* s) {
  s->state = BND_WRITTEN;
  s->has_residual = true;
  s->kind = BND_KIND_NONE;
  s->owed = BND_OWED_NONE;
  s->nsrc = 0;
}

}  // namespace

extern "C" {

const char* bnd_status_str(bnd_status st) {
  switch (st) {
    case BND_OK: return "BND_OK";
    case BND_ERR_INVALID_ARG: return "BND_ERR_INVALID_ARG";
    case BND_ERR_NOT_STARTED: return "BND_ERR_NOT_STARTED";
    case BND_ERR_FOREIGN_OUTPUT: return "BND_ERR_FOREIGN_OUTPUT";
    case BND_ERR_PENDING: return "BND_ERR_PENDING";
    case BND_ERR_WRONG_KIND: return "BND_ERR_WRONG_KIND";
    case BND_ERR_NO_PATH: return "BND_ERR_NO_PATH";
    case BND_ERR_UNAVAILABLE: return "BND_ERR_UNAVAILABLE";
    case BND_ERR_HIP: return "BND_ERR_HIP";
  }
  return "BND_ERR_UNKNOWN";
}

const char* bnd_last_error(void) { return g_last_error.c_str(); }

const char* bnd_version(void) { return "libboundary 0.1 (gfx950)"; }

bnd_status bnd_last_launch_shape(int64_t* rows, int* threads, int* vectors_per_thread, int* one_wavefront) {
  if (rows) *rows = g_last_launch.rows;
  if (threads) *threads = g_last_launch.threads;
  if (vectors_per_thread) *vectors_per_thread = g_last_launch.vpt;
  if (one_wavefront) *one_wavefront = g_last_launch.one_wave ? 1 : 0;
  return ok();
}

bnd_status bnd_last_launch_ring_depth(int* depth) {
  if (depth) *depth = g_last_launch.one_wave ? (g_last_launch.deep ? g_last_launch.vpt : 2) : 0;
  return ok();
}

bnd_status bnd_time_next_launch(void* start_event, void* stop_event) {
  g_time_start = static_cast<hipEvent_t>(start_event);
  g_time_stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

bnd_status bnd_set_option(bnd_option opt, int64_t value) {
  switch (opt) {
    case BND_OPT_FUSED_UNAVAILABLE:
      if (value != 0 && value != 1) return fail(BND_ERR_INVALID_ARG, "fused-unavailable takes 0 or 1");
      g_fused_unavailable.store((int)value);
      return ok();
    case BND_OPT_THREADS_PER_ROW:
      if (value != 0 && (value < 64 || value > 1024 || value % 64 != 0))
        return fail(BND_ERR_INVALID_ARG, "threads per row: 0 or a multiple of 64 in [64, 1024]");
      g_threads_override.store((int)value);
      return ok();
    case BND_OPT_VECTORS_PER_THREAD:
      if (value != 0 && value != 1 && value != 2 && value != 4 && (value < 6 || value > 16 || value % 2 != 0))
        return fail(BND_ERR_INVALID_ARG, "vectors per thread: 0, 1, 2, 4, or 6 .. 16 (even)");
      g_vpt_override.store((int)value);
      return ok();
    case BND_OPT_ONE_WAVEFRONT:
      if (value != BND_ONE_WAVEFRONT_AUTO && value != BND_ONE_WAVEFRONT_ALWAYS && value != BND_ONE_WAVEFRONT_NEVER)
        return fail(BND_ERR_INVALID_ARG, "one-wavefront mode: 0 (automatic), 1 (always) or 2 (never)");
      g_one_wave_mode.store((int)value);
      return ok();
    case BND_OPT_RING_DEPTH:
      if (value != 0 && value != 2 && (value < bnd::kWaveDeepMin || value > bnd::kWaveDeepMax || value % 2 != 0))
        return fail(BND_ERR_INVALID_ARG, "ring depth: 0 (automatic), 2, or %d .. %d (even) for that many vectors "
                    "per lane", bnd::kWaveDeepMin, bnd::kWaveDeepMax);
      g_depth_override.store((int)value);
      return ok();
  }
  return fail(BND_ERR_INVALID_ARG, "unknown option %d", (int)opt);
}

int64_t bnd_get_option(bnd_option opt) {
  switch (opt) {
    case BND_OPT_FUSED_UNAVAILABLE: return fused_unavailable() ? 1 : 0;
    case BND_OPT_THREADS_PER_ROW: return g_threads_override.load();
    case BND_OPT_VECTORS_PER_THREAD: return g_vpt_override.load();
    case BND_OPT_ONE_WAVEFRONT: return g_one_wave_mode.load();
    case BND_OPT_RING_DEPTH: return g_depth_override.load();
  }
  return -1;
}

bnd_status bnd_stream_create(bnd_stream** out, int64_t T, int64_t H, int64_t row_begin, int64_t rows,
                             void* residual, int64_t ld_res) {
  if (!out) return fail(BND_ERR_INVALID_ARG, "out is NULL");
  if (T < 0) return fail(BND_ERR_INVALID_ARG, "T = %lld < 0", (long long)T);
  if (T > BND_MAX_ROWS) return fail(BND_ERR_NO_PATH, "T = %lld: at most %lld token rows", (long long)T,
                                    (long long)BND_MAX_ROWS);
  if (row_begin < 0 || rows < 0 || row_begin > T || rows > T - row_begin)
    return fail(BND_ERR_INVALID_ARG, "slice of %lld rows from %lld is not inside [0, %lld)", (long long)rows,
                (long long)row_begin, (long long)T);
  bnd_status st = check_hidden(H);
  if (st) return st;
  if ((st = check_rows_tensor("residual", residual, ld_res, H, rows > 0))) return st;
  warm_launch_queries();
  bnd_stream* s = new (std::nothrow) bnd_stream;
  if (!s) return fail(BND_ERR_INVALID_ARG, "out of host memory");
  memset(s, 0, sizeof *s);
  s->serial = g_serial.fetch_add(1);
  s->epoch = 0;
  s->T = T;
  s->H = H;
  s->row_begin = row_begin;
  s->rows = rows;
  s->residual = static_cast<uint16_t*>(residual);
  s->ld_res = ld_res;
  s->state = BND_INITIAL;
  s->norm_form = BND_NORM_PLAIN;
  s->has_residual = false;
  s->kind = BND_KIND_NONE;
  s->owed = BND_OWED_NONE;
  *out = s;
  return ok();
}

bnd_status bnd_stream_destroy(bnd_stream* s) {
  if (!s) return fail(BND_ERR_INVALID_ARG, "stream is NULL");
  delete s;
  return ok();
}

bnd_state bnd_stream_state(const bnd_stream* s) { return s ? s->state : BND_INITIAL; }

bnd_kind bnd_stream_pending_kind(const bnd_stream* s) { return s ? s->kind : BND_KIND_NONE; }

int bnd_stream_has_residual(const bnd_stream* s) { return (s && s->has_residual) ? 1 : 0; }

bnd_status bnd_stream_set_norm_form(bnd_stream* s, bnd_norm_form form) {
  if (!s) return fail(BND_ERR_INVALID_ARG, "stream is NULL");
  if (form != BND_NORM_PLAIN && form != BND_NORM_GEMMA)
    return fail(BND_ERR_INVALID_ARG, "unknown norm form %d", (int)form);
  s->norm_form = form;
  return ok();
}

bnd_status bnd_publish_partials(bnd_stream* s, const void* const* partials, int P, int64_t ld, bnd_owed* owed) {
  if (!s) return fail(BND_ERR_INVALID_ARG, "stream is NULL");
  if (!owed) return fail(BND_ERR_INVALID_ARG, "owed is NULL");
  if (s->state == BND_PENDING) return fail(BND_ERR_PENDING, "a contribution is already pending; fold it first");
  if (P < 1 || P > BND_MAX_SOURCES) return fail(BND_ERR_NO_PATH, "P = %d: need 1..%d partials", P, BND_MAX_SOURCES);
  if (s->rows > 0 && !partials) return fail(BND_ERR_INVALID_ARG, "partials is NULL");
  for (int p = 0; p < P && s->rows > 0; ++p) {
    char what[32];
    snprintf(what, sizeof what, "partial %d", p);
    bnd_status st = check_rows_tensor(what, partials[p], ld, s->H, true);
    if (st) return st;
  }
  for (int p = 0; p < P; ++p) s->src[p] = s->rows > 0 ? static_cast<const uint16_t*>(partials[p]) : nullptr;
  s->nsrc = P;
  s->ld_src = ld;
  s->src_origin = 0;
  s->kind = BND_KIND_PARTIALS;
  s->state = BND_PENDING;
  s->epoch++;
  s->owed = make_owed(s);
  *owed = s->owed;
  return ok();
}

bnd_status bnd_publish_moe(bnd_stream* s, const void* expert_rows, int64_t n_rows, int64_t ld, const int32_t* idx,
                           const float* gate, int k, bnd_owed* owed) {
  if (!s) return fail(BND_ERR_INVALID_ARG, "stream is NULL");
  if (!owed) return fail(BND_ERR_INVALID_ARG, "owed is NULL");
  if (s->state == BND_PENDING) return fail(BND_ERR_PENDING, "a contribution is already pending; fold it first");
  if (k < 1 || k > BND_MAX_SOURCES) return fail(BND_ERR_NO_PATH, "k = %d: need 1..%d picks", k, BND_MAX_SOURCES);
  if (n_rows < 0 || n_rows > BND_MAX_ROWS)
    return fail(BND_ERR_INVALID_ARG, "n_rows = %lld: need 0..%lld (int32 row indices)", (long long)n_rows,
                (long long)BND_MAX_ROWS);
  if (s->rows > 0) {
    bnd_status st = check_rows_tensor("expert rows", expert_rows, ld, s->H, n_rows > 0);
    if (st) return st;
    if (!idx || !aligned(idx, 4)) return fail(BND_ERR_INVALID_ARG, "idx is NULL or misaligned");
    if (!gate || !aligned(gate, 4)) return fail(BND_ERR_INVALID_ARG, "gate is NULL or misaligned");
  }
  s->experts = static_cast<const uint16_t*>(expert_rows);
  s->n_expert_rows = n_rows;
  s->ld_e = ld;
  s->idx = idx;
  s->gate = gate;
  s->k = k;
  s->nsrc = 0;
  s->kind = BND_KIND_MOE;
  s->state = BND_PENDING;
  s->epoch++;
  s->owed = make_owed(s);
  *owed = s->owed;
  return ok();
}

bnd_status bnd_enter_norm(bnd_stream* s, const void* x, int64_t ld_x, const float* w, float eps, void* y,
                          int64_t ld_y, void* hip_stream) {
  if (!s) return fail(BND_ERR_INVALID_ARG, "stream is NULL");
  if (s->state == BND_PENDING) return fail(BND_ERR_PENDING, "a contribution is pending; fold it instead of entering");
  const bool entering = s->state == BND_INITIAL;
  const bool any = s->rows > 0;
  bnd_status st;
  if ((st = check_weight(w, eps, any))) return st;
  if ((st = check_rows_tensor("y", y, ld_y, s->H, any))) return st;
  if (entering && (st = check_rows_tensor("x", x, ld_x, s->H, any))) return st;
  const bool alias = entering && x == s->residual && ld_x == s->ld_res;
  Range yr = rows_range(y, s->rows, ld_y, s->H, 2);
  Range in[2] = {rows_range(s->residual, s->rows, s->ld_res, s->H, 2),
                 entering ? rows_range(x, s->rows, ld_x, s->H, 2) : Range{}};
  if (overlap(yr, in[0]) || overlap(yr, in[1])) return fail(BND_ERR_INVALID_ARG, "y overlaps the residual or x");
  const Range wr = rows_range(w, 1, s->H, s->H, 4);
  if (overlap(yr, wr) || (entering && !alias && overlap(in[0], wr)))
    return fail(BND_ERR_INVALID_ARG, "the weight overlaps y or the residual the call writes");
  if (entering && !alias && overlap(in[0], in[1]))
    return fail(BND_ERR_INVALID_ARG, "x partly overlaps the residual storage");
  if (any) {
    Launch l;
    if ((st = choose_launch(s->H, s->rows, WaveFit{}, &l))) return st;
    RowArgs a = base_args(s);
    a.w = w;
    a.eps = eps;
    a.y = static_cast<uint16_t*>(y);
    a.ld_y = ld_y;
    Source src = Source::Residual;
    if (entering) {
      src = Source::Input;
      a.x_in = static_cast<const uint16_t*>(x);
      a.ld_x = ld_x;
      a.copy_input = alias ? 0 : 1;
    }
    if ((st = launch_status(bnd::launch_read(src, 0, false, a, l, (hipStream_t)hip_stream), "enter_norm")))
      return st;
  }
  become_written(s);
  return ok();
}

static bnd_status fold_read(bnd_stream* s, bnd_owed owed, bnd_kind kind, bool fp8, const float* w, float eps,
                            void* y, int64_t ld_y, uint8_t* q, int64_t ld_q, float* scale, void* hip_stream,
                            const char* name) {
  bool fold = false;
  bnd_status st = check_fold_state(s, owed, kind, &fold);
  if (st) return st;
  const bool any = s->rows > 0;
  if ((st = check_weight(w, eps, any))) return st;
  Range outs[2];
  int n_out = 0;
  if (fp8) {
    if (any) {
      if (!q || !aligned(q, 8)) return fail(BND_ERR_INVALID_ARG, "q is NULL or not 8-byte aligned");
      if (ld_q < s->H || ld_q % 8 != 0 || ld_q > BND_MAX_LD)
        return fail(BND_ERR_INVALID_ARG, "ld_q: need a multiple of 8 in [H, BND_MAX_LD]");
      if (!scale || !aligned(scale, 4)) return fail(BND_ERR_INVALID_ARG, "scale is NULL or misaligned");
    }
    outs[n_out++] = rows_range(q, s->rows, ld_q, s->H, 1);
    outs[n_out++] = rows_range(scale, s->rows, 1, 1, 4);
    if (overlap(outs[0], outs[1])) return fail(BND_ERR_INVALID_ARG, "q overlaps scale");
  } else {
    if ((st = check_rows_tensor("y", y, ld_y, s->H, any))) return st;
    outs[n_out++] = rows_range(y, s->rows, ld_y, s->H, 2);
  }
  for (int i = 0; i < n_out; ++i)
    if ((st = check_output_disjoint(s, fp8 ? (i ? "scale" : "q") : "y", outs[i], true))) return st;
  const Range wr = rows_range(w, 1, s->H, s->H, 4);
  for (int i = 0; i < n_out; ++i)
    if (overlap(outs[i], wr)) return fail(BND_ERR_INVALID_ARG, "%s overlaps the weight", fp8 ? (i ? "scale" : "q") : "y");
  if (fold && overlap(rows_range(s->residual, s->rows, s->ld_res, s->H, 2), wr))
    return fail(BND_ERR_INVALID_ARG, "the residual (written by the fold) overlaps the weight");
  if (any) {
    // a fold reads the owed partials or picks; a Written stream's read, the stored residual
    const Source src = !fold ? Source::Residual : kind == BND_KIND_MOE ? Source::Moe : Source::Partials;
    const int n = !fold ? 0 : kind == BND_KIND_MOE ? s->k : s->nsrc;
    Launch l;
    if ((st = choose_launch(s->H, s->rows, fold ? wave_fit_read(src, fp8) : WaveFit{}, &l))) return st;
    RowArgs a = base_args(s);
    a.w = w;
    a.eps = eps;
    a.y = static_cast<uint16_t*>(y);
    a.ld_y = ld_y;
    a.q = q;
    a.ld_q = ld_q;
    a.scale = scale;
    if (fold) pending_args(s, &a);
    if ((st = launch_status(bnd::launch_read(src, n, fp8, a, l, (hipStream_t)hip_stream), name))) return st;
  }
  become_written(s);
  return ok();
}

bnd_status bnd_fold_norm(bnd_stream* s, bnd_owed owed, const float* w, float eps, void* y, int64_t ld_y,
                         void* hip_stream) {
  return fold_read(s, owed, BND_KIND_PARTIALS, false, w, eps, y, ld_y, nullptr, 0, nullptr, hip_stream,
                   "fold_norm");
}

bnd_status bnd_fold_norm_quant_fp8(bnd_stream* s, bnd_owed owed, const float* w, float eps, uint8_t* q,
                                   int64_t ld_q, float* scale, void* hip_stream) {
  return fold_read(s, owed, BND_KIND_PARTIALS, true, w, eps, nullptr, 0, q, ld_q, scale, hip_stream,
                   "fold_norm_quant_fp8");
}

bnd_status bnd_moe_finalize_fold_norm(bnd_stream* s, bnd_owed owed, const float* w, float eps, void* y,
                                      int64_t ld_y, void* hip_stream) {
  return fold_read(s, owed, BND_KIND_MOE, false, w, eps, y, ld_y, nullptr, 0, nullptr, hip_stream,
                   "moe_finalize_fold_norm");
}

// complete_only (extra == NULL) and add_to_output: out = bf16(s [+ extra]) for
// the slice rows, then the stream owes one plain partial that is `out`.
static bnd_status complete_into(bnd_stream* s, bnd_owed owed, bool with_extra, const void* extra,
                                int64_t ld_extra, void* out, int64_t ld_out, bnd_owed* new_owed, void* hip_stream,
                                const char* name) {
  if (!s) return fail(BND_ERR_INVALID_ARG, "stream is NULL");
  if (!new_owed) return fail(BND_ERR_INVALID_ARG, "new_owed is NULL");
  if (s->state == BND_INITIAL) return fail(BND_ERR_NOT_STARTED, "nothing has been published on this stream");
  if (s->state == BND_WRITTEN) return fail(BND_ERR_WRONG_KIND, "the stream owes nothing to complete");
  if (owed != s->owed) return fail(BND_ERR_FOREIGN_OUTPUT, "the handle does not belong to this stream's pending output");
  const bool any = s->rows > 0;
  bnd_status st;
  if ((st = check_rows_tensor("out", out, ld_out, s->H, any))) return st;
  const Range out_r = rows_range(out, s->rows, ld_out, s->H, 2);
  if ((st = check_output_disjoint(s, "out", out_r, true))) return st;
  const uint16_t* extra_rows = nullptr;
  if (with_extra) {
    if ((st = check_rows_tensor("extra", extra, ld_extra, s->H, any))) return st;
    if (any) {
      extra_rows = static_cast<const uint16_t*>(extra) + s->row_begin * ld_extra;
      if (overlap(out_r, rows_range(extra_rows, s->rows, ld_extra, s->H, 2)))
        return fail(BND_ERR_INVALID_ARG, "out overlaps extra");
    }
  }
  if (any) {
    Launch l;
    const Source src = s->kind == BND_KIND_MOE ? Source::Moe : Source::Partials;
    const bnd::Tail tail = with_extra ? bnd::Tail::Extra : bnd::Tail::None;
    if ((st = choose_launch(s->H, s->rows, wave_fit_complete(src, tail), &l))) return st;
    RowArgs a = base_args(s);
    pending_args(s, &a);
    a.extra = extra_rows;
    a.ld_extra = ld_extra;
    a.y = static_cast<uint16_t*>(out);
    a.ld_y = ld_out;
    const int n = s->kind == BND_KIND_MOE ? s->k : s->nsrc;
    if ((st = launch_status(bnd::launch_complete(src, n, false, a, l, (hipStream_t)hip_stream), name)))
      return st;
  }
  // the stream now owes one plain partial: `out`, addressed by slice row
  s->kind = BND_KIND_PARTIALS;
  s->src[0] = any ? static_cast<const uint16_t*>(out) : nullptr;
  s->nsrc = 1;
  s->ld_src = ld_out;
  s->src_origin = s->row_begin;
  s->experts = nullptr;
  s->idx = nullptr;
  s->gate = nullptr;
  s->epoch++;
  s->owed = make_owed(s);
  *new_owed = s->owed;
  return ok();
}

bnd_status bnd_complete_only(bnd_stream* s, bnd_owed owed, void* out, int64_t ld_out, bnd_owed* new_owed,
                             void* hip_stream) {
  return complete_into(s, owed, false, nullptr, 0, out, ld_out, new_owed, hip_stream, "complete_only");
}

bnd_status bnd_add_to_output(bnd_stream* s, bnd_owed owed, const void* extra, int64_t ld_extra, void* out,
                             int64_t ld_out, bnd_owed* new_owed, void* hip_stream) {
  return complete_into(s, owed, true, extra, ld_extra, out, ld_out, new_owed, hip_stream, "add_to_output");
}

bnd_status bnd_snapshot(bnd_stream* s, bnd_owed owed, void* out, int64_t ld_out, void* hip_stream) {
  if (!s) return fail(BND_ERR_INVALID_ARG, "stream is NULL");
  if (s->state == BND_INITIAL) return fail(BND_ERR_NOT_STARTED, "the stream has no residual and owes nothing");
  if (s->state == BND_WRITTEN && owed != BND_OWED_NONE)
    return fail(BND_ERR_FOREIGN_OUTPUT, "the stream owes nothing; the handle is foreign");
  if (s->state == BND_PENDING) {
    if (s->kind == BND_KIND_MOE)
      return fail(BND_ERR_WRONG_KIND, "a snapshot needs a plain contribution; complete the MoE handoff first");
    if (owed != s->owed) return fail(BND_ERR_FOREIGN_OUTPUT, "the handle does not belong to this stream's pending output");
  }
  const bool any = s->rows > 0;
  bnd_status st;
  if ((st = check_rows_tensor("out", out, ld_out, s->H, any))) return st;
  if ((st = check_output_disjoint(s, "out", rows_range(out, s->rows, ld_out, s->H, 2), true))) return st;
  if (any) {
    Launch l;
    const WaveFit fit = s->state == BND_PENDING ? wave_fit_complete(Source::Partials, bnd::Tail::Residual) : WaveFit{};
    if ((st = choose_launch(s->H, s->rows, fit, &l))) return st;
    RowArgs a = base_args(s);
    a.y = static_cast<uint16_t*>(out);
    a.ld_y = ld_out;
    Source src = Source::Residual;
    int n = 0;
    if (s->state == BND_PENDING) {
      pending_args(s, &a);
      src = Source::Partials;
      n = s->nsrc;
    }
    if ((st = launch_status(bnd::launch_complete(src, n, true, a, l, (hipStream_t)hip_stream), "snapshot")))
      return st;
  }
  return ok();
}

bnd_status bnd_rsv_share(const int64_t* counts, int R, int r, int64_t* row_begin, int64_t* rows, int64_t* T) {
  if (!counts || !row_begin || !rows || !T) return fail(BND_ERR_INVALID_ARG, "NULL argument");
  if (R < 1 || r < 0 || r >= R) return fail(BND_ERR_INVALID_ARG, "rank %d outside [0, %d)", r, R);
  int64_t begin = 0, total = 0;
  for (int i = 0; i < R; ++i) {
    if (counts[i] < 0) return fail(BND_ERR_INVALID_ARG, "rank %d has a negative row count", i);
    if (total > INT64_MAX - counts[i]) return fail(BND_ERR_INVALID_ARG, "row counts overflow");
    if (i == r) begin = total;
    total += counts[i];
  }
  *row_begin = begin;
  *rows = counts[r];
  *T = total;
  return ok();
}

bnd_status bnd_written(bnd_stream* s, void* residual, int64_t ld_res) {
  if (!s) return fail(BND_ERR_INVALID_ARG, "stream is NULL");
  bnd_status st = check_rows_tensor("residual", residual, ld_res, s->H, s->rows > 0);
  if (st) return st;
  s->residual = static_cast<uint16_t*>(residual);
  s->ld_res = ld_res;
  become_written(s);
  return ok();
}

bnd_status bnd_take_output(bnd_stream* s) {
  if (!s) return fail(BND_ERR_INVALID_ARG, "stream is NULL");
  if (s->state == BND_PENDING)
    return fail(BND_ERR_PENDING, "a contribution is pending; fold or norm it before taking the output");
  s->state = BND_INITIAL;
  s->has_residual = false;
  s->kind = BND_KIND_NONE;
  s->owed = BND_OWED_NONE;
  s->nsrc = 0;
  return ok();
}

}  // extern "C"
