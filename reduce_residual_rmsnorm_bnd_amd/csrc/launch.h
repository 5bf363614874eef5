// launch.h -- internal interface between the host state machine (host.cpp)
// and the gfx950 kernels (k_*.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bnd {

constexpr int kMaxSources = 16;
constexpr int kMaxThreads = 1024;
constexpr int kWave = 64;
// Vectors per lane of the one-wavefront-per-row kernels: an even count from 2
// to 14 for the reads (rows of up to 1024 .. 7168 elements) and to 16 for the
// completes (up to 8192), one kernel per width. The tables have a slot for
// every width up to kWaveVptMax; the reads leave the widest one empty.
constexpr int kWaveVptMin = 2;
constexpr int kWaveReadVptMax = 14;
// The 4-, 6- and 8-wide kernels also come with a deep ring, every vector of a
// source in flight (a depth equal to the width instead of 2), for launches of
// too few rows per CU to keep the memory busy with two loads in flight per
// wave.
constexpr int kWaveDeepMin = 4;
constexpr int kWaveDeepMax = 8;
constexpr int kWaveDeepWidths = (kWaveDeepMax - kWaveDeepMin) / 2 + 1;
constexpr int deep_slot(int vpt) {
  return vpt >= kWaveDeepMin && vpt <= kWaveDeepMax && vpt % 2 == 0 ? (vpt - kWaveDeepMin) / 2 : -1;
}
constexpr int kWaveVptMax = 16;
constexpr int kWaveWidths = (kWaveVptMax - kWaveVptMin) / 2 + 1;
// the table slot of a one-wavefront width, or -1 for a width without kernels
constexpr int wave_slot(int vpt) {
  return vpt >= kWaveVptMin && vpt <= kWaveVptMax && vpt % 2 == 0 ? (vpt - kWaveVptMin) / 2 : -1;
}
// the narrowest one-wavefront width whose 64 lanes cover a row of nvec vectors
// (may exceed kWaveVptMax: no kernel then)
constexpr int wave_width(int nvec) {
  const int w = 2 * ((nvec + 2 * 64 - 1) / (2 * 64));
  return w < kWaveVptMin ? kWaveVptMin : w;
}

// Arguments of one boundary launch. Every row pointer is already offset to
// the first row the launch processes, so a kernel addresses row i of each
// operand at base + i * ld. The grid has one workgroup per row.
struct RowArgs {
  const uint16_t* src[kMaxSources];  // partial rows (bf16), one pointer per source
  int64_t ld_src;                    // elements
  const uint16_t* experts;           // MoE expert-output rows, indexed by idx (absolute)
  int64_t ld_e;
  int64_t n_expert_rows;
  const int32_t* idx;                // MoE [rows, k], offset to the first row
  const float* gate;                 // MoE [rows, k]
  const uint16_t* extra;             // add_to_output: a contribution added once after the sum
  int64_t ld_extra;
  const uint16_t* x_in;              // stack input (enter)
  int64_t ld_x;
  uint16_t* res;                     // residual storage
  int64_t ld_res;
  const float* w;                    // norm weight [H]
  uint16_t* y;                       // bf16 read output, or complete_only output
  int64_t ld_y;
  uint8_t* q;                        // fp8 read output
  int64_t ld_q;
  float* scale;                      // fp8 per-row scale
  float eps;
  int H;                             // elements per row
  int nvec;                          // H / 8
  int has_residual;                  // 0: fold with r = 0 (Pending without a residual)
  int gemma;                         // 1: the norm weight is an offset from one, y = x inv (1 + w)
  int copy_input;                    // enter: store x_in into the residual storage
  int nsrc;                          // one-wavefront read: number of partials or MoE picks
};

struct Launch {
  int rows = 0;     // grid size
  int threads = 0;  // workgroup size, multiple of 64
  int vpt = 0;      // 16-byte vectors per thread: 1, 2 or 4; for one wavefront per row 2 .. 16, even
  bool one_wave = false;  // one wavefront per row (wave_read_kernel, wave_complete_kernel; threads = 64)
  bool deep = false;      // one wavefront per row with the deep ring (depth = vpt, 4 .. 8)
  bool nt_stores = false;  // multi-wave reads, one vector per thread: the non-temporal-store kernels
  hipEvent_t start = nullptr;  // when set, recorded around the kernel itself (hipExtLaunchKernel)
  hipEvent_t stop = nullptr;
};

enum class Source { Partials, Moe, Input, Residual };

// What a complete adds after the owed partials or picks: nothing
// (complete_only), the extra row (add_to_output) or the residual (snapshot).
enum class Tail { None, Extra, Residual };

// fold_norm / fold_norm_quant_fp8 / moe_finalize_fold_norm / enter / written read.
// n = number of sources (partials P or MoE picks k), ignored for Input/Residual.
hipError_t launch_read(Source src, int n, bool fp8, const RowArgs& a, const Launch& l,
                       hipStream_t stream);

// complete_only / add_to_output: y <- bf16(sum [+ extra]) for partials or MoE picks.
// With fold, y <- bf16(residual + sum) (snapshot); Residual with n = 0 copies the residual.
hipError_t launch_complete(Source src, int n, bool fold, const RowArgs& a, const Launch& l,
                           hipStream_t stream);

// One wavefront per row (l.one_wave): the read of a fold, or a complete.
hipError_t launch_read_wave(Source src, int n, bool fp8, const RowArgs& a, const Launch& l, hipStream_t stream);
hipError_t launch_complete_wave(Source src, int n, Tail tail, const RowArgs& a, const Launch& l,
                                hipStream_t stream);

// Rows of one launch that a compute unit of the current device holds at once
// with the one-wavefront read or complete kernel of vpt (2 .. 16, even)
// vectors per lane, with the deep ring when `deep` (vpt 4, 6 or 8 only):
// its occupancy in 64-thread workgroups, from the HIP runtime, read once per
// kernel; 0 when no such kernel exists or the runtime cannot tell.
int wave_read_rows_per_cu(Source src, bool fp8, int vpt, bool deep = false);
int wave_complete_rows_per_cu(Source src, Tail tail, int vpt, bool deep = false);

}  // namespace bnd
