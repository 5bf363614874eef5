// Boundary reads with one wavefront per row (64 lanes x 2 .. 14 vectors):
// folds of P plain partials with bf16 or fp8 output, and MoE finalize folds
// of k gathered picks with bf16 output; P and k (1..16) are runtime values.
#include "kernels.h"

namespace bnd {

namespace {
template <int VPT>
constexpr std::array<KernelFn, 3> wave_read_row() {
  return {{&wave_read_kernel<Source::Partials, VPT, false>, &wave_read_kernel<Source::Partials, VPT, true>,
           &wave_read_kernel<Source::Moe, VPT, false>}};
}
// [width slot: 2, 4, ..., 14 vectors per lane][partials bf16, partials fp8, MoE bf16]
constexpr std::array<KernelFn, 3> kWaveKernels[kWaveWidths] = {
    wave_read_row<2>(),  wave_read_row<4>(),  wave_read_row<6>(),  wave_read_row<8>(),
    wave_read_row<10>(), wave_read_row<12>(), wave_read_row<14>(), {{nullptr, nullptr, nullptr}}};
static_assert(kWaveWidths == 8 && wave_slot(2) == 0 && wave_slot(kWaveReadVptMax) == 6,
              "one table row per width, the last one empty");

// the 4-, 6- and 8-wide kernels with the deep ring (depth = width), by the same columns
template <int VPT>
constexpr std::array<KernelFn, 3> wave_read_deep_row() {
  return {{&wave_read_kernel<Source::Partials, VPT, false, VPT>, &wave_read_kernel<Source::Partials, VPT, true, VPT>,
           &wave_read_kernel<Source::Moe, VPT, false, VPT>}};
}
constexpr std::array<KernelFn, 3> kWaveDeep[kWaveDeepWidths] = {wave_read_deep_row<4>(), wave_read_deep_row<6>(),
                                                                 wave_read_deep_row<8>()};
static_assert(kWaveDeepWidths == 3 && deep_slot(8) == 2, "one deep table row per width");

// the table column of a call, or -1 when it has no one-wavefront kernel
int wave_kind(Source src, bool fp8) {
  if (src == Source::Partials) return fp8 ? 1 : 0;
  if (src == Source::Moe && !fp8) return 2;
  return -1;
}

std::atomic<int> g_rows_per_cu[kWaveWidths][3];  // 0: not read yet, -1: unknown
std::atomic<int> g_deep_rows_per_cu[kWaveDeepWidths][3];
}  // namespace

int wave_read_rows_per_cu(Source src, bool fp8, int vpt, bool deep) {
  const int kind = wave_kind(src, fp8), w = wave_slot(vpt);
  const int d = deep_slot(vpt);
  if (kind < 0 || w < 0 || vpt > kWaveReadVptMax || (deep && d < 0)) return 0;
  if (deep) return occupancy_rows(kWaveDeep[d][kind], g_deep_rows_per_cu[d][kind]);
  return occupancy_rows(kWaveKernels[w][kind], g_rows_per_cu[w][kind]);
}

hipError_t launch_read_wave(Source src, int n, bool fp8, const RowArgs& a, const Launch& l, hipStream_t stream) {
  const int kind = wave_kind(src, fp8), w = wave_slot(l.vpt);
  if (!l.one_wave || w < 0 || l.vpt > kWaveReadVptMax || kind < 0 || l.threads != kWave || a.nvec > kWave * l.vpt ||
      n < 1 || n > kMaxSources || (l.deep && deep_slot(l.vpt) < 0))
    return hipErrorInvalidValue;
  RowArgs b = a;
  b.nsrc = n;
  return launch_kernel(l.deep ? kWaveDeep[deep_slot(l.vpt)][kind] : kWaveKernels[w][kind], b, l, stream);
}

}  // namespace bnd
