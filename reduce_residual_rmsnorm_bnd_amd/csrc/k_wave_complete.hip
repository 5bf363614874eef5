// complete_only, add_to_output and snapshot with one wavefront per row
// (64 lanes x 2 .. 16 vectors): the owed P partials or k MoE picks, then
// nothing, the extra row or the residual; P and k (1..16) are runtime values.
#include "kernels.h"

namespace bnd {

namespace {
template <int VPT>
constexpr std::array<KernelFn, 5> wave_complete_row() {
  return {{&wave_complete_kernel<Source::Partials, VPT, Tail::None>,
           &wave_complete_kernel<Source::Partials, VPT, Tail::Extra>,
           &wave_complete_kernel<Source::Partials, VPT, Tail::Residual>,
           &wave_complete_kernel<Source::Moe, VPT, Tail::None>, &wave_complete_kernel<Source::Moe, VPT, Tail::Extra>}};
}
// [width slot: 2, 4, ..., 16 vectors per lane][partials: none, extra, residual; MoE picks: none, extra]
constexpr std::array<KernelFn, 5> kWaveComplete[kWaveWidths] = {
    wave_complete_row<2>(),  wave_complete_row<4>(),  wave_complete_row<6>(),  wave_complete_row<8>(),
    wave_complete_row<10>(), wave_complete_row<12>(), wave_complete_row<14>(), wave_complete_row<16>()};
static_assert(kWaveWidths == 8 && wave_slot(kWaveVptMax) == 7, "one table row per width");

// the 4-, 6- and 8-wide kernels with the deep ring (depth = width), by the same columns
template <int VPT>
constexpr std::array<KernelFn, 5> wave_complete_deep_row() {
  return {{&wave_complete_kernel<Source::Partials, VPT, Tail::None, VPT>,
           &wave_complete_kernel<Source::Partials, VPT, Tail::Extra, VPT>,
           &wave_complete_kernel<Source::Partials, VPT, Tail::Residual, VPT>,
           &wave_complete_kernel<Source::Moe, VPT, Tail::None, VPT>, &wave_complete_kernel<Source::Moe, VPT, Tail::Extra, VPT>}};
}
constexpr std::array<KernelFn, 5> kWaveCompleteDeep[kWaveDeepWidths] = {
    wave_complete_deep_row<4>(), wave_complete_deep_row<6>(), wave_complete_deep_row<8>()};

// the table column of a call, or -1 when it has no one-wavefront kernel
int wave_kind(Source src, Tail tail) {
  if (src == Source::Partials) return (int)tail;
  if (src == Source::Moe && tail != Tail::Residual) return 3 + (int)tail;
  return -1;
}

std::atomic<int> g_rows_per_cu[kWaveWidths][5];  // 0: not read yet, -1: unknown
std::atomic<int> g_deep_rows_per_cu[kWaveDeepWidths][5];
}  // namespace

int wave_complete_rows_per_cu(Source src, Tail tail, int vpt, bool deep) {
  const int kind = wave_kind(src, tail), w = wave_slot(vpt);
  const int d = deep_slot(vpt);
  if (kind < 0 || w < 0 || (deep && d < 0)) return 0;
  if (deep) return occupancy_rows(kWaveCompleteDeep[d][kind], g_deep_rows_per_cu[d][kind]);
  return occupancy_rows(kWaveComplete[w][kind], g_rows_per_cu[w][kind]);
}

hipError_t launch_complete_wave(Source src, int n, Tail tail, const RowArgs& a, const Launch& l,
                                hipStream_t stream) {
  const int kind = wave_kind(src, tail), w = wave_slot(l.vpt);
  if (!l.one_wave || w < 0 || kind < 0 || l.threads != kWave || a.nvec > kWave * l.vpt || n < 1 ||
      n > kMaxSources || (l.deep && deep_slot(l.vpt) < 0))
    return hipErrorInvalidValue;
  RowArgs b = a;
  b.nsrc = n;
  return launch_kernel(l.deep ? kWaveCompleteDeep[deep_slot(l.vpt)][kind] : kWaveComplete[w][kind], b, l, stream);
}

}  // namespace bnd
