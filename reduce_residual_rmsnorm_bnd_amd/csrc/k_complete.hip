// complete_only and add_to_output (the owed sum of P partials or k MoE picks,
// plus an optional extra row, stored bf16) and snapshot (residual plus the sum
// of P partials, or a copy of the residual, stored bf16 into a separate output),
// with the multi-wave row shapes or one wavefront per row.
#include "kernels.h"

namespace bnd {

namespace {
using Seq = std::make_integer_sequence<int, kMaxSources>;
constexpr std::array<std::array<KernelFn, kMaxSources>, 3> kPartials = {
    complete_table<Source::Partials, 1, false>(Seq{}), complete_table<Source::Partials, 2, false>(Seq{}),
    complete_table<Source::Partials, 4, false>(Seq{})};
constexpr std::array<std::array<KernelFn, kMaxSources>, 3> kPartialsFold = {
    complete_table<Source::Partials, 1, true>(Seq{}), complete_table<Source::Partials, 2, true>(Seq{}),
    complete_table<Source::Partials, 4, true>(Seq{})};
constexpr std::array<std::array<KernelFn, kMaxSources>, 3> kMoe = {
    complete_table<Source::Moe, 1, false>(Seq{}), complete_table<Source::Moe, 2, false>(Seq{}),
    complete_table<Source::Moe, 4, false>(Seq{})};
constexpr KernelFn kCopy[3] = {&complete_kernel<Source::Residual, 0, 1, true>,
                               &complete_kernel<Source::Residual, 0, 2, true>,
                               &complete_kernel<Source::Residual, 0, 4, true>};
template <int VPT>
constexpr std::array<KernelFn, 5> wave_complete_table() {
  return {{&wave_complete_kernel<Source::Partials, VPT, Tail::None>,
           &wave_complete_kernel<Source::Partials, VPT, Tail::Extra>,
           &wave_complete_kernel<Source::Partials, VPT, Tail::Residual>,
           &wave_complete_kernel<Source::Moe, VPT, Tail::None>, &wave_complete_kernel<Source::Moe, VPT, Tail::Extra>}};
}
// [vectors per lane: 8, 14][partials: none, extra, residual; MoE picks: none, extra]
constexpr std::array<KernelFn, 5> kWaveComplete[2] = {wave_complete_table<kWaveVpt>(),
                                                      wave_complete_table<kWaveVptWide>()};

// the table slot of a call, or -1 when it has no one-wavefront kernel
int wave_kind(Source src, Tail tail) {
  if (src == Source::Partials) return (int)tail;
  if (src == Source::Moe && tail != Tail::Residual) return 3 + (int)tail;
  return -1;
}

hipError_t launch_complete_wave(Source src, int n, Tail tail, const RowArgs& a, const Launch& l,
                                hipStream_t stream) {
  const bool wide = l.vpt == kWaveVptWide;
  if ((l.vpt != kWaveVpt && !wide) || l.threads != kWave || a.nvec > kWave * l.vpt || n < 1 || n > kMaxSources)
    return hipErrorInvalidValue;
  const int kind = wave_kind(src, tail);
  if (kind < 0) return hipErrorInvalidValue;
  RowArgs b = a;
  b.nsrc = n;
  return launch_kernel(kWaveComplete[wide ? 1 : 0][kind], b, l, stream);
}

std::atomic<int> g_rows_per_cu[2][5];  // 0: not read yet, -1: unknown
}  // namespace

int wave_complete_rows_per_cu(Source src, Tail tail, int vpt) {
  const int kind = wave_kind(src, tail);
  if (kind < 0 || (vpt != kWaveVpt && vpt != kWaveVptWide)) return 0;
  const int w = vpt == kWaveVptWide ? 1 : 0;
  return occupancy_rows(kWaveComplete[w][kind], g_rows_per_cu[w][kind]);
}

hipError_t launch_complete(Source src, int n, bool fold, const RowArgs& a, const Launch& l, hipStream_t stream) {
  if (l.vpt == kWaveVpt || l.vpt == kWaveVptWide)
    return launch_complete_wave(src, n, fold ? Tail::Residual : a.extra ? Tail::Extra : Tail::None, a, l, stream);
  const int slot = vpt_slot(l.vpt);
  if (slot < 0) return hipErrorInvalidValue;
  if (src == Source::Residual) return fold ? launch_kernel(kCopy[slot], a, l, stream) : hipErrorInvalidValue;
  if (n < 1 || n > kMaxSources) return hipErrorInvalidValue;
  if (src == Source::Partials) return launch_kernel((fold ? kPartialsFold : kPartials)[slot][n - 1], a, l, stream);
  if (src == Source::Moe && !fold) return launch_kernel(kMoe[slot][n - 1], a, l, stream);
  return hipErrorInvalidValue;
}

}  // namespace bnd
