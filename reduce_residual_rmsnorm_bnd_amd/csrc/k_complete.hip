// complete_only and add_to_output (the owed sum of P partials or k MoE picks,
// plus an optional extra row, stored bf16) and snapshot (residual plus the sum
// of P partials, or a copy of the residual, stored bf16 into a separate output)
// with several wavefronts per row; the one-wavefront forms are in
// k_wave_complete.hip.
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
}  // namespace

hipError_t launch_complete(Source src, int n, bool fold, const RowArgs& a, const Launch& l, hipStream_t stream) {
  if (l.one_wave)
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
