// complete_only: the owed sum alone (P partials or k MoE picks), stored bf16.
#include "kernels.h"

namespace bnd {

namespace {
using Seq = std::make_integer_sequence<int, kMaxSources>;
constexpr std::array<std::array<KernelFn, kMaxSources>, 3> kPartials = {
    complete_table<Source::Partials, 1>(Seq{}), complete_table<Source::Partials, 2>(Seq{}),
    complete_table<Source::Partials, 4>(Seq{})};
constexpr std::array<std::array<KernelFn, kMaxSources>, 3> kMoe = {
    complete_table<Source::Moe, 1>(Seq{}), complete_table<Source::Moe, 2>(Seq{}),
    complete_table<Source::Moe, 4>(Seq{})};
}  // namespace

hipError_t launch_complete(Source src, int n, const RowArgs& a, const Launch& l, hipStream_t stream) {
  const int slot = vpt_slot(l.vpt);
  if (slot < 0 || n < 1 || n > kMaxSources) return hipErrorInvalidValue;
  if (src == Source::Partials) return launch_kernel(kPartials[slot][n - 1], a, l, stream);
  if (src == Source::Moe) return launch_kernel(kMoe[slot][n - 1], a, l, stream);
  return hipErrorInvalidValue;
}

}  // namespace bnd
