// Boundary reads whose owed work is a deferred MoE finalize (k = 1..16
// gathered expert rows), bf16 output, for 1, 2 or 4 vectors per thread.
#include "kernels.h"

namespace bnd {

namespace {
using Seq = std::make_integer_sequence<int, kMaxSources>;
constexpr std::array<std::array<KernelFn, kMaxSources>, 3> kBf16 = {
    read_table<Source::Moe, 1, false>(Seq{}), read_table<Source::Moe, 2, false>(Seq{}),
    read_table<Source::Moe, 4, false>(Seq{})};
// one vector per thread with non-temporal stores (launches of fewer rows than CUs)
constexpr std::array<KernelFn, kMaxSources> kBf16Nt = read_table<Source::Moe, 1, false, true>(Seq{});
}  // namespace

hipError_t launch_read_moe(int n, const RowArgs& a, const Launch& l, hipStream_t stream) {
  const int slot = vpt_slot(l.vpt);
  if (slot < 0 || n < 1 || n > kMaxSources || (l.nt_stores && l.vpt != 1)) return hipErrorInvalidValue;
  return launch_kernel(l.nt_stores ? kBf16Nt[n - 1] : kBf16[slot][n - 1], a, l, stream);
}

}  // namespace bnd
