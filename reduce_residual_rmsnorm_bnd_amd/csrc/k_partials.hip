// Boundary reads whose owed work is P plain partials (P = 1..16), with bf16
// or fp8 output, for 1, 2 or 4 vectors per thread.
#include "kernels.h"

namespace bnd {

namespace {
using Seq = std::make_integer_sequence<int, kMaxSources>;
constexpr std::array<std::array<KernelFn, kMaxSources>, 3> kBf16 = {
    read_table<Source::Partials, 1, false>(Seq{}), read_table<Source::Partials, 2, false>(Seq{}),
    read_table<Source::Partials, 4, false>(Seq{})};
constexpr std::array<std::array<KernelFn, kMaxSources>, 3> kFp8 = {
    read_table<Source::Partials, 1, true>(Seq{}), read_table<Source::Partials, 2, true>(Seq{}),
    read_table<Source::Partials, 4, true>(Seq{})};
// one vector per thread with non-temporal stores (launches of fewer rows than CUs), bf16 and fp8
constexpr std::array<std::array<KernelFn, kMaxSources>, 2> kNt = {
    read_table<Source::Partials, 1, false, true>(Seq{}), read_table<Source::Partials, 1, true, true>(Seq{})};
}  // namespace

hipError_t launch_read_partials(int n, bool fp8, const RowArgs& a, const Launch& l, hipStream_t stream) {
  const int slot = vpt_slot(l.vpt);
  if (slot < 0 || n < 1 || n > kMaxSources || (l.nt_stores && l.vpt != 1)) return hipErrorInvalidValue;
  if (l.nt_stores) return launch_kernel(kNt[fp8 ? 1 : 0][n - 1], a, l, stream);
  return launch_kernel((fp8 ? kFp8 : kBf16)[slot][n - 1], a, l, stream);
}

}  // namespace bnd
