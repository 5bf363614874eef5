// One wavefront per row: folds of P plain partials with fp8 output, P = 1..16.
#include "kernels.h"

namespace bnd {

namespace {
using Seq = std::make_integer_sequence<int, kMaxSources>;
constexpr std::array<KernelFn, kMaxSources> kTable = wave_table<Source::Partials, true>(Seq{});
}  // namespace

// n in 1..16, checked by the caller
KernelFn wave_kernel_partials_fp8(int n) { return kTable[n - 1]; }

}  // namespace bnd
