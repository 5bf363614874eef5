// One wavefront per row: MoE finalize folds of k gathered picks, bf16 output,
// k = 1..16.
#include "kernels.h"

namespace bnd {

namespace {
using Seq = std::make_integer_sequence<int, kMaxSources>;
constexpr std::array<KernelFn, kMaxSources> kTable = wave_table<Source::Moe, false>(Seq{});
}  // namespace

// n in 1..16, checked by the caller
KernelFn wave_kernel_moe(int n) { return kTable[n - 1]; }

}  // namespace bnd
