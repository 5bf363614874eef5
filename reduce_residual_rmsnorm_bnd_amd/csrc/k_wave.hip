// Boundary reads with one wavefront per row (64 lanes x 8 vectors): the
// dispatcher, and folds of P plain partials with bf16 output, P = 1..16.
// fp8 output and MoE picks are instantiated in k_wave_fp8.hip and
// k_wave_moe.hip (compiled in parallel).
#include "kernels.h"

namespace bnd {

KernelFn wave_kernel_partials_fp8(int n);
KernelFn wave_kernel_moe(int n);

namespace {
using Seq = std::make_integer_sequence<int, kMaxSources>;
constexpr std::array<KernelFn, kMaxSources> kPartialsBf16 = wave_table<Source::Partials, false>(Seq{});
}  // namespace

hipError_t launch_read_wave(Source src, int n, bool fp8, const RowArgs& a, const Launch& l, hipStream_t stream) {
  if (l.vpt != kWaveVpt || l.threads != kWave || a.nvec > kWave * kWaveVpt || n < 1 || n > kMaxSources)
    return hipErrorInvalidValue;
  if (src == Source::Partials)
    return launch_kernel(fp8 ? wave_kernel_partials_fp8(n) : kPartialsBf16[n - 1], a, l, stream);
  if (src == Source::Moe && !fp8) return launch_kernel(wave_kernel_moe(n), a, l, stream);
  return hipErrorInvalidValue;
}

}  // namespace bnd
