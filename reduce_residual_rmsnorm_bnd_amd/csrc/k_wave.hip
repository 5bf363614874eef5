// Boundary reads with one wavefront per row (64 lanes x 8 or 14 vectors):
// folds of P plain partials with bf16 or fp8 output, and MoE finalize folds
// of k gathered picks with bf16 output; P and k (1..16) are runtime values.
#include "kernels.h"

namespace bnd {

namespace {
// [vectors per lane: 8, 14][partials bf16, partials fp8, MoE bf16]
constexpr KernelFn kWaveKernels[2][3] = {
    {&wave_read_kernel<Source::Partials, kWaveVpt, false>, &wave_read_kernel<Source::Partials, kWaveVpt, true>,
     &wave_read_kernel<Source::Moe, kWaveVpt, false>},
    {&wave_read_kernel<Source::Partials, kWaveVptWide, false>,
     &wave_read_kernel<Source::Partials, kWaveVptWide, true>, &wave_read_kernel<Source::Moe, kWaveVptWide, false>}};

// the table slot of a call, or -1 when it has no one-wavefront kernel
int wave_kind(Source src, bool fp8) {
  if (src == Source::Partials) return fp8 ? 1 : 0;
  if (src == Source::Moe && !fp8) return 2;
  return -1;
}

std::atomic<int> g_rows_per_cu[2][3];  // 0: not read yet, -1: unknown
}  // namespace

int wave_read_rows_per_cu(Source src, bool fp8, int vpt) {
  const int kind = wave_kind(src, fp8);
  if (kind < 0 || (vpt != kWaveVpt && vpt != kWaveVptWide)) return 0;
  const int w = vpt == kWaveVptWide ? 1 : 0;
  return occupancy_rows(kWaveKernels[w][kind], g_rows_per_cu[w][kind]);
}

hipError_t launch_read_wave(Source src, int n, bool fp8, const RowArgs& a, const Launch& l, hipStream_t stream) {
  const bool wide = l.vpt == kWaveVptWide;
  if ((l.vpt != kWaveVpt && !wide) || l.threads != kWave || a.nvec > kWave * l.vpt || n < 1 || n > kMaxSources)
    return hipErrorInvalidValue;
  const int kind = wave_kind(src, fp8);
  if (kind < 0) return hipErrorInvalidValue;
  RowArgs b = a;
  b.nsrc = n;
  return launch_kernel(kWaveKernels[wide ? 1 : 0][kind], b, l, stream);
}

}  // namespace bnd
