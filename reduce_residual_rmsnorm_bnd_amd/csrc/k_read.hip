// Reads without owed work (enter from Initial, read of a Written stream) and
// the dispatcher of every boundary read.
#include "kernels.h"

namespace bnd {

hipError_t launch_read_partials(int n, bool fp8, const RowArgs& a, const Launch& l, hipStream_t stream);
hipError_t launch_read_moe(int n, const RowArgs& a, const Launch& l, hipStream_t stream);

namespace {
// enter (bf16 output only: the stack input's read has no fp8 form), by vpt slot
constexpr KernelFn kInput[3] = {&read_kernel<Source::Input, 0, 1, false>, &read_kernel<Source::Input, 0, 2, false>,
                                &read_kernel<Source::Input, 0, 4, false>};
// the read of a Written stream: [vpt slot][bf16, fp8]
constexpr KernelFn kResidual[3][2] = {
    {&read_kernel<Source::Residual, 0, 1, false>, &read_kernel<Source::Residual, 0, 1, true>},
    {&read_kernel<Source::Residual, 0, 2, false>, &read_kernel<Source::Residual, 0, 2, true>},
    {&read_kernel<Source::Residual, 0, 4, false>, &read_kernel<Source::Residual, 0, 4, true>}};
// one vector per thread with non-temporal stores (launches of fewer rows than CUs)
constexpr KernelFn kInputNt = &read_kernel<Source::Input, 0, 1, false, true>;
constexpr KernelFn kResidualNt[2] = {&read_kernel<Source::Residual, 0, 1, false, true>,
                                     &read_kernel<Source::Residual, 0, 1, true, true>};
}  // namespace

hipError_t launch_read(Source src, int n, bool fp8, const RowArgs& a, const Launch& l, hipStream_t stream) {
  if (l.one_wave) return launch_read_wave(src, n, fp8, a, l, stream);
  switch (src) {
    case Source::Partials:
      return launch_read_partials(n, fp8, a, l, stream);
    case Source::Moe:
      if (fp8) return hipErrorInvalidValue;
      return launch_read_moe(n, a, l, stream);
    case Source::Input: {
      const int slot = vpt_slot(l.vpt);
      if (fp8 || slot < 0 || (l.nt_stores && l.vpt != 1)) return hipErrorInvalidValue;
      return launch_kernel(l.nt_stores ? kInputNt : kInput[slot], a, l, stream);
    }
    case Source::Residual: {
      const int slot = vpt_slot(l.vpt);
      if (slot < 0 || (l.nt_stores && l.vpt != 1)) return hipErrorInvalidValue;
      return launch_kernel(l.nt_stores ? kResidualNt[fp8 ? 1 : 0] : kResidual[slot][fp8 ? 1 : 0], a, l, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace bnd
