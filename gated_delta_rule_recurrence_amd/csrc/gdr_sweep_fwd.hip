// The per-step forward sweep (gdr_sweep.h) for fp32 and bf16 inputs, and its
// launch.  The reverse sweep has a file of its own (gdr_sweep_bwd.hip) so
// that the two compile side by side.
#include "gdr_sweep.h"

namespace gdr {

hipError_t launch_fwd_sweep(const FwdSweepArgs& a, bool bf16, hipStream_t s) {
  const int cu = device_cu_count();
  return bf16 ? sweep::fwd_dispatch<gdr::bf16>(a, cu, s) : sweep::fwd_dispatch<float>(a, cu, s);
}

}  // namespace gdr
