// The per-step reverse sweep (gdr_sweep.h) for fp32 and bf16 inputs, and its
// launch.
#include "gdr_sweep.h"

namespace gdr {

hipError_t launch_bwd_sweep(const BwdSweepArgs& a, bool bf16, hipStream_t s) {
  const int cu = device_cu_count();
  return bf16 ? sweep::bwd_dispatch<gdr::bf16>(a, cu, s) : sweep::bwd_dispatch<float>(a, cu, s);
}

}  // namespace gdr
