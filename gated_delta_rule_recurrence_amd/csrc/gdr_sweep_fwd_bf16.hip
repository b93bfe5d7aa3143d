// Instantiates the forward sweep kernels for bf16 inputs (see gdr_sweep.h).
#include "gdr_sweep.h"

namespace gdr {

hipError_t launch_fwd_sweep_bf16(const FwdSweepArgs& a, int num_cu, hipStream_t s) {
  return sweep::fwd_dispatch<gdr::bf16>(a, num_cu, s);
}

}  // namespace gdr
