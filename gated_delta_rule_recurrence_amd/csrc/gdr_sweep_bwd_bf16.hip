// Instantiates the reverse sweep kernels for bf16 inputs (see gdr_sweep.h).
#include "gdr_sweep.h"

namespace gdr {

hipError_t launch_bwd_sweep_bf16(const BwdSweepArgs& a, int num_cu, hipStream_t s) {
  return sweep::bwd_dispatch<gdr::bf16>(a, num_cu, s);
}

}  // namespace gdr
