// Instantiates the reverse sweep kernels for f32 inputs (see gdr_sweep.h).
#include "gdr_sweep.h"

namespace gdr {

hipError_t launch_bwd_sweep_f32(const BwdSweepArgs& a, int num_cu, hipStream_t s) {
  return sweep::bwd_dispatch<float>(a, num_cu, s);
}

}  // namespace gdr
