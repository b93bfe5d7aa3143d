// Instantiates the forward sweep kernels for f32 inputs (see gdr_sweep.h).
#include "gdr_sweep.h"

namespace gdr {

hipError_t launch_fwd_sweep_f32(const FwdSweepArgs& a, int num_cu, hipStream_t s) {
  return sweep::fwd_dispatch<float>(a, num_cu, s);
}

}  // namespace gdr
