// sweep_g2.hip -- sweep kernels for 2 query heads per KV head.
#include "sweep_impl.h"

namespace slimkv {
hipError_t launch_sweep_g2(const SweepArgs& a, int dtype, int nch, hipStream_t s) {
  return launch_sweep_group<2>(a, dtype, nch, s);
}
}  // namespace slimkv
