// sweep_g3.hip -- sweep kernels for 3 query heads per KV head.
#include "sweep_impl.h"

namespace slimkv {
hipError_t launch_sweep_g3(const SweepArgs& a, int dtype, int nch, hipStream_t s) {
  return launch_sweep_group<3>(a, dtype, nch, s);
}
}  // namespace slimkv
