// sweep_g6.hip -- sweep kernels for 6 query heads per KV head.
#include "sweep_impl.h"

namespace slimkv {
hipError_t launch_sweep_g6(const SweepArgs& a, int dtype, int nch, hipStream_t s) {
  return launch_sweep_group<6>(a, dtype, nch, s);
}
}  // namespace slimkv
