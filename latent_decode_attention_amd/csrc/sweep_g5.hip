// sweep_g5.hip -- sweep kernels for 5 query heads per KV head.
#include "sweep_impl.h"

namespace slimkv {
hipError_t launch_sweep_g5(const SweepArgs& a, int dtype, int nch, hipStream_t s) {
  return launch_sweep_group<5>(a, dtype, nch, s);
}
}  // namespace slimkv
