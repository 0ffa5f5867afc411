// sweep_g7.hip -- sweep kernels for 7 query heads per KV head.
#include "sweep_impl.h"

namespace slimkv {
hipError_t launch_sweep_g7(const SweepArgs& a, int dtype, int nch, hipStream_t s) {
  return launch_sweep_group<7>(a, dtype, nch, s);
}
}  // namespace slimkv
