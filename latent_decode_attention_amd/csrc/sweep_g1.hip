// sweep_g1.hip -- sweep kernels for 1 query head per KV head.
#include "sweep_impl.h"

namespace slimkv {
hipError_t launch_sweep_g1(const SweepArgs& a, int dtype, int nch, hipStream_t s) {
  return launch_sweep_group<1>(a, dtype, nch, s);
}
}  // namespace slimkv
