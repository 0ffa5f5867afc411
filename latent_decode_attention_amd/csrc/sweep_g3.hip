// sweep_g3.hip -- attention kernels (uniform and ragged) for 3 query heads per KV head.
#include "sweep_impl.h"

namespace slimkv {
hipError_t launch_attention_g3(AttnArgs a, int dtype, int nch, hipStream_t s,
                                 hipEvent_t ev0, hipEvent_t ev1) {
  return launch_attention_group<3>(a, dtype, nch, s, ev0, ev1);
}
hipError_t launch_ragged_g3(AttnArgs a, int dtype, int nch, int64_t max_wgs, hipStream_t s,
                              hipEvent_t ev0, hipEvent_t ev1) {
  return launch_ragged_group<3>(a, dtype, nch, max_wgs, s, ev0, ev1);
}
int attention_slots_g3(int dtype, int nch, bool alibi) {
  return attention_slots_group<3>(dtype, nch, alibi);
}
}  // namespace slimkv
