// sweep_g8.hip -- attention kernels (uniform and ragged) for 8 query heads per KV head.
#include "sweep_impl.h"

namespace slimkv {
hipError_t launch_attention_g8(AttnArgs a, int dtype, int nch, hipStream_t s,
                                 hipEvent_t ev0, hipEvent_t ev1) {
  return launch_attention_group<8>(a, dtype, nch, s, ev0, ev1);
}
hipError_t launch_ragged_g8(AttnArgs a, int dtype, int nch, int64_t max_wgs, hipStream_t s,
                              hipEvent_t ev0, hipEvent_t ev1) {
  return launch_ragged_group<8>(a, dtype, nch, max_wgs, s, ev0, ev1);
}
int attention_slots_g8(int dtype, int nch, bool alibi) {
  return attention_slots_group<8>(dtype, nch, alibi);
}
}  // namespace slimkv
