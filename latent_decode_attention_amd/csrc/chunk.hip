// chunk.hip -- the chunk kernels (several query tokens per sequence, bf16
// or fp32; capacity-sized or paged caches) and their launcher.
#include "sweep_impl.h"
#include "chunk_impl.h"
#include "chunk_f32_impl.h"

namespace slimkv {

template <bool PG, bool AL>
static const void* chunk_kernel_for(int nch) {
  switch (nch) {
    case 0: return reinterpret_cast<const void*>(&chunk_kernel<0, PG, AL>);
    case 1: return reinterpret_cast<const void*>(&chunk_kernel<1, PG, AL>);
    case 2: return reinterpret_cast<const void*>(&chunk_kernel<2, PG, AL>);
    case 3: return reinterpret_cast<const void*>(&chunk_kernel<3, PG, AL>);
    default: return reinterpret_cast<const void*>(&chunk_kernel<4, PG, AL>);
  }
}

template <bool PG, bool AL>
static const void* chunk_f32_kernel_for(bool lat) {
  return lat ? reinterpret_cast<const void*>(&chunk_f32_kernel<true, PG, AL>)
             : reinterpret_cast<const void*>(&chunk_f32_kernel<false, PG, AL>);
}

// P = a.chunks (> 0: as given; <= 0: the device's workgroup slots), at most
// kChunkMaxSlots and 64 per unit; the grid adds one block per unit, so the
// pieces (at most max(P, units)) fit the workspace's units + kChunkMaxSlots
// partial slots.
hipError_t launch_chunk(AttnArgs a, int dtype, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const bool lat = a.seg[0].kind == kSegLatent && a.seg[0].rows > 0;
  const int nch = lat ? std::max((a.seg[0].rk + 31) / 32, (a.seg[0].rv + 31) / 32) : 0;
  const bool paged = a.page_table[0] != nullptr || a.page_table[1] != nullptr;
  const bool alibi = a.alibi_slopes != nullptr;
  const void* kfn;
  if (dtype == 0)
    kfn = paged ? (alibi ? chunk_f32_kernel_for<true, true>(lat) : chunk_f32_kernel_for<true, false>(lat))
                : (alibi ? chunk_f32_kernel_for<false, true>(lat) : chunk_f32_kernel_for<false, false>(lat));
  else
    kfn = paged ? (alibi ? chunk_kernel_for<true, true>(nch) : chunk_kernel_for<true, false>(nch))
                : (alibi ? chunk_kernel_for<false, true>(nch) : chunk_kernel_for<false, false>(nch));
  const int64_t units = (int64_t)a.batch * a.num_kv_heads;
  int64_t P = a.chunks;
  if (P <= 0) {
    P = device_slots(kfn);
    if (P <= 0) return hipErrorInvalidDeviceFunction;
  }
  P = std::min<int64_t>(std::min<int64_t>(P, kChunkMaxSlots), units * kMaxChunks);
  a.chunks = (int32_t)P;
  const dim3 grid((unsigned)std::max<int64_t>(P, units)), block(kThreads);
  if (ev0) {
    const hipError_t err = hipEventRecord(ev0, s);
    if (err != hipSuccess) return err;
  }
  void* args[] = {&a};
  hipError_t err = hipLaunchKernel(kfn, grid, block, args, 0, s);
  if (err == hipSuccess) err = hipGetLastError();
  if (err == hipSuccess && ev1) return hipEventRecord(ev1, s);
  return err;
}

}  // namespace slimkv
