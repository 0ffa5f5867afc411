// bench_kernels.hip -- measurement helpers declared in include/slimkv_bench.h:
// a plain streaming-read kernel (the ceiling an attention call that streams
// the same bytes can be compared with) and a cache flush.  Neither computes
// any part of the attention.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "slimkv_bench.h"

namespace slimkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Cache policy of the reads: non-temporal, as for the attention kernels'
// cache rows (each byte is read once).
constexpr int kNonTemporal = 2;

// F 16-byte loads in flight per lane: iteration i of thread t reads words
// (i * F + f) * nthreads + t, f < F, so each load instruction of a wave
// covers 1 KB of consecutive bytes and the wave's F loads are independent.
// Words past the end read as zeros through the buffer descriptor's bound.
template <int F>
__global__ __launch_bounds__(256) void stream_read_kernel(const void* src, uint32_t bytes,
                                                          uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), 0, (int)bytes, 0x00020000);
  const uint32_t nthreads = gridDim.x * 256u;
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  const uint32_t words = bytes / 16u;
  uint32_t x = 0;
  for (uint32_t w0 = 0; w0 < words; w0 += F * nthreads) {
    u32x4_t v[F];
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const uint32_t w = w0 + (uint32_t)f * nthreads + t;
      // past the end (w >= words) the offset lies beyond the bound: zeros
      const uint32_t off = w < words ? w * 16u : bytes;
      v[f] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNonTemporal);
    }
#pragma unroll
    for (int f = 0; f < F; ++f) x ^= v[f][0] ^ v[f][1] ^ v[f][2] ^ v[f][3];
  }
  // one checksum per workgroup: xor over the wave, then one atomic per wave
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m);
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_xor(sink, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void flush_kernel(u32x4_t* buf, size_t words, uint32_t seed) {
  const size_t nthreads = (size_t)gridDim.x * 256u;
  for (size_t w = (size_t)blockIdx.x * 256u + threadIdx.x; w < words; w += nthreads) {
    const uint32_t s = seed ^ (uint32_t)w;
    buf[w] = u32x4_t{s, s + 1u, s + 2u, s + 3u};
  }
}

int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

}  // namespace
}  // namespace slimkv

extern "C" {

slimkv_status slimkv_bench_stream_read(const void* src, size_t bytes, int32_t in_flight,
                                       int32_t workgroups, uint32_t* sink, void* stream) {
  using namespace slimkv;
  if (!src || !sink) return SLIMKV_ERR_NULL;
  if ((uintptr_t)src % 16 != 0 || (uintptr_t)sink % 4 != 0) return SLIMKV_ERR_ALIGN;
  if (bytes < 16 || bytes % 16 != 0 || bytes > ((size_t)1 << 31) - 16) return SLIMKV_ERR_SHAPE;
  if (in_flight != 1 && in_flight != 2 && in_flight != 4 && in_flight != 8 && in_flight != 16)
    return SLIMKV_ERR_UNSUPPORTED;
  if (workgroups < 0 || workgroups > 65536) return SLIMKV_ERR_SHAPE;
  const uintptr_t s0 = (uintptr_t)src, s1 = s0 + bytes, k0 = (uintptr_t)sink;
  if (k0 + 4 > s0 && k0 < s1) return SLIMKV_ERR_ALIAS;
  int wgs = workgroups;
  if (wgs == 0) {
    const int cus = cu_count();
    if (cus <= 0) return SLIMKV_ERR_HIP;
    wgs = 2 * cus;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)wgs), block(256);
  const uint32_t b = (uint32_t)bytes;
  switch (in_flight) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, grid, block, 0, s, src, b, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, grid, block, 0, s, src, b, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, s, src, b, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, s, src, b, sink); break;
    default: hipLaunchKernelGGL(stream_read_kernel<16>, grid, block, 0, s, src, b, sink); break;
  }
  return hipGetLastError() == hipSuccess ? SLIMKV_OK : SLIMKV_ERR_HIP;
}

slimkv_status slimkv_bench_flush(void* buf, size_t bytes, uint32_t seed, void* stream) {
  using namespace slimkv;
  if (!buf) return SLIMKV_ERR_NULL;
  if ((uintptr_t)buf % 16 != 0) return SLIMKV_ERR_ALIGN;
  if (bytes < 16 || bytes % 16 != 0) return SLIMKV_ERR_SHAPE;
  const int cus = cu_count();
  if (cus <= 0) return SLIMKV_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(flush_kernel, dim3((unsigned)(4 * cus)), dim3(256), 0, s,
                     static_cast<u32x4_t*>(buf), bytes / 16, seed);
  return hipGetLastError() == hipSuccess ? SLIMKV_OK : SLIMKV_ERR_HIP;
}

}  // extern "C"
