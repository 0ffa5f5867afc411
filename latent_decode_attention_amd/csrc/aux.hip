// aux.hip -- the full-width beacon rebuild used only by the reconstruction
// comparison path, the tile-height rule, and the attention dispatcher.
#include <math.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

#include "internal.h"

namespace slimkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Rebuild (reconstruction comparison paths only): dst = C U^T per unit, i.e.
// the full-dimension beacon keys or values the latent path never forms,
// rounded to the storage dtype.  With a.pos (the variant that keeps
// beacon-key rotation, page "Can SlimKV compress KV cache jointly across
// tokens and features", section "Speedups are real, but memory is set by
// the ratio") row j is rotated at position pos[j] -- rotate-half pairs
// (i, i + d/2), angle pos * theta^(-2i/d) formed and reduced mod 2*pi in
// fp64, sine and cosine in fp32 -- before it is rounded.  bf16: one wave
// per 16 rows, MFMA 16x16x32 over 8 column tiles, staged through LDS in
// fp32 for 16-byte stores.

// Sine and cosine of pos * theta^(-2i/d) for pair i < 64 (see above).
__device__ __forceinline__ void rebuild_sincos(const RebuildArgs& a, int pos, int i, float& s,
                                               float& c) {
  double f = 1.0;
#pragma unroll
  for (int k = 0; k < 6; ++k) f *= ((i >> k) & 1) ? a.inv_freq_pow2[k] : 1.0;
  const double ang = (double)pos * f;
  constexpr double kTwoPiHi = 6.283185307179586232;
  constexpr double kTwoPiLo = 2.4492935982947064e-16;
  const double kk = rint(ang * 0.15915494309189534561);
  const double r = fma(-kk, kTwoPiLo, fma(-kk, kTwoPiHi, ang));
  sincosf((float)r, &s, &c);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(kThreads) void rebuild_bf16_kernel(RebuildArgs a) {
  constexpr int kPitch = kHeadDim + 4;  // fp32 elements per LDS row
  __shared__ __attribute__((aligned(16))) float tile[kWaves][16][kPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int nblk = (a.num_beacons + 63) / 64;
  const int unit = blockIdx.x / nblk;
  const int rb = blockIdx.x - unit * nblk;
  const int h = unit % a.num_kv_heads;
  const int r = a.rank;
  const int row0 = rb * 64 + wave * 16;
  const uint16_t* C = static_cast<const uint16_t*>(a.C) + (size_t)unit * a.num_beacons * r;
  const uint16_t* U = static_cast<const uint16_t*>(a.U) + (size_t)h * kHeadDim * r;
  uint16_t* D = static_cast<uint16_t*>(a.dst) + (size_t)unit * a.num_beacons * kHeadDim;
  const int nchk = (r + 31) / 32;

  bf16x8_t av[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int row = row0 + n, k0 = 32 * c + 8 * kg;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (c < nchk && row < a.num_beacons && k0 < r)
      v = *reinterpret_cast<const u32x4_t*>(C + (size_t)row * r + k0);
    av[c] = __builtin_bit_cast(bf16x8_t, v);
  }
#pragma unroll
  for (int nt = 0; nt < kHeadDim / 16; ++nt) {
    f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c < nchk) {
        const int col = nt * 16 + n, k0 = 32 * c + 8 * kg;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (k0 < r) v = *reinterpret_cast<const u32x4_t*>(U + (size_t)col * r + k0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[c], __builtin_bit_cast(bf16x8_t, v), d, 0, 0, 0);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[wave][4 * kg + e][nt * 16 + n] = d[e];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // each lane writes 8 columns of both halves of a row, i.e. the 8 rotation
  // pairs (i, i + d/2) of one row, whose angles it computes once
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = lane + 64 * j;
    const int row = idx >> 3, seg = idx & 7;
    if (row0 + row < a.num_beacons) {
      const float* t = &tile[wave][row][0];
      float lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = t[seg * 8 + e];
        hi[e] = t[seg * 8 + e + kHeadDim / 2];
      }
      if (a.pos) {
        const int p = a.pos[row0 + row];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float sn, cs;
          rebuild_sincos(a, p, seg * 8 + e, sn, cs);
          const float x = lo[e], y = hi[e];
          lo[e] = x * cs - y * sn;
          hi[e] = y * cs + x * sn;
        }
      }
      u32x4_t wl, wh;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wl[e] = (uint32_t)f32_to_bf16(lo[2 * e]) | ((uint32_t)f32_to_bf16(lo[2 * e + 1]) << 16);
        wh[e] = (uint32_t)f32_to_bf16(hi[2 * e]) | ((uint32_t)f32_to_bf16(hi[2 * e + 1]) << 16);
      }
      uint16_t* dst = D + (size_t)(row0 + row) * kHeadDim + seg * 8;
      *reinterpret_cast<u32x4_t*>(dst) = wl;
      *reinterpret_cast<u32x4_t*>(dst + kHeadDim / 2) = wh;
    }
  }
}

__global__ __launch_bounds__(kThreads) void rebuild_f32_kernel(RebuildArgs a) {
  const size_t total = (size_t)a.batch * a.num_kv_heads * a.num_beacons * kHeadDim;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const int col = (int)(idx % kHeadDim);
  const size_t row = idx / kHeadDim;  // global beacon row
  const size_t unit = row / a.num_beacons;
  const int h = (int)(unit % a.num_kv_heads);
  const int r = a.rank;
  const float* C = static_cast<const float*>(a.C) + row * r;
  const float* U = static_cast<const float*>(a.U) + ((size_t)h * kHeadDim + col) * r;
  float acc = 0.0f;
  for (int k = 0; k < r; ++k) acc = fmaf(C[k], U[k], acc);
  if (a.pos) {
    // the partner column i +- d/2 of the same row, rebuilt the same way
    const int pc = col ^ (kHeadDim / 2);
    const float* Up = static_cast<const float*>(a.U) + ((size_t)h * kHeadDim + pc) * r;
    float pacc = 0.0f;
    for (int k = 0; k < r; ++k) pacc = fmaf(C[k], Up[k], pacc);
    float sn, cs;
    rebuild_sincos(a, a.pos[row % a.num_beacons], col & (kHeadDim / 2 - 1), sn, cs);
    acc = col < kHeadDim / 2 ? acc * cs - pacc * sn : acc * cs + pacc * sn;
  }
  static_cast<float*>(a.dst)[idx] = acc;
}

// ---------------------------------------------------------------------------
int tile_rows(int dtype, int rk, int rv) {
  if (dtype == 0) return 16;
  int nch = (rk + 31) / 32;
  const int nv = (rv + 31) / 32;
  if (nv > nch) nch = nv;
  return nch == 1 ? 64 : (nch == 2 ? 32 : 16);
}

hipError_t launch_rebuild(const RebuildArgs& a, int dtype, hipStream_t s) {
  const dim3 block(kThreads);
  if (dtype == 0) {
    const size_t total = (size_t)a.batch * a.num_kv_heads * a.num_beacons * kHeadDim;
    const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(rebuild_f32_kernel, grid, block, 0, s, a);
  } else {
    const dim3 grid((unsigned)(a.batch * a.num_kv_heads * ((a.num_beacons + 63) / 64)));
    hipLaunchKernelGGL(rebuild_bf16_kernel, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

int choose_chunks(int64_t units, int64_t unit_bytes, int64_t slots, int64_t min_chunk_bytes) {
  int best = 1;
  double best_fill = -1.0;
  for (int k = 1; k <= kMaxChunks; ++k) {
    if (k > 1 && unit_bytes / k < min_chunk_bytes) break;
    const int64_t wgs = units * k;
    const int64_t rounds = (wgs + slots - 1) / slots;
    const double fill = (double)wgs / (double)(rounds * slots);
    if (fill > best_fill + 1e-9) {  // ties keep the smaller k
      best = k;
      best_fill = fill;
    }
  }
  return best;
}

int device_slots(const void* kfn) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const std::pair<int, const void*> key(dev, kfn);
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, kThreads, 0) != hipSuccess)
    return -1;
  // Two resident workgroups per CU at most: 8 waves per CU, each with one
  // tile (~8 KB) in flight, already keep HBM saturated; a third workgroup
  // only lengthens the memory queues, and the latency that adds is paid by
  // every call's ramp-up and by its merge at the end (measured on MI355X:
  // 70 vs 75 us per call on a 128K, 16x, batch-16 Llama-8B layer).
  const int slots = cus * std::min(per_cu > 0 ? per_cu : 1, kWgPerCu);
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = slots;
  return slots;
}

hipError_t launch_attention_g1(AttnArgs, int, int, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_attention_g2(AttnArgs, int, int, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_attention_g3(AttnArgs, int, int, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_attention_g4(AttnArgs, int, int, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_attention_g5(AttnArgs, int, int, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_attention_g6(AttnArgs, int, int, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_attention_g7(AttnArgs, int, int, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_attention_g8(AttnArgs, int, int, hipStream_t, hipEvent_t, hipEvent_t);

hipError_t launch_ragged_g1(AttnArgs, int, int, int64_t, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_ragged_g2(AttnArgs, int, int, int64_t, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_ragged_g3(AttnArgs, int, int, int64_t, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_ragged_g4(AttnArgs, int, int, int64_t, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_ragged_g5(AttnArgs, int, int, int64_t, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_ragged_g6(AttnArgs, int, int, int64_t, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_ragged_g7(AttnArgs, int, int, int64_t, hipStream_t, hipEvent_t, hipEvent_t);
hipError_t launch_ragged_g8(AttnArgs, int, int, int64_t, hipStream_t, hipEvent_t, hipEvent_t);

// MFMA chunks of a latent beacon segment's rows (0: full width, or none)
static int beacon_chunks(const AttnArgs& a) {
  if (a.seg[0].kind != kSegLatent || a.seg[0].rows <= 0) return 0;
  return std::max((a.seg[0].rk + 31) / 32, (a.seg[0].rv + 31) / 32);
}

hipError_t launch_ragged(AttnArgs a, int dtype, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int nch = beacon_chunks(a);
  // partial slots: one per (workgroup, unit) piece, rank + unit < grid + units
  const int64_t max_wgs = (int64_t)a.batch * a.num_kv_heads * kMaxChunks;
  switch (a.group) {
    case 1: return launch_ragged_g1(a, dtype, nch, max_wgs, s, ev0, ev1);
    case 2: return launch_ragged_g2(a, dtype, nch, max_wgs, s, ev0, ev1);
    case 3: return launch_ragged_g3(a, dtype, nch, max_wgs, s, ev0, ev1);
    case 4: return launch_ragged_g4(a, dtype, nch, max_wgs, s, ev0, ev1);
    case 5: return launch_ragged_g5(a, dtype, nch, max_wgs, s, ev0, ev1);
    case 6: return launch_ragged_g6(a, dtype, nch, max_wgs, s, ev0, ev1);
    case 7: return launch_ragged_g7(a, dtype, nch, max_wgs, s, ev0, ev1);
    default: return launch_ragged_g8(a, dtype, nch, max_wgs, s, ev0, ev1);
  }
}

int attention_slots_g1(int, int, bool);
int attention_slots_g2(int, int, bool);
int attention_slots_g3(int, int, bool);
int attention_slots_g4(int, int, bool);
int attention_slots_g5(int, int, bool);
int attention_slots_g6(int, int, bool);
int attention_slots_g7(int, int, bool);
int attention_slots_g8(int, int, bool);

int attention_slots(const AttnArgs& a, int dtype) {
  const int nch = beacon_chunks(a);
  const bool alibi = a.alibi_slopes != nullptr;
  switch (a.group) {
    case 1: return attention_slots_g1(dtype, nch, alibi);
    case 2: return attention_slots_g2(dtype, nch, alibi);
    case 3: return attention_slots_g3(dtype, nch, alibi);
    case 4: return attention_slots_g4(dtype, nch, alibi);
    case 5: return attention_slots_g5(dtype, nch, alibi);
    case 6: return attention_slots_g6(dtype, nch, alibi);
    case 7: return attention_slots_g7(dtype, nch, alibi);
    default: return attention_slots_g8(dtype, nch, alibi);
  }
}

hipError_t launch_attention(AttnArgs a, int dtype, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int nch = beacon_chunks(a);  // 0: beacon rows at full width, or none
  switch (a.group) {
    case 1: return launch_attention_g1(a, dtype, nch, s, ev0, ev1);
    case 2: return launch_attention_g2(a, dtype, nch, s, ev0, ev1);
    case 3: return launch_attention_g3(a, dtype, nch, s, ev0, ev1);
    case 4: return launch_attention_g4(a, dtype, nch, s, ev0, ev1);
    case 5: return launch_attention_g5(a, dtype, nch, s, ev0, ev1);
    case 6: return launch_attention_g6(a, dtype, nch, s, ev0, ev1);
    case 7: return launch_attention_g7(a, dtype, nch, s, ev0, ev1);
    default: return launch_attention_g8(a, dtype, nch, s, ev0, ev1);
  }
}

}  // namespace slimkv
