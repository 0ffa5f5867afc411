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
// Rebuild (reconstruction comparison paths only): K_b = C_K U_K^T and
// V_b = C_V U_V^T for every (b, kv head), i.e. the full-dimension beacon keys
// and values the latent path never forms, rounded to the storage dtype.
// With a.pos (the variant that keeps beacon-key rotation, page "Can SlimKV
// compress KV cache jointly across tokens and features", section "Speedups
// are real, but memory is set by the ratio") rebuilt key row j is rotated at
// position pos[j] -- rotate-half pairs (i, i + d/2), angle pos * theta^(-2i/d)
// formed and reduced mod 2*pi in fp64, sine and cosine in fp32 -- before it
// is rounded.  One launch rebuilds both: job 0 the keys, job 1 the values.
//
// bf16 (MFMA 16x16x32): a workgroup takes 64 beacon rows of one KV head and
// walks the batch, so the head's basis (staged in LDS) and the rows'
// rotation are loaded and formed once and serve every sequence.  The basis
// is the A operand (basis row = output column on M, rank on K) and the
// transposed latent rows the B operand (rank on K, beacon row on N):
// lane (n, kg) then ends with columns 16t + 4kg .. +3 of row n for each
// 16-column tile t -- the two halves of every rotation pair in one lane.
// Each wave turns its 16 finished rows around in LDS, so that its stores
// write whole rows, 16 bytes per lane (four rows per store), with the
// non-temporal policy.  The latent
// rows of the next four sequences are in flight while one is multiplied.

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
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

constexpr int kRebuildRows = 64;  // beacon rows per workgroup (16 per wave)
constexpr int kUPad = 8;           // staged basis rows padded by 16 bytes (LDS banks)
constexpr int kRebuildAhead = 4;   // sequences whose latent rows are in flight per wave
constexpr int kOPitch = kHeadDim + 8;  // a wave's staged output rows (elements; padded)

template <int NCHK>
__global__ __launch_bounds__(kThreads, 2) void rebuild_bf16_kernel(RebuildArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ul[kHeadDim * (32 * NCHK + kUPad)];
  __shared__ __attribute__((aligned(16))) uint16_t ot[kWaves][16 * kOPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int nb = a.num_beacons, hkv = a.num_kv_heads;
  const int nblk = (nb + kRebuildRows - 1) / kRebuildRows;
  const int per_job = hkv * nblk;
  const int job = blockIdx.x / per_job;
  const int rem = blockIdx.x - job * per_job;
  const int h = rem / nblk, rb = rem - h * nblk;
  const int r = a.rank[job];
  const int nchk = (r + 31) / 32;  // workgroup-uniform
  const int us = r + kUPad;        // staged row stride (elements)
  const int row = rb * kRebuildRows + wave * 16 + n;
  const int rowc = row < nb ? row : nb - 1;  // loads stay in bounds; the store is skipped
  uint16_t* ow = ot[wave];

  const uint16_t* C = static_cast<const uint16_t*>(a.C[job]);
  uint16_t* D = static_cast<uint16_t*>(a.dst[job]);
  auto load_rows = [&](int b, bf16x8_t* cb) {
    const uint16_t* Cr = C + (((size_t)b * hkv + h) * nb + rowc) * r;
#pragma unroll
    for (int c = 0; c < NCHK; ++c) {
      const int k0 = 32 * c + 8 * kg;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (c < nchk && k0 < r) v = *reinterpret_cast<const u32x4_t*>(Cr + k0);
      cb[c] = __builtin_bit_cast(bf16x8_t, v);
    }
  };
  // the latent rows of the next kRebuildAhead sequences are in flight while
  // one is multiplied: a ring of buffers, indexed at compile time
  bf16x8_t ring[kRebuildAhead][NCHK];
#pragma unroll
  for (int i = 0; i < kRebuildAhead; ++i) load_rows(min(i, a.batch - 1), ring[i]);
  // the head's basis, staged once: row i (output column), rank k
  {
    const uint16_t* U = static_cast<const uint16_t*>(a.U[job]) + (size_t)h * kHeadDim * r;
    const int words = kHeadDim * r / 8, wpr = r / 8;
    for (int w = tid; w < words; w += kThreads) {
      const int i = w / wpr, k8 = w - i * wpr;
      *reinterpret_cast<u32x4_t*>(&ul[i * us + 8 * k8]) =
          *reinterpret_cast<const u32x4_t*>(U + (size_t)w * 8);
    }
  }
  // rotation of this lane's pairs (16t + 4kg + e, + d/2), t < 4 (keys with pos)
  const bool rot = job == 0 && a.pos != nullptr;
  float cs[4][4], sn[4][4];
  if (rot) {
    const int p = a.pos[rowc];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) rebuild_sincos(a, p, 16 * t + 4 * kg + e, sn[t][e], cs[t][e]);
  }
  __syncthreads();
  for (int b0 = 0; b0 < a.batch; b0 += kRebuildAhead) {
#pragma unroll
    for (int i = 0; i < kRebuildAhead; ++i) {
      const int b = b0 + i;
      if (b < a.batch) {  // workgroup-uniform
        bf16x8_t cur[NCHK];
#pragma unroll
        for (int c = 0; c < NCHK; ++c) cur[c] = ring[i][c];
        if (b + kRebuildAhead < a.batch) load_rows(b + kRebuildAhead, ring[i]);
        uint16_t* orow = ow + n * kOPitch + 4 * kg;
        // column tiles t and t + 4 together: they hold the two halves of this
        // lane's rotation pairs
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          f32x4_t d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int c = 0; c < NCHK; ++c) {
            if (c < nchk) {
              const int k0 = 32 * c + 8 * kg;
              u32x4_t a0 = {0u, 0u, 0u, 0u}, a1 = {0u, 0u, 0u, 0u};
              if (k0 < r) {
                a0 = *reinterpret_cast<const u32x4_t*>(&ul[(16 * t + n) * us + k0]);
                a1 = *reinterpret_cast<const u32x4_t*>(&ul[(16 * t + 64 + n) * us + k0]);
              }
              d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0), cur[c], d0, 0,
                                                           0, 0);
              d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), cur[c], d1, 0,
                                                           0, 0);
            }
          }
          if (rot) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = d0[e], y = d1[e];
              d0[e] = x * cs[t][e] - y * sn[t][e];
              d1[e] = y * cs[t][e] + x * sn[t][e];
            }
          }
          *reinterpret_cast<uint2*>(orow + 16 * t) =
              make_uint2(f32_to_bf16(d0[0]) | (f32_to_bf16(d0[1]) << 16),
                         f32_to_bf16(d0[2]) | (f32_to_bf16(d0[3]) << 16));
          *reinterpret_cast<uint2*>(orow + 16 * t + 64) =
              make_uint2(f32_to_bf16(d1[0]) | (f32_to_bf16(d1[1]) << 16),
                         f32_to_bf16(d1[2]) | (f32_to_bf16(d1[3]) << 16));
        }
        // the wave's 16 rows, read back row by row: store i writes rows
        // 4i .. 4i + 3, lane (row 4i + lane / 16) taking 8 columns
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        u32x4_t ov[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ov[i] = *reinterpret_cast<const u32x4_t*>(ow + (4 * i + (lane >> 4)) * kOPitch + 8 * (lane & 15));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int row0 = rb * kRebuildRows + wave * 16;
        uint16_t* Dw = D + (((size_t)b * hkv + h) * nb + row0) * kHeadDim + 8 * (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * i + (lane >> 4);
          if (row0 + rr < nb)  // streamed out (non-temporal): read once, by the next kernel
            __builtin_nontemporal_store(ov[i], reinterpret_cast<u32x4_t*>(Dw + (size_t)rr * kHeadDim));
        }
      }
    }
  }
}

// fp32: one thread per output element (the fp32 workloads are small).
__global__ __launch_bounds__(kThreads) void rebuild_f32_kernel(RebuildArgs a, int job) {
  const size_t total = (size_t)a.batch * a.num_kv_heads * a.num_beacons * kHeadDim;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const int col = (int)(idx % kHeadDim);
  const size_t row = idx / kHeadDim;  // global beacon row
  const size_t unit = row / a.num_beacons;
  const int h = (int)(unit % a.num_kv_heads);
  const int r = a.rank[job];
  const float* C = static_cast<const float*>(a.C[job]) + row * r;
  const float* U = static_cast<const float*>(a.U[job]) + ((size_t)h * kHeadDim + col) * r;
  float acc = 0.0f;
  for (int k = 0; k < r; ++k) acc = fmaf(C[k], U[k], acc);
  if (job == 0 && a.pos) {
    // the partner column i +- d/2 of the same row, rebuilt the same way
    const int pc = col ^ (kHeadDim / 2);
    const float* Up = static_cast<const float*>(a.U[job]) + ((size_t)h * kHeadDim + pc) * r;
    float pacc = 0.0f;
    for (int k = 0; k < r; ++k) pacc = fmaf(C[k], Up[k], pacc);
    float sn, cs;
    rebuild_sincos(a, a.pos[row % a.num_beacons], col & (kHeadDim / 2 - 1), sn, cs);
    acc = col < kHeadDim / 2 ? acc * cs - pacc * sn : acc * cs + pacc * sn;
  }
  static_cast<float*>(a.dst[job])[idx] = acc;
}

// ---------------------------------------------------------------------------
// The workspace check (SLIMKV_FLAG_CHECK_WORKSPACE).
__global__ __launch_bounds__(256) void workspace_check_kernel(uint32_t* ws, uint32_t begin,
                                                              uint32_t end) {
  bool found = false;
  for (uint32_t i = begin + blockIdx.x * 256u + threadIdx.x; i < end; i += gridDim.x * 256u) {
    if (ws[i] != 0u) {
      found = true;
      ws[i] = 0u;
    }
  }
  if (__builtin_amdgcn_ballot_w64(found) != 0 && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(&ws[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_workspace_check(uint32_t* ws, size_t begin, size_t end, hipStream_t s) {
  const uint32_t b = (uint32_t)(begin / 4), e = (uint32_t)(end / 4);
  const unsigned blocks = std::max(1u, std::min((e - b + 255u) / 256u, 256u));
  hipLaunchKernelGGL(workspace_check_kernel, dim3(blocks), dim3(256), 0, s, ws, b, e);
  return hipGetLastError();
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
    for (int job = 0; job < 2; ++job) {
      hipLaunchKernelGGL(rebuild_f32_kernel, grid, block, 0, s, a, job);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int nchk = std::max((a.rank[0] + 31) / 32, (a.rank[1] + 31) / 32);
  const dim3 grid((unsigned)(2 * a.num_kv_heads * ((a.num_beacons + kRebuildRows - 1) / kRebuildRows)));
  switch (nchk) {
    case 1: hipLaunchKernelGGL(rebuild_bf16_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(rebuild_bf16_kernel<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(rebuild_bf16_kernel<3>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(rebuild_bf16_kernel<4>, grid, block, 0, s, a); break;
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
