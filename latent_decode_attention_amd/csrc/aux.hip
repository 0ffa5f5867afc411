// aux.hip -- the kernels around the sweep: query prologue, split merge with
// the single up-projection, and the full-width beacon rebuild used only by
// the reconstruction comparison path.
#include <math.h>

#include "internal.h"

namespace slimkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, size_t i) {
  if constexpr (BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
  else
    return static_cast<const float*>(p)[i];
}

// ---------------------------------------------------------------------------
// Prologue, one workgroup per (b, kv head).  Rotates the G query heads of the
// group at the query position (rotate-half pairs (i, i + d/2), angle
// pos * theta^(-2i/d), angles and the rotation in double precision) and
// pre-scales them by scale * log2(e) so later scores are in log2 units.
// With a latent segment it also projects them into the head's latent key
// space: q_lat = U_K^T q_rot.  (Page "Can SlimKV compress KV cache jointly
// across tokens and features", section "Latent-space attention removes the
// rebuild step": queries keep RoPE and are projected after GQA grouping.)
template <bool BF16>
__global__ __launch_bounds__(kThreads) void prologue_kernel(PrologueArgs a) {
  __shared__ float qs[kMaxGroup][kHeadDim];
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int b = unit / a.num_kv_heads;
  const int h = unit - b * a.num_kv_heads;
  const int G = a.group;
  const double pos = (double)a.q_pos[b];
  constexpr int half = kHeadDim / 2;
  for (int p = tid; p < G * half; p += kThreads) {
    const int g = p / half, i = p - (p / half) * half;
    const size_t base = ((size_t)b * a.num_q_heads + (size_t)h * G + g) * kHeadDim;
    const double x1 = ld<BF16>(a.q, base + i), x2 = ld<BF16>(a.q, base + i + half);
    const double inv_freq = pow(a.rope_theta, -(double)(2 * i) / (double)kHeadDim);
    double sn, cs;
    sincos(pos * inv_freq, &sn, &cs);
    const float r1 = (float)((x1 * cs - x2 * sn) * a.score_scale);
    const float r2 = (float)((x2 * cs + x1 * sn) * a.score_scale);
    a.q_rot[base + i] = r1;
    a.q_rot[base + i + half] = r2;
    qs[g][i] = r1;
    qs[g][i + half] = r2;
  }
  if (!a.q_lat) return;
  __syncthreads();
  const int rk = a.rank_k;
  const size_t u0 = (size_t)h * kHeadDim * rk;
  for (int p = tid; p < G * rk; p += kThreads) {
    const int g = p / rk, k = p - (p / rk) * rk;
    float acc = 0.0f;
    for (int i = 0; i < kHeadDim; ++i) acc = fmaf(qs[g][i], ld<BF16>(a.U_K, u0 + (size_t)i * rk + k), acc);
    a.q_lat[((size_t)b * a.num_q_heads + (size_t)h * G + g) * rk + k] = acc;
  }
}

// ---------------------------------------------------------------------------
// Combine, one workgroup per (b, kv head).  Merges the per-chunk partials of
// all G heads by log-sum-exp (one softmax over every beacon and raw row),
// lifts the merged latent value sum once by U_V and adds the full-width sum:
//   out = U_V (sum_latent w_s acc_s) / L + (sum_full w_s acc_s) / L,
//   w_s = 2^(m_s - M), L = sum_s w_s l_s, lse = ln 2 * (M + log2 L).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  constexpr int kBlock = 256;
  __shared__ float sM[kMaxGroup], sL[kMaxGroup];
  __shared__ float wts[kBlock][kMaxGroup];
  __shared__ float olat[kMaxGroup][kHeadDim];
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int b = unit / a.num_kv_heads;
  const int h = unit - b * a.num_kv_heads;
  const int G = a.group, S = a.splits_total, rv = a.rank_v;
  const float* ml = a.part_ml + (size_t)unit * S * G * 2;
  const float* acc = a.part_acc + (size_t)unit * S * G * kHeadDim;

  if (tid < G) {
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[(s * G + tid) * 2]);
    float L = 0.0f;
    for (int s = 0; s < S; ++s) L += exp2f(ml[(s * G + tid) * 2] - M) * ml[(s * G + tid) * 2 + 1];
    sM[tid] = M;
    sL[tid] = L;
  }
  __syncthreads();

  constexpr int kPer = kMaxGroup * kHeadDim / kThreads;  // outputs per thread
  float lat[kPer], full[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) lat[j] = full[j] = 0.0f;
  for (int s0 = 0; s0 < S; s0 += kBlock) {
    const int ns = min(kBlock, S - s0);
    for (int q = tid; q < ns * G; q += kThreads) {
      const int si = q / G, g = q - (q / G) * G;
      wts[si][g] = exp2f(ml[((s0 + si) * G + g) * 2] - sM[g]) / sL[g];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = tid + kThreads * j;
      if (p < G * kHeadDim) {
        const int g = p / kHeadDim, col = p - (p / kHeadDim) * kHeadDim;
        for (int si = 0; si < ns; ++si) {
          const int s = s0 + si;
          const float w = wts[si][g];
          if (s < a.latent_splits) {
            if (col < rv) lat[j] = fmaf(w, acc[((size_t)s * G + g) * kHeadDim + col], lat[j]);
          } else {
            full[j] = fmaf(w, acc[((size_t)s * G + g) * kHeadDim + col], full[j]);
          }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int p = tid + kThreads * j;
    if (p < G * kHeadDim) olat[p / kHeadDim][p % kHeadDim] = lat[j];
  }
  __syncthreads();
  const size_t uv0 = (size_t)h * kHeadDim * rv;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int p = tid + kThreads * j;
    if (p < G * kHeadDim) {
      const int g = p / kHeadDim, i = p - (p / kHeadDim) * kHeadDim;
      float o = full[j];
      if (a.latent_splits > 0)
        for (int k = 0; k < rv; ++k) o = fmaf(ld<BF16>(a.U_V, uv0 + (size_t)i * rv + k), olat[g][k], o);
      a.out[((size_t)b * a.num_q_heads + (size_t)h * G + g) * kHeadDim + i] = o;
    }
  }
  if (a.lse && tid < G)
    a.lse[(size_t)b * a.num_q_heads + (size_t)h * G + tid] =
        (float)(0.69314718055994530942 * ((double)sM[tid] + log2((double)sL[tid])));
}

// ---------------------------------------------------------------------------
// Rebuild (reconstruction comparison path only): dst = C U^T per unit, i.e.
// the full-dimension beacon keys or values the latent path never forms,
// rounded to the storage dtype.  bf16: one wave per 16 rows, MFMA
// 16x16x32 over 8 column tiles, staged through LDS for 16-byte stores.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(kThreads) void rebuild_bf16_kernel(RebuildArgs a) {
  constexpr int kPitch = kHeadDim + 8;  // bf16 elements per LDS row
  __shared__ __attribute__((aligned(16))) uint16_t tile[kWaves][16][kPitch];
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
    for (int e = 0; e < 4; ++e) tile[wave][4 * kg + e][nt * 16 + n] = f32_to_bf16(d[e]);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = lane + 64 * j;
    const int row = idx >> 4, seg = idx & 15;
    if (row0 + row < a.num_beacons)
      *reinterpret_cast<u32x4_t*>(D + (size_t)(row0 + row) * kHeadDim + seg * 8) =
          *reinterpret_cast<const u32x4_t*>(&tile[wave][row][seg * 8]);
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

hipError_t launch_prologue(const PrologueArgs& a, int dtype, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.num_kv_heads)), block(kThreads);
  if (dtype == 0)
    hipLaunchKernelGGL(prologue_kernel<false>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(prologue_kernel<true>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.num_kv_heads)), block(kThreads);
  if (dtype == 0)
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, s, a);
  return hipGetLastError();
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

hipError_t launch_sweep_g1(const SweepArgs&, int, int, hipStream_t);
hipError_t launch_sweep_g2(const SweepArgs&, int, int, hipStream_t);
hipError_t launch_sweep_g3(const SweepArgs&, int, int, hipStream_t);
hipError_t launch_sweep_g4(const SweepArgs&, int, int, hipStream_t);
hipError_t launch_sweep_g5(const SweepArgs&, int, int, hipStream_t);
hipError_t launch_sweep_g6(const SweepArgs&, int, int, hipStream_t);
hipError_t launch_sweep_g7(const SweepArgs&, int, int, hipStream_t);
hipError_t launch_sweep_g8(const SweepArgs&, int, int, hipStream_t);

hipError_t launch_sweep(const SweepArgs& a, int dtype, hipStream_t s) {
  int nch = 4;
  if (a.seg[0].kind == kSegLatent) {
    nch = (a.seg[0].rk + 31) / 32;
    const int nv = (a.seg[0].rv + 31) / 32;
    if (nv > nch) nch = nv;
  }
  switch (a.group) {
    case 1: return launch_sweep_g1(a, dtype, nch, s);
    case 2: return launch_sweep_g2(a, dtype, nch, s);
    case 3: return launch_sweep_g3(a, dtype, nch, s);
    case 4: return launch_sweep_g4(a, dtype, nch, s);
    case 5: return launch_sweep_g5(a, dtype, nch, s);
    case 6: return launch_sweep_g6(a, dtype, nch, s);
    case 7: return launch_sweep_g7(a, dtype, nch, s);
    default: return launch_sweep_g8(a, dtype, nch, s);
  }
}

}  // namespace slimkv
