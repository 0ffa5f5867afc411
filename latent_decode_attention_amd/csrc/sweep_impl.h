// sweep_impl.h -- the split-K sweep over one row chunk of a (b, kv head) unit.
//
// What one workgroup computes (page "Can SlimKV compress KV cache jointly
// across tokens and features", section "Latent-space attention removes the
// rebuild step"): for the G query heads of one KV head and a contiguous run
// of cached rows, the scores against the rows' keys (latent keys C_K scored
// with the latent query U_K^T q', or rotated full-width keys scored with q'),
// and the online-softmax partial (max, sum of exp, exp-weighted value sum)
// over those rows.  For beacon rows the value sum stays in latent space
// (width r_V); it is lifted by U_V only once, after all chunks are merged.
//
// Mapping onto CDNA4:
//   * 4 waves per workgroup, each sweeping a contiguous sub-range of the
//     chunk in tiles of 16/32/64 rows, all with 16-byte global loads.
//   * Scores are a [G x K] x [K x 16 rows] contraction per 16-row subtile,
//     done on the matrix cores with v_mfma_f32_16x16x32_bf16 (fp32 data:
//     v_mfma_f32_16x16x4_f32).  Query heads sit on the M axis (rows >= G
//     are zero), cache rows on N, features on K.  The bf16 path feeds the
//     query as two bf16 terms (hi + lo), so scores carry ~16 mantissa bits
//     of the fp32 query against exact bf16 keys.
//   * The MFMA output keeps head 4*(lane/16)+i of row lane%16 in register
//     i, so the running max is a 16-lane DPP reduction and the softmax
//     state lives in the same layout.
//   * exp-weights go through LDS to the value lanes, which hold 16 bytes of
//     one value row each (rows are read as one contiguous block) and keep
//     G x 8 fp32 partial sums per lane.
//   * At the end the four waves' partials are merged through LDS (per head,
//     rescaled to a common max) and written to the workspace.
#pragma once
#include "internal.h"

namespace slimkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// All-reduce within each 16-lane DPP row (row_ror 8, 4, 2, 1).
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0x128>(x));
  x = fmaxf(x, dpp_f<0x124>(x));
  x = fmaxf(x, dpp_f<0x122>(x));
  x = fmaxf(x, dpp_f<0x121>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0x128>(x);
  x += dpp_f<0x124>(x);
  x += dpp_f<0x122>(x);
  x += dpp_f<0x121>(x);
  return x;
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Storage traits: bytes per element, elements per 16-byte lane load,
// feature elements one MFMA chunk covers (4 k-groups of lanes).
template <bool BF16>
struct Traits;
template <>
struct Traits<true> {
  static constexpr int kElemBytes = 2;
  static constexpr int kEpl = 8;       // elements per 16-byte load
  static constexpr int kChunkK = 32;   // features per MFMA chunk
  static constexpr int kMaxLoads = 4;  // 16-byte loads per lane per tile (K and V each)
};
template <>
struct Traits<false> {
  static constexpr int kElemBytes = 4;
  static constexpr int kEpl = 4;
  static constexpr int kChunkK = 16;
  static constexpr int kMaxLoads = 8;
};

// Subtiles of 16 rows per tile for a given chunk count (K or V, the larger).
template <bool BF16, int NCH>
struct TileShape {
  static constexpr int kSub = BF16 ? (NCH == 1 ? 4 : (NCH == 2 ? 2 : 1)) : 1;
  static constexpr int kRows = 16 * kSub;
};

struct alignas(16) SweepShared {
  // exp-weights of the current tile, per wave: [rows][GP] (GP = 4 or 8)
  float p[kWaves][64 * 8];
  // per-head merge buffer: one fp32 value-chunk per lane per wave
  float red[kWaves][64][8];
  float ml[kWaves][kMaxGroup][2];
};

// Sweep rows [r0, r1) of one unit's segment and write one partial.
// NCH: MFMA feature chunks per row (template so register arrays are static).
template <int G, int NCH, bool BF16>
__device__ __forceinline__ void sweep_segment(const SweepArgs& a, const Segment& sg, int unit,
                                              int slot, int r0, int r1, SweepShared& sh) {
  using Tr = Traits<BF16>;
  constexpr int EPL = Tr::kEpl;
  constexpr int KCH = Tr::kChunkK;
  constexpr int SUB = TileShape<BF16, NCH>::kSub;
  constexpr int TR = TileShape<BF16, NCH>::kRows;
  constexpr int VMAX = Tr::kMaxLoads;
  constexpr int GP = G <= 4 ? 4 : 8;      // padded heads per LDS row
  constexpr int NGRP = (G + 3) / 4;       // 16-lane groups holding real heads
  static_assert(SUB * NCH <= Tr::kMaxLoads || !BF16, "tile too large");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;   // MFMA row/column index within a subtile
  const int kg = lane >> 4;  // MFMA k-group / output row group

  const int rk = sg.rk, rv = sg.rv;
  const int b = unit / a.num_kv_heads;
  const int h = unit - b * a.num_kv_heads;
  const size_t urow = (size_t)unit * (size_t)sg.rows;
  const char* Kb = static_cast<const char*>(sg.K) + urow * rk * Tr::kElemBytes;
  const char* Vb = static_cast<const char*>(sg.V) + urow * rv * Tr::kElemBytes;

  // ---- query operand (A matrix: head m = lane%16, features of k-group kg)
  const int rq = sg.kind == kSegLatent ? rk : kHeadDim;
  const float* qsrc = (sg.kind == kSegLatent ? a.q_lat : a.q_rot) +
                      ((size_t)b * a.num_q_heads + (size_t)h * G) * rq;
  const int nchk = (rk + KCH - 1) / KCH;  // chunks that carry key features
  bf16x8_t qhi[BF16 ? NCH : 1], qlo[BF16 ? NCH : 1];
  float qf[BF16 ? 1 : NCH][4];
  {
    const int m = lane & 15;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int k0 = c * KCH + kg * (KCH / 4);
      float x[8];
#pragma unroll
      for (int e = 0; e < KCH / 4; ++e)
        x[e] = (m < G && k0 < rq) ? qsrc[(size_t)m * rq + k0 + e] : 0.0f;
      if constexpr (BF16) {
        uint32_t hb[8], lb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          hb[e] = f32_to_bf16_rne(x[e]);
          lb[e] = f32_to_bf16_rne(x[e] - __uint_as_float(hb[e] << 16));
        }
        u32x4_t hw, lw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hw[e] = hb[2 * e] | (hb[2 * e + 1] << 16);
          lw[e] = lb[2 * e] | (lb[2 * e + 1] << 16);
        }
        qhi[c] = __builtin_bit_cast(bf16x8_t, hw);
        qlo[c] = __builtin_bit_cast(bf16x8_t, lw);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[c][e] = x[e];
      }
    }
  }

  // ---- value-lane mapping: LPR lanes hold one value row, RPI rows per load
  const int lpr = rv / EPL;
  const int rpi = 64 / lpr;
  const int vrow = lane / lpr;
  const int vcc = lane - vrow * lpr;
  const bool vact = vrow < rpi;
  const int vi_count = (TR + rpi - 1) / rpi;

  float acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
  }
  float* pw = sh.p[wave];

  for (int t0 = r0; t0 < r1; t0 += TR) {
    // -- issue every load of the tile: keys (MFMA B layout) and values
    u32x4_t kbuf[SUB][NCH];
#pragma unroll
    for (int s = 0; s < SUB; ++s)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int row = t0 + 16 * s + n;
        const int k0 = c * KCH + kg * EPL;
        if (row < r1 && k0 < rk)
          kbuf[s][c] = load16(Kb + ((size_t)row * rk + k0) * Tr::kElemBytes);
        else
          kbuf[s][c] = u32x4_t{0u, 0u, 0u, 0u};
      }
    u32x4_t vbuf[VMAX];
#pragma unroll
    for (int i = 0; i < VMAX; ++i) {
      const int rt = i * rpi + vrow;
      const bool ok = i < vi_count && vact && rt < TR && t0 + rt < r1;
      if (ok)
        vbuf[i] = load16(Vb + ((size_t)(t0 + rt) * rv + vcc * EPL) * Tr::kElemBytes);
      else
        vbuf[i] = u32x4_t{0u, 0u, 0u, 0u};
    }

    // -- scores on the matrix cores, log2 units (the query is pre-scaled)
    f32x4_t sc[SUB];
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (c < nchk) {
          if constexpr (BF16) {
            const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, kbuf[s][c]);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi[c], kv, d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo[c], kv, d, 0, 0, 0);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              d = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[c][e], __uint_as_float(kbuf[s][c][e]),
                                                       d, 0, 0, 0);
          }
        }
      }
      if (t0 + 16 * s + n >= r1) d = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      sc[s] = d;
    }

    // -- online softmax: tile max per head, rescale only when it grows
    float mnew[4];
    bool grew = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = sc[0][i];
#pragma unroll
      for (int s = 1; s < SUB; ++s) mx = fmaxf(mx, sc[s][i]);
      mx = row16_max(mx);
      mnew[i] = fmaxf(m_run[i], mx);
      grew |= mnew[i] > m_run[i];
    }
    if (__builtin_amdgcn_ballot_w64(grew) != 0) {
      float alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        alpha[i] = __builtin_amdgcn_exp2f(m_run[i] - mnew[i]);
        l_run[i] *= alpha[i];
        m_run[i] = mnew[i];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float ag =
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[g & 3]), 16 * (g >> 2)));
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= ag;
      }
    }
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sc[s][i] - m_run[i]);
        l_run[i] += p;
        sc[s][i] = p;
      }
      if (kg < NGRP) *reinterpret_cast<f32x4_t*>(&pw[(16 * s + n) * GP + 4 * kg]) = sc[s];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // -- value sums: acc[g][:] += p[row][g] * V[row][cols of this lane]
#pragma unroll
    for (int i = 0; i < VMAX; ++i) {
      if (i < vi_count) {
        const int rt = i * rpi + vrow;
        const bool ok = vact && rt < TR && t0 + rt < r1;
        const int rr = ok ? rt : 0;
        float pv[GP];
#pragma unroll
        for (int j = 0; j < GP; j += 4) {
          const f32x4_t p4 = *reinterpret_cast<const f32x4_t*>(&pw[rr * GP + j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[j + e] = ok ? p4[e] : 0.0f;
        }
        float v[EPL];
        if constexpr (BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(vbuf[i][e] << 16);
            v[2 * e + 1] = __uint_as_float(vbuf[i][e] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(vbuf[i][e]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pv[g], v[e], acc[g][e]);
      }
    }
    // the next tile overwrites pw: make sure every lane has read it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four waves' partials and write this chunk's partial
#pragma unroll
  for (int i = 0; i < 4; ++i) l_run[i] = row16_sum(l_run[i]);
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * kg + i;
      if (g < G) {
        sh.ml[wave][g][0] = m_run[i];
        sh.ml[wave][g][1] = l_run[i];
      }
    }
  }
  __syncthreads();
  float* ml_out = a.part_ml + (size_t)slot * G * 2;
  float* acc_out = a.part_acc + (size_t)slot * G * kHeadDim;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = sh.ml[0][g][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh.ml[w][g][0]);
    const float sw = __builtin_amdgcn_exp2f(sh.ml[wave][g][0] - M);
#pragma unroll
    for (int e = 0; e < EPL; ++e) sh.red[wave][lane][e] = acc[g][e] * sw;
    __syncthreads();
    for (int col = tid; col < rv; col += kThreads) {
      const int cc = col / EPL, e = col - (col / EPL) * EPL;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        for (int r = 0; r < rpi; ++r) sum += sh.red[w][r * lpr + cc][e];
      acc_out[(size_t)g * kHeadDim + col] = sum;
    }
    if (tid == 0) {
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) L += __builtin_amdgcn_exp2f(sh.ml[w][g][0] - M) * sh.ml[w][g][1];
      ml_out[2 * g] = M;
      ml_out[2 * g + 1] = L;
    }
    __syncthreads();
  }
}

// Grid: one workgroup per (unit, chunk); chunk index runs over both segments.
template <int G, int NCH, bool BF16>
__global__ __launch_bounds__(kThreads) void sweep_kernel(SweepArgs a) {
  __shared__ SweepShared sh;
  const int unit = blockIdx.x / a.splits_total;
  const int s = blockIdx.x - unit * a.splits_total;
  const int si = s < a.seg[0].splits ? 0 : 1;
  const Segment sg = si == 0 ? a.seg[0] : a.seg[1];
  const int chunk = si == 0 ? s : s - a.seg[0].splits;
  const int c0 = chunk * sg.chunk_rows;
  const int c1 = min(sg.rows, c0 + sg.chunk_rows);
  // split the chunk over the waves in whole tiles
  const int tr = sg.kind == kSegFull ? TileShape<BF16, BF16 ? 4 : 8>::kRows
                                     : TileShape<BF16, NCH>::kRows;
  const int per_wave = ((c1 - c0 + kWaves - 1) / kWaves + tr - 1) / tr * tr;
  const int wave = threadIdx.x >> 6;
  const int r0 = min(c1, c0 + wave * per_wave);
  const int r1 = min(c1, r0 + per_wave);
  const int slot = unit * a.splits_total + s;
  if (sg.kind == kSegFull)
    sweep_segment<G, BF16 ? 4 : 8, BF16>(a, sg, unit, slot, r0, r1, sh);
  else
    sweep_segment<G, NCH, BF16>(a, sg, unit, slot, r0, r1, sh);
}

// Launch the sweep for group size G; nch is the MFMA chunk count of the
// latent segment (1..4 for bf16; fp32 always uses 8).
template <int G>
hipError_t launch_sweep_group(const SweepArgs& a, int dtype, int nch, hipStream_t s) {
  const dim3 grid((unsigned)(a.batch * a.num_kv_heads * a.splits_total));
  const dim3 block(kThreads);
  if (dtype == 0) {
    hipLaunchKernelGGL((sweep_kernel<G, 8, false>), grid, block, 0, s, a);
  } else {
    switch (nch) {
      case 1: hipLaunchKernelGGL((sweep_kernel<G, 1, true>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((sweep_kernel<G, 2, true>), grid, block, 0, s, a); break;
      case 3: hipLaunchKernelGGL((sweep_kernel<G, 3, true>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((sweep_kernel<G, 4, true>), grid, block, 0, s, a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace slimkv
