// sweep_impl.h -- the fused decode-attention kernel: query prologue, split-K
// sweep over one row chunk of a (b, kv head) unit, and the merge of all of
// the unit's chunks by whichever workgroup finishes last.
//
// What is computed (page "Can SlimKV compress KV cache jointly across tokens
// and features", section "Latent-space attention removes the rebuild step"):
// the G query heads of one KV head are rotated at the query position and,
// for beacon rows, projected into the head's latent key space (q' U_K).
// Scores against the latent beacon keys C_K (no rotation) and against the
// rotated raw keys share one softmax.  Beacon values are summed in latent
// form (A C_V) and lifted once by U_V after every chunk is merged, so beacon
// keys and values are never rebuilt at full dimension.
//
// Mapping onto CDNA4 (gfx950):
//   * One workgroup of 4 waves per (unit, row chunk); each wave sweeps a
//     contiguous sub-range of the chunk in tiles of 16/32/64 rows, every
//     global read a 16-byte load.
//   * Prologue per workgroup: rotation in double precision (angles reduced
//     mod 2*pi before sincos), the
//     latent projection U_K^T q' as an fp32 MFMA (16x16x4) into LDS.  Its
//     loads and the first tile's loads are all issued up front.
//   * Scores are a [G x K] x [K x 16 rows] contraction per 16-row subtile on
//     the matrix cores (v_mfma_f32_16x16x32_bf16; fp32 data uses
//     v_mfma_f32_16x16x4_f32).  Query heads sit on the M axis, cache rows on
//     N, features on K.  The bf16 path feeds the fp32 query as two bf16
//     terms (hi + lo): ~16 mantissa bits of query against exact bf16 keys.
//   * The MFMA output keeps head 4*(lane/16)+i of row lane%16 in register
//     i, so the running max is a 16-lane DPP reduction and the softmax state
//     lives in that layout.  exp-weights reach the value lanes through LDS;
//     each value lane holds 16 bytes of one value row and G x 8 fp32 sums.
//   * The waves' partials merge in LDS into one partial per chunk, written
//     to the workspace with device-coherent stores.  A device-scope counter
//     per unit elects the last chunk's workgroup, which reads the partials
//     back with device-coherent loads, merges them by log-sum-exp, lifts the
//     latent sum with U_V on the matrix cores, writes out and lse, and resets
//     the counter for the next call.
#pragma once
#include <math.h>

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

// Eight fp32 values as two bf16 vectors, hi + lo ~= x to ~2^-17 relative.
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8_t& hi, bf16x8_t& lo) {
  u32x4_t hw, lw;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h0 = f32_to_bf16_rne(x[2 * e]), h1 = f32_to_bf16_rne(x[2 * e + 1]);
    const uint32_t l0 = f32_to_bf16_rne(x[2 * e] - __uint_as_float(h0 << 16));
    const uint32_t l1 = f32_to_bf16_rne(x[2 * e + 1] - __uint_as_float(h1 << 16));
    hw[e] = h0 | (h1 << 16);
    lw[e] = l0 | (l1 << 16);
  }
  hi = __builtin_bit_cast(bf16x8_t, hw);
  lo = __builtin_bit_cast(bf16x8_t, lw);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Partials cross workgroups (and XCDs, whose L2s are not coherent with each
// other).  They are stored and loaded as relaxed agent-scope atomics, i.e.
// with device-coherent cache policy, so no whole-L2 writeback/invalidate is
// needed to hand them over -- only completion of the stores (see below).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool BF16>
__device__ __forceinline__ float ld_elem(const void* p, size_t i) {
  if constexpr (BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
  else
    return static_cast<const float*>(p)[i];
}

// Storage traits: bytes per element, elements per 16-byte lane load,
// features one MFMA chunk covers (4 k-groups of lanes), loads per tile.
template <bool BF16>
struct Traits;
template <>
struct Traits<true> {
  static constexpr int kElemBytes = 2;
  static constexpr int kEpl = 8;
  static constexpr int kChunkK = 32;
  static constexpr int kMaxLoads = 4;
};
template <>
struct Traits<false> {
  static constexpr int kElemBytes = 4;
  static constexpr int kEpl = 4;
  static constexpr int kChunkK = 16;
  static constexpr int kMaxLoads = 8;
};

// 16-row subtiles per tile for a given chunk count (of K or V, the larger).
template <bool BF16, int NCH>
struct TileShape {
  static constexpr int kSub = BF16 ? (NCH == 1 ? 4 : (NCH == 2 ? 2 : 1)) : 1;
  static constexpr int kRows = 16 * kSub;
};

struct alignas(16) AttnShared {
  union {
    float p[kWaves][64 * 8];                 // exp-weights of the current tile, per wave
    float red[kWaves][kMaxGroup][kHeadDim];  // each wave's rescaled value sums
    struct {
      float ml[kMaxMergeSlots][2];  // every chunk's (max, sum); then weights
      float olat[kMaxGroup][kHeadDim];
      float ofull[kMaxGroup][kHeadDim];
    } comb;
  } u;
  float qrot[kMaxGroup][kHeadDim];  // rotated query, pre-scaled (prologue)
  float qlat[kMaxGroup][kHeadDim];  // latent query, pre-scaled (prologue)
  float ml[kWaves][kMaxGroup][2];
  float M[kMaxGroup], L[kMaxGroup];
  int is_last;
};

// Angle reduced into [-pi, pi] with a two-term 2*pi (fma keeps each step
// exact up to one rounding), so sincos never sees a large argument.
__device__ __forceinline__ void rope_sincos(double ang, double& s, double& c) {
  constexpr double kTwoPiHi = 6.283185307179586232;     // 2*pi rounded to double
  constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2*pi - kTwoPiHi
  constexpr double kInvTwoPi = 0.15915494309189534561;
  const double k = rint(ang * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, ang);
  r = fma(-k, kTwoPiLo, r);
  sincos(r, &s, &c);
}

// ---------------------------------------------------------------------------
// Prologue, run by every workgroup for its (b, kv head): the G query heads
// rotated at the query position (rotate-half pairs (i, i + d/2), double
// precision, angles reduced mod 2*pi) and pre-scaled by scale * log2(e) into
// sh.qrot; with a latent beacon segment also sh.qlat = U_K^T qrot (fp32 MFMA
// 16x16x4, exact products).  Every global read is issued up front.
template <int G, bool BF16>
__device__ __forceinline__ void prologue(const AttnArgs& a, int b, int h, AttnShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int rk = a.rank_k;
  const bool latent = rk > 0;
  constexpr int half = kHeadDim / 2;
  constexpr int kPairs = (G * half + kThreads - 1) / kThreads;  // rotation pairs per thread
  constexpr int kTiles = kHeadDim / 16 / kWaves;                // latent column tiles per wave

  // loads are unconditional from clamped (in-bounds) addresses: a load under
  // a divergent branch costs a full wait for the memory round trip
  float x1[kPairs], x2[kPairs];
#pragma unroll
  for (int j = 0; j < kPairs; ++j) {
    const int p = min(tid + kThreads * j, G * half - 1);
    const int g = p / half, i = p % half;
    const size_t base = ((size_t)b * a.num_q_heads + (size_t)h * G + g) * kHeadDim;
    x1[j] = ld_elem<BF16>(a.q, base + i);
    x2[j] = ld_elem<BF16>(a.q, base + i + half);
  }
  const double pos = (double)a.q_pos[b];
  // U_K columns of this wave's first latent tile (a second tile, r_K > 64,
  // is loaded after the first one's products)
  float ub[kHeadDim / 4];
  const char* U = static_cast<const char*>(a.U_K) + (size_t)h * kHeadDim * rk * Traits<BF16>::kElemBytes;
  auto load_ub = [&](int c0) {
#pragma unroll
    for (int s = 0; s < kHeadDim / 4; ++s) ub[s] = ld_elem<BF16>(U, (size_t)(4 * s + kg) * rk + c0 + n);
  };
  if (latent && 16 * wave < rk) load_ub(16 * wave);  // wave-uniform

#pragma unroll
  for (int j = 0; j < kPairs; ++j) {
    const int p = tid + kThreads * j;
    if (p < G * half) {
      const int g = p / half, i = p % half;
      double sn, cs;
      // theta^(-2i/d) = 2^(-(2i/d) log2 theta), in double precision
      const double inv_freq = exp2(-(double)(2 * i) / (double)kHeadDim * a.log2_theta);
      rope_sincos(pos * inv_freq, sn, cs);
      const double v1 = x1[j], v2 = x2[j];
      sh.qrot[g][i] = (float)((v1 * cs - v2 * sn) * a.score_scale);
      sh.qrot[g][i + half] = (float)((v2 * cs + v1 * sn) * a.score_scale);
    }
  }
  __syncthreads();
  if (!latent) return;
  // qlat[g][k] = sum_i qrot[g][i] U_K[i][k]: D[m=g][n=k], K = i in steps of 4
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const int c0 = 16 * (wave + kWaves * t);
    if (c0 < rk) {
      if (t > 0) load_ub(c0);
      f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < kHeadDim / 4; ++s) {
        const float av = n < G ? sh.qrot[n][4 * s + kg] : 0.0f;
        d = __builtin_amdgcn_mfma_f32_16x16x4f32(av, ub[s], d, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * kg + e < G) sh.qlat[4 * kg + e][c0 + n] = d[e];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Merge of all chunks of one unit (run by the unit's last workgroup).
//   M = max_s m_s, L = sum_s 2^(m_s - M) l_s,
//   o_lat = sum_{latent s} 2^(m_s - M) acc_s / L, o_full likewise,
//   out = U_V o_lat + o_full, lse = ln 2 * (M + log2 L).
// U_V rows, every (max, sum) and a first batch of chunk sums are loaded in
// one round trip; more batches only when a unit has many chunks.
template <int G, bool BF16>
__device__ __forceinline__ void merge_unit(const AttnArgs& a, int unit, int b, int h,
                                           AttnShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = 2 * a.chunks, rv = a.rank_v;
  const bool lat_beacons = a.seg[0].kind == kSegLatent;
  const float* ml = a.part_ml + (size_t)unit * S * G * 2;
  const float* acc = a.part_acc + (size_t)unit * S * G * kHeadDim;
  float (*sml)[2] = sh.u.comb.ml;
  constexpr int kPer = (G * kHeadDim + kThreads - 1) / kThreads;  // outputs per thread
  constexpr int kBatch = 64 / kPer;                               // chunks per load batch
  constexpr int kMlPer = kMaxMergeSlots * 2 / kThreads;           // (max, sum) loads per thread
  const int m16 = lane & 15, kg = lane >> 4;
  const char* U = static_cast<const char*>(a.U_V) + (size_t)h * kHeadDim * rv * Traits<BF16>::kElemBytes;

  // -- one round trip: U_V rows of this wave's output tiles, (max, sum) pairs,
  //    and the first batch of chunk sums
  u32x4_t uw[2][4];
  if constexpr (BF16) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 16 * (wave + kWaves * t) + m16, k0 = 32 * c + 8 * kg;
        // features past r_V are multiplied by zero latent entries below
        uw[t][c] = lat_beacons ? load16(U + ((size_t)i * rv + min(k0, rv - 8)) * 2)
                               : u32x4_t{0u, 0u, 0u, 0u};
      }
  }
  // (unconditional loads from clamped indexes; out-of-range values unused)
  float mlv[kMlPer];
#pragma unroll
  for (int j = 0; j < kMlPer; ++j)
    mlv[j] = load_coherent(&ml[min(tid + kThreads * j, S * G * 2 - 1)]);
  float v[kBatch][kPer];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int su = min(s0 + u, S - 1);
        const int p = min(tid + kThreads * j, G * kHeadDim - 1);
        v[u][j] = load_coherent(&acc[(size_t)su * G * kHeadDim + p]);
      }
  };
  load_batch(0);
#pragma unroll
  for (int j = 0; j < kMlPer; ++j) {
    const int q = tid + kThreads * j;
    if (q < S * G * 2) (&sml[0][0])[q] = mlv[j];
  }
  __syncthreads();

  // -- M and L per head: 32 lanes per head; then weights w_s = 2^(m_s - M) / L
  {
    const int g = tid >> 5, l32 = tid & 31;
    float M = -INFINITY;
    if (g < G)
      for (int s = l32; s < S; s += 32) M = fmaxf(M, sml[s * G + g][0]);
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 32));
    float L = 0.0f;
    if (g < G)
      for (int s = l32; s < S; s += 32) L += __builtin_amdgcn_exp2f(sml[s * G + g][0] - M) * sml[s * G + g][1];
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) L += __shfl_xor(L, off, 32);
    if (g < G && l32 == 0) {
      sh.M[g] = M;
      sh.L[g] = L;
    }
  }
  __syncthreads();
  for (int q = tid; q < S * G; q += kThreads)
    sml[q][0] = __builtin_amdgcn_exp2f(sml[q][0] - sh.M[q % G]) / sh.L[q % G];
  __syncthreads();

  // -- weighted sums: thread owns outputs p = tid + 256 j (p = g * d + col)
  float lat[kPer], full[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) lat[j] = full[j] = 0.0f;
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    if (s0 > 0) load_batch(s0);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = s0 + u;
      if (s < S) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int p = tid + kThreads * j;
          if (p < G * kHeadDim) {
            const int g = p / kHeadDim, col = p % kHeadDim;
            const float w = sml[s * G + g][0];
            // empty slots carry weight 0 and stale sums: skip, don't multiply
            const float wv = w != 0.0f ? w * v[u][j] : 0.0f;
            if ((s & 1) == 0 && lat_beacons) {
              if (col < rv) lat[j] += wv;
            } else {
              full[j] += wv;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int p = tid + kThreads * j;
    if (p < G * kHeadDim) {
      sh.u.comb.olat[p / kHeadDim][p % kHeadDim] = lat[j];
      sh.u.comb.ofull[p / kHeadDim][p % kHeadDim] = full[j];
    }
  }
  __syncthreads();

  // -- lift the latent sum once and add the full-width sum
  float* out = a.out + ((size_t)b * a.num_q_heads + (size_t)h * G) * kHeadDim;
  if (lat_beacons) {
    // out^T[i][g] = sum_k U_V[i][k] olat[g][k]: D[m=i][n=g] over 16-row tiles of i
    const int n = lane & 15;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i0 = 16 * (wave + kWaves * t);
      f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (BF16) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (32 * c < rv) {
            const int k0 = 32 * c + 8 * kg;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (k0 < rv && n < G) ? sh.u.comb.olat[n][k0 + e] : 0.0f;
            bf16x8_t hi, lo;
            split_bf16x8(x, hi, lo);
            const bf16x8_t uv = __builtin_bit_cast(bf16x8_t, uw[t][c]);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uv, hi, d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uv, lo, d, 0, 0, 0);
          }
        }
      } else {
        for (int s = 0; s < rv / 4; ++s) {
          const int k = 4 * s + kg;
          const float uvv = ld_elem<false>(U, (size_t)(i0 + m16) * rv + k);
          const float ov = n < G ? sh.u.comb.olat[n][k] : 0.0f;
          d = __builtin_amdgcn_mfma_f32_16x16x4f32(uvv, ov, d, 0, 0, 0);
        }
      }
      // lane (n = g, kg) holds rows i = i0 + 4kg + e
      if (n < G) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = i0 + 4 * kg + e;
          out[(size_t)n * kHeadDim + row] = d[e] + sh.u.comb.ofull[n][row];
        }
      }
    }
  } else {
    for (int p = tid; p < G * kHeadDim; p += kThreads)
      out[(size_t)(p / kHeadDim) * kHeadDim + p % kHeadDim] = sh.u.comb.ofull[p / kHeadDim][p % kHeadDim];
  }
  if (a.lse && tid < G)
    a.lse[(size_t)b * a.num_q_heads + (size_t)h * G + tid] =
        (float)(0.69314718055994530942 * ((double)sh.M[tid] + log2((double)sh.L[tid])));
}

// ---------------------------------------------------------------------------
// This workgroup's share of one unit's segment.  The unit's tiles (beacon
// tiles, then raw tiles; all about the same size in bytes) are dealt
// round-robin to the unit's `nwaves` waves, so every wave gets the same
// number of tiles to within one and all waves of a unit advance through one
// sliding window of rows.  `base` is the dealt index of this segment's first
// tile, `wu` this wave's number.  Writes the workgroup's partial to `slot`
// (max -inf, sum 0 if none of its waves got a tile).
template <int G, int NCH, bool BF16>
__device__ __forceinline__ void attend_segment(const AttnArgs& a, const Segment& sg, int unit,
                                               int slot, int wu, int nwaves, int base,
                                               bool run_prologue, AttnShared& sh) {
  using Tr = Traits<BF16>;
  constexpr int EPL = Tr::kEpl;
  constexpr int KCH = Tr::kChunkK;
  constexpr int SUB = TileShape<BF16, NCH>::kSub;
  constexpr int TR = TileShape<BF16, NCH>::kRows;
  constexpr int VMAX = Tr::kMaxLoads;
  constexpr int GP = G <= 4 ? 4 : 8;  // padded heads per LDS row
  constexpr int NGRP = (G + 3) / 4;   // 16-lane groups holding real heads
  static_assert(!BF16 || SUB * NCH <= Tr::kMaxLoads, "tile too large");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;   // MFMA column (cache row) within a subtile
  const int kg = lane >> 4;  // MFMA k-group / output row group

  float* ml_out = a.part_ml + (size_t)slot * G * 2;
  float* acc_out = a.part_acc + (size_t)slot * G * kHeadDim;
  const int ntiles = (sg.rows + TR - 1) / TR;
  // this wave's first tile in the segment: the first index >= base dealt to wu
  const int first = ((wu - base) % nwaves + nwaves) % nwaves;
  const int b = unit / a.num_kv_heads;
  const int h = unit - b * a.num_kv_heads;
  if (__syncthreads_or(first < ntiles) == 0) {  // no wave of this workgroup has a tile
    if (tid < G) {
      store_coherent(&ml_out[2 * tid], -INFINITY);
      store_coherent(&ml_out[2 * tid + 1], 0.0f);
    }
    if (run_prologue) prologue<G, BF16>(a, b, h, sh);
    return;
  }
  // this wave's tiles: first, first + nwaves, ...; rows past the segment end masked
  const int r1 = sg.rows;
  const int t_first = first * TR, t_step = nwaves * TR;

  const int rk = sg.rk, rv = sg.rv;
  const bool latent = sg.kind == kSegLatent;
  const size_t urow = (size_t)unit * (size_t)sg.rows;
  const char* Kb = static_cast<const char*>(sg.K) + urow * rk * Tr::kElemBytes;
  const char* Vb = static_cast<const char*>(sg.V) + urow * rv * Tr::kElemBytes;

  // value-lane mapping: a value row spans rv/EPL lanes, padded to a power of
  // two (LPR) so the row groups can be summed by a butterfly; RPI rows per load
  const int lanes_row = rv / EPL;
  const int lpr = 1 << (32 - __builtin_clz(lanes_row - 1));
  const int rpi = 64 / lpr;
  const int vrow = lane / lpr;
  const int vcc = lane & (lpr - 1);
  const bool vact = vcc < lanes_row;
  const int vcol = min(vcc, lanes_row - 1) * EPL;  // clamped for idle lanes
  const int vi_count = (TR + rpi - 1) / rpi;
  const int nchk = (rk + KCH - 1) / KCH;  // chunks that carry key features

  u32x4_t kbuf[SUB][NCH];
  u32x4_t vbuf[VMAX];
  // Every load is unconditional, from an address clamped into the segment and
  // the row's width: rows past r1 get score -inf, features past r_K meet
  // zero query entries, and value rows past r1 get weight 0, so the clamped
  // data never contributes (a load under a divergent branch would cost a
  // full memory round trip each).
  auto load_keys = [&](int t0) {
#pragma unroll
    for (int s = 0; s < SUB; ++s)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int row = min(t0 + 16 * s + n, r1 - 1);
        const int k0 = min(c * KCH + kg * EPL, rk - EPL);
        kbuf[s][c] = load16(Kb + ((size_t)row * rk + k0) * Tr::kElemBytes);
      }
  };
  auto load_values = [&](int t0) {
#pragma unroll
    for (int i = 0; i < VMAX; ++i) {
      const int row = min(t0 + i * rpi + vrow, r1 - 1);
      vbuf[i] = load16(Vb + ((size_t)row * rv + vcol) * Tr::kElemBytes);
    }
  };

  // the first tile is in flight while the prologue runs
  if (t_first < r1) {
    load_keys(t_first);
    load_values(t_first);
  }
  if (run_prologue) prologue<G, BF16>(a, b, h, sh);
  const int rq = latent ? rk : kHeadDim;
  const float* qsrc = latent ? &sh.qlat[0][0] : &sh.qrot[0][0];  // row stride kHeadDim
  bf16x8_t qhi[BF16 ? NCH : 1], qlo[BF16 ? NCH : 1];
  float qf[BF16 ? 1 : NCH][4];
  {
    // A matrix: head m = lane%16, features of k-group kg
    const int m = lane & 15;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int k0 = c * KCH + kg * (KCH / 4);
      const bool ok = m < G && k0 < rq;
      const int mc = min(m, G - 1), kc = min(k0, rq - KCH / 4);
      float x[8];
#pragma unroll
      for (int e = 0; e < KCH / 4; ++e) x[e] = ok ? qsrc[mc * kHeadDim + kc + e] : 0.0f;
      if constexpr (BF16) {
        split_bf16x8(x, qhi[c], qlo[c]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[c][e] = x[e];
      }
    }
  }

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
  float* pw = sh.u.p[wave];

  // Software pipeline: the next tile's keys are requested as soon as the
  // scores have consumed this tile's keys, its values as soon as the value
  // sums have consumed this tile's values.
  for (int t0 = t_first; t0 < r1; t0 += t_step) {
    const int tn = t0 + t_step;

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
    if (tn < r1) load_keys(tn);

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
    if (tn < r1) load_values(tn);
    // the next tile overwrites pw: every lane has read it by now
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four waves' partials into this chunk's partial
  // (1) per wave: sum the row groups (lanes with equal vcc) by a butterfly:
  //     DPP rotations inside 16-lane rows, lane swaps across rows
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = acc[g][e];
      if (lpr <= 8) x += dpp_f<0x128>(x);
      if (lpr <= 4) x += dpp_f<0x124>(x);
      if (lpr <= 2) x += dpp_f<0x122>(x);
      if (lpr <= 16) x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[g][e] = x;
    }
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
  // (2) each wave rescales its sums to the workgroup max and parks them in LDS
  if (vrow == 0 && vact) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float M = sh.ml[0][g][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh.ml[w][g][0]);
      const float sw = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sh.ml[wave][g][0] - M);
#pragma unroll
      for (int e = 0; e < EPL; ++e) sh.u.red[wave][g][vcc * EPL + e] = acc[g][e] * sw;
    }
  }
  __syncthreads();
  // (3) sum the four waves, write the piece's partial with coherent stores
  for (int p = tid; p < G * rv; p += kThreads) {
    const int g = p / rv, col = p - (p / rv) * rv;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += sh.u.red[w][g][col];
    store_coherent(&acc_out[(size_t)g * kHeadDim + col], sum);
  }
  if (tid < G) {
    float M = sh.ml[0][tid][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh.ml[w][tid][0]);
    float L = 0.0f;
    if (M != -INFINITY)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) L += __builtin_amdgcn_exp2f(sh.ml[w][tid][0] - M) * sh.ml[w][tid][1];
    store_coherent(&ml_out[2 * tid], M);
    store_coherent(&ml_out[2 * tid + 1], L);
  }

}

// Grid: `chunks` workgroups per (b, kv head) unit.  Workgroup c hosts the
// unit's waves 4c .. 4c+3; the unit's tiles (beacon, then raw) are dealt
// round-robin over its 4*chunks waves.  The beacon rows' partial goes to slot 2c, the
// raw rows' to slot 2c+1; the workgroup that finishes last merges the unit.
template <int G, int NCH, bool BF16>
__global__ __launch_bounds__(kThreads, (BF16 && G <= 4) ? 3 : 2) void attention_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  const int tid = threadIdx.x;
  const int k = a.chunks;
  const int unit = blockIdx.x / k;
  const int c = blockIdx.x - unit * k;
  const int b = unit / a.num_kv_heads;
  const int h = unit - b * a.num_kv_heads;
  const int nwaves = kWaves * k;
  const int wu = kWaves * c + (tid >> 6);
  const size_t slot0 = ((size_t)unit * k + c) * 2;
  constexpr int kFullNch = BF16 ? 4 : 8;

  // beacon rows (latent, or rebuilt at full width)
  Segment sg;
  sg.K = a.seg[0].K;
  sg.V = a.seg[0].V;
  sg.kind = a.seg[0].kind;
  sg.rows = a.seg[0].rows;
  sg.rk = a.seg[0].rk;
  sg.rv = a.seg[0].rv;
  const int btile = sg.kind == kSegLatent ? TileShape<BF16, NCH>::kRows
                                           : TileShape<BF16, kFullNch>::kRows;
  const int beacon_tiles = (sg.rows + btile - 1) / btile;
  if (sg.kind == kSegLatent)
    attend_segment<G, NCH, BF16>(a, sg, unit, (int)slot0, wu, nwaves, 0, true, sh);
  else
    attend_segment<G, kFullNch, BF16>(a, sg, unit, (int)slot0, wu, nwaves, 0, true, sh);
  __syncthreads();  // LDS is reused by the next segment

  // raw rows
  sg.K = a.seg[1].K;
  sg.V = a.seg[1].V;
  sg.kind = kSegFull;
  sg.rows = a.seg[1].rows;
  sg.rk = kHeadDim;
  sg.rv = kHeadDim;
  attend_segment<G, kFullNch, BF16>(a, sg, unit, (int)slot0 + 1, wu, nwaves, beacon_tiles,
                                    false, sh);

  // ---- the last chunk of the unit merges everything.  Every thread waits
  // for its coherent partial stores to complete before the barrier; only
  // then does thread 0 count the chunk as done.  The workgroup that brings
  // the count to k reads all partials with coherent loads.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t done =
        __hip_atomic_fetch_add(&a.counters[unit], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.is_last = done == (uint32_t)(k - 1);
  }
  __syncthreads();
  if (!sh.is_last) return;
  merge_unit<G, BF16>(a, unit, b, h, sh);
  if (tid == 0)  // ready for the next call
    __hip_atomic_store(&a.counters[unit], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroups of `kfn` resident per CU and the CU count of the current
// device, cached per (device, kernel).
int device_slots(const void* kfn);

// Launch for group size G; nch is the MFMA chunk count of the latent
// segment (1..4 for bf16; fp32 always uses 8).
template <int G>
hipError_t launch_attention_group(AttnArgs a, int dtype, int nch, hipStream_t s, hipEvent_t ev0,
                                  hipEvent_t ev1) {
  const void* kfn;
  if (dtype == 0) {
    kfn = reinterpret_cast<const void*>(&attention_kernel<G, 8, false>);
  } else {
    switch (nch) {
      case 1: kfn = reinterpret_cast<const void*>(&attention_kernel<G, 1, true>); break;
      case 2: kfn = reinterpret_cast<const void*>(&attention_kernel<G, 2, true>); break;
      case 3: kfn = reinterpret_cast<const void*>(&attention_kernel<G, 3, true>); break;
      default: kfn = reinterpret_cast<const void*>(&attention_kernel<G, 4, true>); break;
    }
  }
  const int64_t units = (int64_t)a.batch * a.num_kv_heads;
  if (a.chunks <= 0) {
    const int slots = device_slots(kfn);
    if (slots <= 0) return hipErrorInvalidDeviceFunction;
    a.chunks = choose_chunks(units, a.unit_bytes, slots, 64 << 10);
  }
  const dim3 grid((unsigned)(units * a.chunks)), block(kThreads);
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, s);
    if (e != hipSuccess) return e;
  }
  void* args[] = {&a};
  hipError_t err = hipLaunchKernel(kfn, grid, block, args, 0, s);
  if (err == hipSuccess) err = hipGetLastError();
  if (err == hipSuccess && ev1) return hipEventRecord(ev1, s);
  return err;
}

}  // namespace slimkv
