// sweep_impl.h -- the fused decode-attention kernel: query prologue, split-K
// sweep over one unit's rows, and the merge of all of the unit's workgroups
// by whichever finishes last.
//
// What is computed (page "Can SlimKV compress KV cache jointly across tokens
// and features", section "Latent-space attention removes the rebuild step"):
// the G query heads of one KV head are rotated at the query position and,
// for beacon rows, projected into the head's latent key space (q' U_K).
// Scores against the latent beacon keys C_K (no rotation) and against the
// rotated raw keys share one softmax.  Beacon values are summed in latent
// form (A C_V) and lifted by U_V once per workgroup, on the workgroup's
// merged latent sum, so beacon keys and values are never rebuilt at full
// dimension.
//
// Mapping onto CDNA4 (gfx950):
//   * Workgroups of 4 waves; a unit's tiles (16/32/64 rows, every global read
//     a 16-byte non-temporal buffer load) are dealt round-robin over all waves
//     of its workgroups, beacon tiles first, then raw tiles.  One tile per
//     wave is in flight at all times, across the boundary between the two
//     segments too.
//   * Prologue per workgroup: the rotation angle formed and reduced mod 2*pi
//     in double precision, sine and cosine of the reduced angle in fp32; the
//     latent projection U_K^T q' on the matrix cores (U_K staged in LDS), both
//     while the first tile is in flight.
//   * Scores are a [G x K] x [K x 16 rows] contraction per 16-row subtile on
//     the matrix cores (v_mfma_f32_16x16x32_bf16; fp32 data uses
//     v_mfma_f32_16x16x4_f32).  Query heads sit on the M axis, cache rows on
//     N, features on K.  The bf16 path feeds the fp32 query as two bf16
//     terms (hi + lo): ~16 mantissa bits of query against exact bf16 keys.
//   * The MFMA output keeps head 4*(lane/16)+i of row lane%16 in register
//     i, so the running max is a 16-lane DPP reduction and the softmax state
//     lives in that layout.  exp-weights reach the value lanes through LDS;
//     each value lane holds 16 bytes of one value row and G x 8 fp32 sums.
//   * Each wave parks its beacon state in LDS and goes straight on to its raw
//     tiles.  At the end the four waves merge both segments in LDS, the
//     workgroup lifts its latent sum with U_V on the matrix cores (each wave
//     requested its U_V rows in place of a further tile, so they arrive with
//     its last tile), combines it with the raw sum and writes one partial
//     with device-coherent stores.  A device-scope counter per unit elects
//     the unit's last workgroup, which reads the partials back with
//     device-coherent loads, merges them by log-sum-exp, writes out and lse,
//     and resets the counters for the next call.
#pragma once
#include <math.h>

#include <algorithm>

#include "internal.h"

namespace slimkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// x + x of lane ^ 16 (resp. ^ 32), on the VALU: gfx950's permlane swap of x
// with itself returns, in every lane, its own 16-lane row's value and the
// partner row's, whose sum is the butterfly step.
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Eight fp32 values as two bf16 vectors, hi + lo ~= x to ~2^-17 relative:
// hi = x rounded to bf16 by the hardware conversion (nearest even), lo = the
// exact fp32 remainder x - hi, rounded the same way.
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)x[e];
    hi[e] = h;
    lo[e] = (__bf16)(x[e] - (float)h);
  }
}

// Workgroup barrier that orders LDS only.  __syncthreads() is a workgroup
// fence over all memory, so each wave would first wait for every global load,
// store and atomic it has in flight (the next tile, the tile counter's reply);
// data exchanged through LDS needs only its own LDS operations complete.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// The (max, sum) pairs of partials are stored as relaxed agent-scope atomics,
// i.e. with the device-coherent cache policy, so no whole-L2 writeback or
// invalidate is needed to hand them over -- only completion of the stores.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raw storage bits of element i (bf16 zero-extended), converted later by
// bits_to_float: the conversion is what a load's wait attaches to.
template <bool BF16>
__device__ __forceinline__ uint32_t ld_bits(const void* p, size_t i) {
  if constexpr (BF16)
    return static_cast<const uint16_t*>(p)[i];
  else
    return static_cast<const uint32_t*>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ float bits_to_float(uint32_t u) {
  return __uint_as_float(BF16 ? u << 16 : u);
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

// 16-row subtiles per tile for a given chunk count (of K or V, the larger):
// about 8 KB of keys and values per tile, times D (the tile depth).
template <bool BF16, int NCH, int D = 1>
struct TileShape {
  static constexpr int kSub = (BF16 ? (NCH == 1 ? 4 : (NCH == 2 ? 2 : 1)) : 1) * D;
  static constexpr int kRows = 16 * kSub;
};

// LDS of one attention workgroup.  The prologue's staged U_K is dead once
// the latent query is formed; the sweep reuses its space.
struct alignas(16) AttnShared {
  union {
    struct {
      uint16_t uk[kHeadDim * (kHeadDim + 2)];  // bf16 U_K, rows padded by 2 elements
    } pro;
    struct {
      union {
        float p[kWaves][128 * 8];                // exp-weights of the current tile, per wave
        float raw[kWaves][kMaxGroup][kHeadDim];  // each wave's raw-row sums (after the sweeps)
      } t;
      float beacon[kWaves][kMaxGroup][kHeadDim];  // each wave's beacon-row sums
    } s;
  } u;
  // rotated and latent query, pre-scaled (prologue); after the sweeps the
  // workgroup's merged raw and beacon sums
  float qrot[kMaxGroup][kHeadDim];
  float qlat[kMaxGroup][kHeadDim];
  float wml[2][kWaves][kMaxGroup][2];  // each wave's (max, sum) per head, per segment
  float sml[2][kMaxGroup][2];          // the workgroup's (max, sum) per head, per segment
  float pml[kMaxGroup][2];             // the workgroup's partial: (max, sum) per head
  uint32_t tokk[kHeadDim];             // the new token's key, rotated and rounded (storage bits)
  int is_last;
};

// The workgroup's partial sums, [G][d], once the sweeps' per-wave sums are
// merged (they reuse the first wave's beacon-sum space).
__device__ __forceinline__ float* partial_sums(AttnShared& sh) { return &sh.u.s.beacon[0][0][0]; }

// Rotation angle q_pos * theta^(-2i/d) for pair i < 64: the frequency is the
// product of the host's theta^(-2 * 2^k / d) over i's set bits (a few fp64
// roundings), the angle is formed and reduced into [-pi, pi] in fp64 with a
// two-term 2*pi (each fma step exact up to one rounding).  For the query
// only the sine and cosine of the reduced angle are taken in fp32 (~2e-7
// absolute).
__device__ __forceinline__ double rope_angle(const AttnArgs& a, int pos, int i) {
  double f = 1.0;
#pragma unroll
  for (int k = 0; k < 6; ++k) f *= ((i >> k) & 1) ? a.inv_freq_pow2[k] : 1.0;
  const double ang = (double)pos * f;
  constexpr double kTwoPiHi = 6.283185307179586232;     // 2*pi rounded to double
  constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2*pi - kTwoPiHi
  constexpr double kInvTwoPi = 0.15915494309189534561;
  const double kk = rint(ang * kInvTwoPi);
  double r = fma(-kk, kTwoPiHi, ang);
  return fma(-kk, kTwoPiLo, r);
}
__device__ __forceinline__ void rope_sincos(const AttnArgs& a, int pos, int i, float& s, float& c) {
  sincosf((float)rope_angle(a, pos, i), &s, &c);
}

// ---------------------------------------------------------------------------
// Prologue, run by every workgroup for its (b, kv head): the G query heads
// rotated at the query position (rotate-half pairs (i, i + d/2), angles in
// fp64 reduced mod 2*pi, see rope_sincos) and pre-scaled by scale * log2(e) into
// sh.qrot; with latent beacons also sh.qlat = U_K^T qrot on the matrix cores
// (bf16: the query as hi + lo bf16 terms against exact U_K staged in LDS;
// fp32: exact products).  issue() requests every input; the caller then requests
// its first cache tile and calls finish().  Memory returns in request order,
// so the prologue's inputs arrive ahead of the tile and its arithmetic
// overlaps the tile's flight.
template <int G, bool BF16, int NCH, bool ROTATE = true>
struct QueryPrologue {
  static constexpr bool kLat = NCH > 0;           // latent beacons: project the query
  static constexpr bool kStage = BF16 && kLat;    // U_K staged through LDS
  static constexpr int kHalf = kHeadDim / 2;
  static constexpr int kPairs = (G * kHalf + kThreads - 1) / kThreads;  // rotation pairs per thread
  static_assert(kThreads % kHalf == 0, "a thread's pairs share one index");
  static constexpr int kTiles = kLat ? kHeadDim / 16 / kWaves : 0;       // latent column tiles per wave
  // 16-byte words of U_K per thread when staged: r_K <= 32 * NCH
  static constexpr int kWords = kStage ? kHeadDim * 32 * NCH / 8 / kThreads : 1;
  static constexpr int kGather = (kLat && !kStage) ? kTiles : 1;

  uint32_t x1[kPairs], x2[kPairs];    // storage bits of the query pairs
  int pos;
  u32x4_t uk[kWords];                 // staged: U_K words, row-major
  uint32_t ub[kGather][kHeadDim / 4]; // fp32: U_K column (c0 + n) of each tile, rows 4s + kg

  // Every load here is unconditional, from a clamped (in-bounds) address, and
  // nothing converts or stores its result before finish(): a load whose
  // value is used under a branch, or early, would be waited for before the
  // tile's loads are even issued.
  __device__ __forceinline__ void issue(const AttnArgs& a, int b, int h, int wave) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int n = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
      const int p = min(tid + kThreads * j, G * kHalf - 1);
      const int g = p / kHalf, i = p % kHalf;
      const size_t base = ((size_t)b * a.num_q_heads + (size_t)h * G + g) * kHeadDim;
      x1[j] = ld_bits<BF16>(a.q, base + i);
      x2[j] = ld_bits<BF16>(a.q, base + i + kHalf);
    }
    pos = a.q_pos[b];
    if constexpr (kLat) {
      const int rk = a.rank_k;
      const char* U = static_cast<const char*>(a.U_K) + (size_t)h * kHeadDim * rk * Traits<BF16>::kElemBytes;
      if constexpr (kStage) {
        const int words = kHeadDim * rk / 8;  // surplus words load the last one again
#pragma unroll
        for (int w = 0; w < kWords; ++w) uk[w] = load16(U + (size_t)min(tid + kThreads * w, words - 1) * 16);
      } else {
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          // tiles past r_K load a valid tile again; finish() skips them
          const int c0 = min(16 * (wave + kWaves * t), rk - 16);
#pragma unroll
          for (int s = 0; s < kHeadDim / 4; ++s)
            ub[t][s] = ld_bits<BF16>(U, (size_t)(4 * s + kg) * rk + c0 + n);
        }
      }
    }
  }

  __device__ __forceinline__ void finish(const AttnArgs& a, AttnShared& sh, int wave) const {
    const int tid = threadIdx.x, lane = tid & 63;
    const int n = lane & 15, kg = lane >> 4;
    const int rk = kLat ? a.rank_k : 0;
    const int ustride = rk + 2;  // staged row stride in elements: conflict-free column reads
    uint16_t* ul = sh.u.pro.uk;
    if constexpr (kStage) {
      const int words = kHeadDim * rk / 8, wpr = rk / 8;
#pragma unroll
      for (int w = 0; w < kWords; ++w) {
        const int idx = tid + kThreads * w;
        if (idx < words) {
          const int row = idx / wpr, c8 = idx - row * wpr;
          uint32_t* dst = reinterpret_cast<uint32_t*>(ul + row * ustride + c8 * 8);
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = uk[w][e];
        }
      }
    }
    // a thread's pairs all have index i = lane (kThreads is a multiple of
    // kHalf), and the heads share the position: with more than one pair per
    // thread (G > 4) one angle, taken first, serves them all
    float sn1 = 0.0f, cs1 = 1.0f;
    if constexpr (ROTATE && kPairs > 1) rope_sincos(a, pos, lane, sn1, cs1);
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
      const int p = tid + kThreads * j;
      if (p < G * kHalf) {
        const int g = p / kHalf, i = p % kHalf;
        const float v1 = bits_to_float<BF16>(x1[j]), v2 = bits_to_float<BF16>(x2[j]);
        const float sc = (float)a.score_scale;
        if constexpr (ROTATE) {
          float sn = sn1, cs = cs1;
          if constexpr (kPairs == 1) rope_sincos(a, pos, i, sn, cs);
          sh.qrot[g][i] = (v1 * cs - v2 * sn) * sc;
          sh.qrot[g][i + kHalf] = (v2 * cs + v1 * sn) * sc;
        } else {  // an ALiBi backbone rotates nothing
          sh.qrot[g][i] = v1 * sc;
          sh.qrot[g][i + kHalf] = v2 * sc;
        }
      }
    }
    lds_barrier();
    if constexpr (kLat) {
      // qlat[g][k] = sum_i qrot[g][i] U_K[i][k]: D[m=g][n=k] per 16-column tile
      if constexpr (kStage) {
        // bf16 MFMA over K = i in chunks of 32.  A operand: query head n as
        // hi + lo bf16 terms (rows n >= G compute heads that are never
        // stored), split once for all of this wave's tiles; B operand: U_K
        // exact, lane (n, kg) takes rows 32c + 8kg .. +7 of column c0 + n.
        bf16x8_t qh[kHeadDim / 32], ql[kHeadDim / 32];
#pragma unroll
        for (int c = 0; c < kHeadDim / 32; ++c) {
          const int i0 = 32 * c + 8 * kg;
          const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(&sh.qrot[n & (kMaxGroup - 1)][i0]);
          const f32x4_t x1v = *reinterpret_cast<const f32x4_t*>(&sh.qrot[n & (kMaxGroup - 1)][i0 + 4]);
          const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1v[0], x1v[1], x1v[2], x1v[3]};
          split_bf16x8(x, qh[c], ql[c]);
        }
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          const int c0 = 16 * (wave + kWaves * t);
          if (c0 < rk) {
            u32x4_t bw[kHeadDim / 32];  // every LDS read first, then the products
#pragma unroll
            for (int c = 0; c < kHeadDim / 32; ++c)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int i = 32 * c + 8 * kg + 2 * e;
                bw[c][e] = (uint32_t)ul[i * ustride + c0 + n] | ((uint32_t)ul[(i + 1) * ustride + c0 + n] << 16);
              }
            f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int c = 0; c < kHeadDim / 32; ++c) {
              const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, bw[c]);
              d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[c], bv, d, 0, 0, 0);
              d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[c], bv, d, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * kg + e < G) sh.qlat[4 * kg + e][c0 + n] = d[e];
          }
        }
      } else {
        // fp32: exact products, K = i in steps of 4
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          const int c0 = 16 * (wave + kWaves * t);
          if (c0 < rk) {
            f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < kHeadDim / 4; ++s) {
              const float av = n < G ? sh.qrot[n][4 * s + kg] : 0.0f;
              d = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bits_to_float<BF16>(ub[t][s]), d, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * kg + e < G) sh.qlat[4 * kg + e][c0 + n] = d[e];
          }
        }
      }
      lds_barrier();
    }
  }
};

// ---------------------------------------------------------------------------
// Partials cross workgroups and XCDs (whose L2s are not coherent with each
// other).  The 16-byte ones go through buffer instructions with the
// device-coherent cache policy (sc1); the descriptor's size also bounds them.
constexpr int kCoherent = 16;  // cache-policy bits: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, (int)bytes, 0x00020000);
}

// Cache-policy bits of the cache-row loads: non-temporal.  Every row is read
// once per call, so the rows should not push the small, reused data (the
// bases, the query, partials, counters) out of the caches.
constexpr int kStream = 2;

// Buffer descriptor over `bytes` bytes at `base` (raw, no swizzle): loads at
// offsets past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// One segment of one unit (a run of rows: its beacons, or its raw window) as
// this lane sees it.  Keys and values are read through buffer descriptors
// bounded by the unit's rows, so loads past its last row return zeros: rows
// past `rows` get score -inf and weight 0 anyway, and features past r_K (a
// chunk wider than the keys) meet zero query entries.  A value row spans
// rv / EPL lanes, padded to a power of two (lpr) so that row groups can be
// summed by a butterfly.  Tiles are kRows rows.
//
// PAGED: the rows lie in pages of 2^pshift rows (at least 64, so no tile
// spans two pages) drawn from pools [pages, H_kv, 2^pshift, width]; the
// unit's page ids sit in LDS (tab, from index tab0).  Each tile then gets
// its own descriptors, over the live rows of its page only; a page id
// outside [0, npages) gets empty descriptors, so its rows read as zeros.
template <int NCH, bool BF16, bool PAGED = false, int D = 1>
struct SegView {
  using Tr = Traits<BF16>;
  static constexpr int kSub = TileShape<BF16, NCH, D>::kSub;
  static constexpr int kRows = TileShape<BF16, NCH, D>::kRows;
  static constexpr int kKeySlots = kSub * NCH;
  static constexpr int kLoads = Tr::kMaxLoads * D;  // 16-byte loads per lane per tile (keys or values)
  static_assert(!PAGED || kRows <= (1 << kMinPageShift), "a tile must fit in a page");
  __amdgpu_buffer_rsrc_t kr, vr;  // this unit's key and value rows (contiguous)
  int rows, rk, rv, ntiles;
  int kstride, vstride;  // bytes per key / value row
  int klane, vlane;      // this lane's byte offset within a tile (row 0 of the tile)
  int lpr, rpi, vrow, vcc, lanes_row;
  bool vact;
  // paged only
  const char* kp;               // this head's row 0 of page 0 in the key pool
  const char* vp;               // and in the value pool
  size_t kpage, vpage;          // bytes per page (all heads)
  const int32_t* tab;           // the unit's page ids (LDS)
  int tab0, pshift, npages;

  // cap: rows each unit's arrays hold (the unit stride); rows_: live rows
  __device__ __forceinline__ void init(const void* Kp, const void* Vp, int cap, int rows_, int rk_,
                                       int rv_, int unit, int lane) {
    rows = rows_;
    rk = rk_;
    rv = rv_;
    kstride = rk * Tr::kElemBytes;
    vstride = rv * Tr::kElemBytes;
    const size_t urow = (size_t)unit * (size_t)cap;
    kr = make_rsrc(static_cast<const char*>(Kp) + urow * kstride, (uint32_t)rows * kstride);
    vr = make_rsrc(static_cast<const char*>(Vp) + urow * vstride, (uint32_t)rows * vstride);
    lane_init(lane);
  }
  // pools of `pages` pages of 2^shift rows; h of hkv heads; the unit's page
  // ids at tab_[t0 ..]
  __device__ __forceinline__ void init_paged(const void* Kp, const void* Vp, int shift, int pages,
                                             int rows_, int rk_, int rv_, int h, int hkv,
                                             const int32_t* tab_, int t0, int lane) {
    rows = rows_;
    rk = rk_;
    rv = rv_;
    kstride = rk * Tr::kElemBytes;
    vstride = rv * Tr::kElemBytes;
    pshift = shift;
    npages = pages;
    tab = tab_;
    tab0 = t0;
    const size_t hrow = (size_t)h << shift;
    kp = static_cast<const char*>(Kp) + hrow * kstride;
    vp = static_cast<const char*>(Vp) + hrow * vstride;
    kpage = ((size_t)hkv << shift) * kstride;
    vpage = ((size_t)hkv << shift) * vstride;
    lane_init(lane);
  }
  __device__ __forceinline__ void lane_init(int lane) {
    ntiles = (rows + kRows - 1) / kRows;
    lanes_row = rv / Tr::kEpl;
    lpr = 1 << (32 - __builtin_clz(lanes_row - 1));
    rpi = 64 / lpr;
    vrow = lane / lpr;
    vcc = lane & (lpr - 1);
    vact = vcc < lanes_row;
    const int n = lane & 15, kg = lane >> 4;
    // key slot s * NCH + c as an MFMA B operand: lane (n, kg) holds features
    // c*KCH + kg*EPL ... of row 16 s + n
    klane = n * kstride + kg * Tr::kEpl * Tr::kElemBytes;
    // value slot i: row i * rpi + vrow, this lane's 16 bytes (idle lanes clamped)
    vlane = vrow * vstride + min(vcc, lanes_row - 1) * 16;
  }
  // descriptor and this lane's byte offset for the keys / values of the
  // tile at row ta (pid: its page id when paged)
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const char* pool, size_t page,
                                                              int stride, int ta, int pid) const {
    const bool ok = (uint32_t)pid < (uint32_t)npages;
    const int live = min(rows - ((ta >> pshift) << pshift), 1 << pshift);
    return make_rsrc(pool + (size_t)(ok ? pid : 0) * page, ok ? (uint32_t)(live * stride) : 0u);
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t key_rsrc(int ta, int pid) const {
    if constexpr (PAGED) return page_rsrc(kp, kpage, kstride, ta, pid);
    else return kr;
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t val_rsrc(int ta, int pid) const {
    if constexpr (PAGED) return page_rsrc(vp, vpage, vstride, ta, pid);
    else return vr;
  }
  __device__ __forceinline__ int key_base(int ta) const {
    return klane + (PAGED ? (ta & ((1 << pshift) - 1)) : ta) * kstride;
  }
  __device__ __forceinline__ int val_base(int ta) const {
    return vlane + (PAGED ? (ta & ((1 << pshift) - 1)) : ta) * vstride;
  }
  // uniform byte offsets of key / value slot i within a tile
  __device__ __forceinline__ int key_off(int i) const {
    return (i / NCH) * 16 * kstride + (i % NCH) * Tr::kChunkK * Tr::kElemBytes;
  }
  __device__ __forceinline__ int val_off(int i) const { return i * rpi * vstride; }
};

// Where a wave's tile slots read when it has no further tile: with bf16
// latent beacons, this wave's U_V rows for the lift -- key slot c
// holds row 16 wave + n, value slot c row 16 wave + 64 + n, features
// 32c + 8kg .. +7 (past r_V they read on into the next row, or zeros past
// the end, and meet zero latent entries) -- so the lift's inputs arrive
// while the wave's last tile is processed; otherwise a 16-byte window on q
// at offsets past its end, so the loads return zeros and go unused.
struct TailRows {
  __amdgpu_buffer_rsrc_t r;
  int klane, vlane;
  __device__ __forceinline__ int key_off(int c) const { return c * 64; }
  __device__ __forceinline__ int val_off(int c) const { return c * 64; }
};

// Page id of the tile a wave requests next (row ta of `a` if use_a, else
// row tb of `b` if use_b), one LDS read; 0 for contiguous views and for the
// tail.
template <int NA, int NB, bool BF16, bool PG, int D>
__device__ __forceinline__ int tile_page(const SegView<NA, BF16, PG, D>& a, int ta, bool use_a,
                                         const SegView<NB, BF16, PG, D>& b, int tb, bool use_b) {
  if constexpr (!PG) {
    return 0;
  } else {
    const int i = use_a ? a.tab0 + (ta >> a.pshift) : (use_b ? b.tab0 + (tb >> b.pshift) : 0);
    return __builtin_amdgcn_readfirstlane(a.tab[i]);
  }
}

// Request one tile's keys (or values) into the wave's tile registers: tile
// starting at row ta of `a` if use_a, else row tb of `b` if use_b (only with
// CROSS), else the tail's rows.  The choice is wave-uniform, so it selects a
// descriptor and a base offset; every slot is one unconditional load, and the
// registers need no copies afterwards (separate loads per source under a
// branch would be merged by copies that wait for the loads).  pid: the
// chosen tile's page id (see tile_page) when the views are paged.
template <bool CROSS, int NA, int NB, bool BF16, bool PG, int D>
__device__ __forceinline__ void load_tile_keys(const SegView<NA, BF16, PG, D>& a, int ta, bool use_a,
                                               const SegView<NB, BF16, PG, D>& b, int tb, bool use_b,
                                               const TailRows& tail, int pid, u32x4_t* kbuf) {
  constexpr int KA = SegView<NA, BF16, PG, D>::kKeySlots, KB = SegView<NB, BF16, PG, D>::kKeySlots;
  constexpr int K = SegView<NA, BF16, PG, D>::kLoads;
  static_assert(KA <= K && KB <= K, "tile too large");
  const bool ub = CROSS && use_b;
  const __amdgpu_buffer_rsrc_t r = use_a ? a.key_rsrc(ta, pid) : (ub ? b.key_rsrc(tb, pid) : tail.r);
  const int base = use_a ? a.key_base(ta) : (ub ? b.key_base(tb) : tail.klane);
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int off = use_a ? (i < KA ? a.key_off(i) : 0)
                          : (ub ? (i < KB ? b.key_off(i) : 0) : tail.key_off(i));
    kbuf[i] = __builtin_amdgcn_raw_buffer_load_b128(r, base + off, 0, kStream);
  }
}
template <bool CROSS, int NA, int NB, bool BF16, bool PG, int D>
__device__ __forceinline__ void load_tile_values(const SegView<NA, BF16, PG, D>& a, int ta, bool use_a,
                                                 const SegView<NB, BF16, PG, D>& b, int tb, bool use_b,
                                                 const TailRows& tail, int pid, u32x4_t* vbuf) {
  const bool ub = CROSS && use_b;
  const __amdgpu_buffer_rsrc_t r = use_a ? a.val_rsrc(ta, pid) : (ub ? b.val_rsrc(tb, pid) : tail.r);
  const int base = use_a ? a.val_base(ta) : (ub ? b.val_base(tb) : tail.vlane);
#pragma unroll
  for (int i = 0; i < SegView<NA, BF16, PG, D>::kLoads; ++i) {
    const int off = use_a ? a.val_off(i) : (ub ? b.val_off(i) : tail.val_off(i));
    vbuf[i] = __builtin_amdgcn_raw_buffer_load_b128(r, base + off, 0, kStream);
  }
}

// One wave's running softmax state over the rows it has swept: max and sum
// per head in the MFMA output layout (head 4*kg + i in element i), value sums
// for this lane's columns.
template <int G, bool BF16>
struct WaveState {
  float m[4], l[4];
  float acc[G][Traits<BF16>::kEpl];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[i] = -INFINITY;
      l[i] = 0.0f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < Traits<BF16>::kEpl; ++e) acc[g][e] = 0.0f;
  }
};

// ---------------------------------------------------------------------------
// Where a wave's next tile comes from.  A unit's tiles have positions
// 0 .. total-1 (beacon tiles, then raw tiles); wave w of the unit starts at
// position w.  By default (`fixed`) the positions are dealt round-robin:
// wave w gets w, w + base, w + 2 base, ... -- the same tiles in the same
// order on every call, so results repeat bit for bit.  Otherwise every later
// position is handed out by the unit's counter (offset by the unit's wave
// count), so waves that run faster take more tiles; a position is then
// requested one tile ahead, and the counter's reply comes back while a tile
// is in flight.  Either way positions only grow, so a wave meets its beacon
// tiles before its raw tiles.
struct TileFeed {
  uint32_t* grab;    // the unit's counter (zero between calls)
  int base;          // positions below base are the waves' first tiles
  bool fixed;        // wave-uniform
  uint32_t pending;  // lane 0: the counter's reply to the last request

  // An increment with wrap-around at 2^32 - 1, i.e. a plain +1.  (A fetch-add
  // here would be rewritten into a wave-wide atomic whose per-lane results
  // are formed right away, waiting for every load in flight.)
  __device__ __forceinline__ void request(int lane) {
    if (!fixed && lane == 0)
      pending = __builtin_amdgcn_atomic_inc32(grab, 0xffffffffu, __ATOMIC_RELAXED, "agent");
  }
  // the position after j
  __device__ __forceinline__ int take(int j) const {
    return fixed ? j + base : base + (int)__builtin_amdgcn_readfirstlane(pending);
  }
};

// One wave's tiles of one segment, whose tile 0 has position pbase.  On
// entry the loads of the tile at position j are in kbuf/vbuf and a request
// to `feed` is outstanding.  Software pipeline: the next tile's keys are
// requested as soon as the scores have consumed this tile's keys, its
// values as soon as the value sums have consumed this tile's values.  When
// the next position lies past this segment but before pend, it is a tile of
// the next segment (`nx`, tile 0 at position nxbase) and is requested the
// same way, so the stream of loads does not stop between segments (CROSS;
// past pend the slots take the tail's addresses instead).  Positions from
// pend on are not this sweep's to process.  On exit j is the first position
// past this segment (or pend) the wave drew.
//
// ALIBI: each score also gets slope2[i] * (row * astep - adist0) for head
// 4kg + i (slope2 = the head's slope times log2 e; row * astep - adist0 =
// k_pos - q_pos for this segment's row, an affine function of the row).
// The bias grows towards the query, so the positions of a segment map to
// its tiles in reverse (position p -> tile ntiles - 1 - p): each wave takes
// its nearest tiles first, and its running max stops growing after its
// first tile of the segment instead of growing (and rescaling every sum)
// on every tile.
template <int G, int NCH, bool BF16, bool CROSS, int NCH2, bool PG, bool ALIBI = false, int D = 1>
__device__ __forceinline__ void sweep(const SegView<NCH, BF16, PG, D>& sv, int pbase,
                                      const SegView<NCH2, BF16, PG, D>& nx, int nxbase, int pend, int& j,
                                      TileFeed& feed, const TailRows& tail, const float* qsrc, int rq,
                                      u32x4_t* kbuf, u32x4_t* vbuf, float* pw,
                                      WaveState<G, BF16>& st, const float* slope2 = nullptr,
                                      int adist0 = 0, int astep = 0) {
  using Tr = Traits<BF16>;
  constexpr int EPL = Tr::kEpl;
  constexpr int KCH = Tr::kChunkK;
  constexpr int SUB = SegView<NCH, BF16, PG, D>::kSub;
  constexpr int TR = SegView<NCH, BF16, PG, D>::kRows;
  constexpr int VMAX = SegView<NCH, BF16, PG, D>::kLoads;
  constexpr int GP = G <= 4 ? 4 : 8;  // padded heads per LDS row
  constexpr int NGRP = (G + 3) / 4;   // 16-lane groups holding real heads
  static_assert(SUB * NCH <= VMAX, "tile too large");
  static_assert(TR * GP <= 128 * 8, "exp-weights of a tile exceed their LDS space");
  constexpr int TR2 = SegView<NCH2, BF16, PG, D>::kRows;
  const int pstop = min(pbase + sv.ntiles, pend);
  if (j >= pstop) return;  // wave-uniform

  const int lane = threadIdx.x & 63;
  const int n = lane & 15;   // MFMA column (cache row) within a subtile
  const int kg = lane >> 4;  // MFMA k-group / output row group

  // A operand: head m = lane % 16, features of k-group kg (qsrc row stride d)
  bf16x8_t qhi[BF16 ? NCH : 1], qlo[BF16 ? NCH : 1];
  float qf[BF16 ? 1 : NCH][4];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int k0 = c * KCH + kg * (KCH / 4);
    const bool ok = n < G && k0 < rq;
    const int mc = min(n, G - 1), kc = min(k0, rq - KCH / 4);
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
  const int nchk = (sv.rk + KCH - 1) / KCH;  // chunks that carry key features
  const int r1 = sv.rows;

  while (j < pstop) {
    const int t0 = (ALIBI ? sv.ntiles - 1 - (j - pbase) : j - pbase) * TR;

    // -- scores on the matrix cores, log2 units (the query is pre-scaled)
    f32x4_t sc[SUB];
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (c < nchk) {
          if constexpr (BF16) {
            const bf16x8_t kv = __builtin_bit_cast(bf16x8_t, kbuf[s * NCH + c]);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi[c], kv, d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo[c], kv, d, 0, 0, 0);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              d = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[c][e], __uint_as_float(kbuf[s * NCH + c][e]),
                                                       d, 0, 0, 0);
          }
        }
      }
      if constexpr (ALIBI) {
        const float x = (float)((t0 + 16 * s + n) * astep - adist0);
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = fmaf(slope2[i], x, d[i]);
      }
      if (t0 + 16 * s + n >= r1) d = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      sc[s] = d;
    }
    const int jn = feed.take(j);  // wave-uniform
    const bool more = jn < pstop;
    const bool cross = CROSS && !more && jn < pend;
    const int ta = (ALIBI ? sv.ntiles - 1 - (jn - pbase) : jn - pbase) * TR;
    const int tb = (ALIBI ? nx.ntiles - 1 - (jn - nxbase) : jn - nxbase) * TR2;
    const int pid = tile_page(sv, ta, more, nx, tb, cross);
    load_tile_keys<CROSS>(sv, ta, more, nx, tb, cross, tail, pid,
                          kbuf);
    feed.request(lane);

    // -- online softmax: tile max per head, rescale only when it grows
    float mnew[4];
    bool grew = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = sc[0][i];
#pragma unroll
      for (int s = 1; s < SUB; ++s) mx = fmaxf(mx, sc[s][i]);
      mx = row16_max(mx);
      mnew[i] = fmaxf(st.m[i], mx);
      grew |= mnew[i] > st.m[i];
    }
    if (__builtin_amdgcn_ballot_w64(grew) != 0) {
      float alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        alpha[i] = __builtin_amdgcn_exp2f(st.m[i] - mnew[i]);
        st.l[i] *= alpha[i];
        st.m[i] = mnew[i];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float ag =
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[g & 3]), 16 * (g >> 2)));
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.acc[g][e] *= ag;
      }
    }
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sc[s][i] - st.m[i]);
        st.l[i] += p;
        sc[s][i] = p;
      }
      if (kg < NGRP) *reinterpret_cast<f32x4_t*>(&pw[(16 * s + n) * GP + 4 * kg]) = sc[s];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // -- value sums: acc[g][:] += p[row][g] * V[row][cols of this lane]
    const int vi_count = (TR + sv.rpi - 1) / sv.rpi;
#pragma unroll
    for (int i = 0; i < VMAX; ++i) {
      if (i < vi_count) {
        const int rt = i * sv.rpi + sv.vrow;
        const bool ok = sv.vact && rt < TR && t0 + rt < r1;
        const int rr = ok ? rt : 0;
        float pv[GP];
#pragma unroll
        for (int jj = 0; jj < GP; jj += 4) {
          const f32x4_t p4 = *reinterpret_cast<const f32x4_t*>(&pw[rr * GP + jj]);
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[jj + e] = ok ? p4[e] : 0.0f;
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
          for (int e = 0; e < EPL; ++e) st.acc[g][e] = fmaf(pv[g], v[e], st.acc[g][e]);
      }
    }
    load_tile_values<CROSS>(sv, ta, more, nx, tb, cross, tail, pid,
                            vbuf);
    // the next tile overwrites pw: every lane has read it by now
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    j = jn;
  }
}

// Sum a wave's state over its row groups: the value sums of lanes with equal
// column (vcc) by a butterfly -- DPP rotations inside 16-lane rows, permlane
// swaps across rows -- and the softmax sums over the 16 lanes of each head row.
template <int G, bool BF16>
__device__ __forceinline__ void wave_reduce(WaveState<G, BF16>& st, int lpr) {
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < Traits<BF16>::kEpl; ++e) {
      float x = st.acc[g][e];
      if (lpr <= 8) x += dpp_f<0x128>(x);
      if (lpr <= 4) x += dpp_f<0x124>(x);
      if (lpr <= 2) x += dpp_f<0x122>(x);
      if (lpr <= 16) x = xor16_sum(x);
      x = xor32_sum(x);
      st.acc[g][e] = x;
    }
#pragma unroll
  for (int i = 0; i < 4; ++i) st.l[i] = row16_sum(st.l[i]);
}

// Park a reduced wave state in LDS: (max, sum) per head and the G x rv sums.
template <int G, int NCH, bool BF16, bool PG, int D>
__device__ __forceinline__ void wave_park(const WaveState<G, BF16>& st, const SegView<NCH, BF16, PG, D>& sv,
                                          float (*wacc)[kHeadDim], float (*wml)[2]) {
  const int lane = threadIdx.x & 63, n = lane & 15, kg = lane >> 4;
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * kg + i;
      if (g < G) {
        wml[g][0] = st.m[i];
        wml[g][1] = st.l[i];
      }
    }
  }
  if (sv.vrow == 0 && sv.vact) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < Traits<BF16>::kEpl; ++e)
        wacc[g][sv.vcc * Traits<BF16>::kEpl + e] = st.acc[g][e];
  }
}

// ---------------------------------------------------------------------------
// The workgroup's partial.  The four waves' parked states are merged per
// segment in LDS (beacon sums into qlat, raw sums into qrot, each scaled to
// its segment's max); the latent beacon sum is lifted once with U_V on the
// matrix cores (bf16: the latent sum as hi + lo bf16 terms; fp32: exact
// products); beacon and raw are combined by their maxima; the result --
// (max, sum) and G x d sums per head -- is left in LDS (sh.pml and
// partial_sums(sh)), for the unit's merge or for publishing.
template <int G, bool BF16, bool BLAT>
__device__ __forceinline__ void wg_partial(const AttnArgs& a, AttnShared& sh, int h, int wave, int rvb,
                                           const u32x4_t (&uw)[2][4]) {
  float* acc_out = partial_sums(sh);
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = lane & 15, kg = lane >> 4;
  // (1) each segment's sums over the waves, rescaled to the segment's max
  // (columns past `width` are written as zeros, so the lift can read whole
  // 32-column chunks)
  auto merge_waves = [&](const float (*wacc)[kMaxGroup][kHeadDim], const float (*wml)[kMaxGroup][2],
                         int width, float (*dst)[kHeadDim]) {
    if (tid < G * kHeadDim / 4) {  // one 16-byte word of one head each
      const int g = tid / (kHeadDim / 4), col = 4 * (tid % (kHeadDim / 4));
      float M = wml[0][g][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wml[w][g][0]);
      f32x4_t sum = {0.0f, 0.0f, 0.0f, 0.0f};
      if (M != -INFINITY && col < width) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          sum += __builtin_amdgcn_exp2f(wml[w][g][0] - M) * *reinterpret_cast<const f32x4_t*>(&wacc[w][g][col]);
      }
      *reinterpret_cast<f32x4_t*>(&dst[g][col]) = sum;
    }
  };
  merge_waves(sh.u.s.beacon, sh.wml[0], rvb, sh.qlat);
  merge_waves(sh.u.s.t.raw, sh.wml[1], kHeadDim, sh.qrot);
  if (tid < 2 * G) {
    const int sg = tid / G, g = tid - sg * G;
    float M = sh.wml[sg][0][g][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh.wml[sg][w][g][0]);
    float L = 0.0f;
    if (M != -INFINITY)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) L += __builtin_amdgcn_exp2f(sh.wml[sg][w][g][0] - M) * sh.wml[sg][w][g][1];
    sh.sml[sg][g][0] = M;
    sh.sml[sg][g][1] = L;
  }
  lds_barrier();

  // weights of the two segments for head g within the combined partial
  auto weights = [&](int g, float& wb, float& wr) {
    const float mb = sh.sml[0][g][0], mr = sh.sml[1][g][0];
    const float M = fmaxf(mb, mr);
    wb = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mb - M);
    wr = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mr - M);
  };
  if constexpr (BLAT) {
    // out^T[i][g] = sum_k U_V[i][k] olat[g][k]: D[m=i][n=g] over this wave's
    // two 16-row tiles of i.  B operand: latent sums of head n, features
    // 32c + 8kg .. +7 (columns n >= G compute heads that are never stored;
    // latent columns past r_V hold zeros).
    const int rv = a.rank_v;
    const int gl = n & (kMaxGroup - 1);
    f32x4_t d[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    if constexpr (BF16) {
      // the latent sums as hi + lo bf16 terms, read and split once for both tiles
      bf16x8_t hi[4], lo[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(&sh.qlat[gl][32 * c + 8 * kg]);
        const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(&sh.qlat[gl][32 * c + 8 * kg + 4]);
        const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        split_bf16x8(x, hi[c], lo[c]);
      }
      const int nc = (rv + 31) / 32;  // wave-uniform
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < nc) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16x8_t uv = __builtin_bit_cast(bf16x8_t, uw[t][c]);
            d[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uv, hi[c], d[t], 0, 0, 0);
            d[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uv, lo[c], d[t], 0, 0, 0);
          }
        }
      }
    } else {
      const char* U = static_cast<const char*>(a.U_V) + (size_t)h * kHeadDim * rv * 4;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int i0 = 16 * (wave + kWaves * t);
        for (int s4 = 0; s4 < rv / 4; ++s4) {
          const int kk = 4 * s4 + kg;
          const float uvv = ld_elem<false>(U, (size_t)(i0 + n) * rv + kk);
          d[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(uvv, sh.qlat[gl][kk], d[t], 0, 0, 0);
        }
      }
    }
    // lane (n = g, kg) holds rows 16 (wave + 4t) + 4kg + e
    float wb, wr;
    weights(gl, wb, wr);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r0 = 16 * (wave + kWaves * t) + 4 * kg;
      const f32x4_t raw = *reinterpret_cast<const f32x4_t*>(&sh.qrot[gl][r0]);
      if (n < G) {
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = wb * d[t][e] + wr * raw[e];
        *reinterpret_cast<f32x4_t*>(&acc_out[n * kHeadDim + r0]) = v;
      }
    }
  } else {
    // full-width (or absent) beacon rows: no lift
    if (tid < G * kHeadDim / 4) {
      const int g = tid / (kHeadDim / 4), col = 4 * (tid % (kHeadDim / 4));
      float wb, wr;
      weights(g, wb, wr);
      const f32x4_t v = wb * *reinterpret_cast<const f32x4_t*>(&sh.qlat[g][col]) +
                        wr * *reinterpret_cast<const f32x4_t*>(&sh.qrot[g][col]);
      *reinterpret_cast<f32x4_t*>(&acc_out[g * kHeadDim + col]) = v;
    }
  }
  if (tid < G) {
    float wb, wr;
    weights(tid, wb, wr);
    sh.pml[tid][0] = fmaxf(sh.sml[0][tid][0], sh.sml[1][tid][0]);
    sh.pml[tid][1] = wb * sh.sml[0][tid][1] + wr * sh.sml[1][tid][1];
  }
}

// Publish the workgroup's partial (from LDS) into partial slot `slot` with
// device-coherent stores, then -- once every store has completed -- raise
// the slot's flag, which the unit's merging workgroup waits for.
template <int G>
__device__ __forceinline__ void publish_partial(const AttnArgs& a, AttnShared& sh, size_t slot) {
  const int tid = threadIdx.x;
  const float* acc = partial_sums(sh);
  if (tid < G * kHeadDim / 4) {
    const int g = tid / (kHeadDim / 4), c4 = tid % (kHeadDim / 4);
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&acc[g * kHeadDim + 4 * c4]);
    const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(a.part_acc + slot * G * kHeadDim, G * kHeadDim * 4);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rs, (g * kHeadDim + 4 * c4) * 4,
                                           0, kCoherent);
  }
  if (tid < G) {
    store_coherent(&a.part_ml[(slot * G + tid) * 2], sh.pml[tid][0]);
    store_coherent(&a.part_ml[(slot * G + tid) * 2 + 1], sh.pml[tid][1]);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every thread's stores have completed
  if (tid == 0) __hip_atomic_store(&a.flags[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Run by the unit's merging workgroup: wait until the flags of the unit's
// other n - 1 partial slots (slot0 + i, i != own) are raised, i.e. their
// partials are complete in memory.  Their workgroups have all counted
// themselves done before this one, so each is past its sweep and about to
// publish; the wait ends within a few microseconds.  It is bounded anyway
// (kSpinLimit polls): false if it ran out.  Wave 0 polls; the caller
// synchronises the workgroup after it.  No other workgroup touches these
// flags again in this call, so the merger lowers them right after.
constexpr int kSpinLimit = 1 << 20;
__device__ __forceinline__ bool wait_flags(const AttnArgs& a, size_t slot0, int n, int own) {
  const int lane = threadIdx.x & 63;
  for (int it = 0; it < kSpinLimit; ++it) {
    uint32_t f = 1u;
    if (lane < n && lane != own)
      f = __hip_atomic_load(&a.flags[slot0 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_ballot_w64(f == 0u) == 0) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// ---------------------------------------------------------------------------
// Merge of the unit's k partials (run by the unit's merging workgroup, after
// wait_flags): slots slot0 .. slot0 + k - 1, its own (slot0 + own) still in
// LDS, in slot order whichever workgroup merges:
//   M = max_s m_s, L = sum_s 2^(m_s - M) l_s, out = sum_s 2^(m_s - M) acc_s / L,
//   lse = ln 2 * (M + log2 L).
// Thread (g, c4) owns 16-byte column c4 of head g and folds the partials in
// one at a time; a batch of 8 partials' loads is in flight at once.  The
// other slots' flags are lowered once their partials are read.
template <int G>
__device__ __forceinline__ void merge_unit(const AttnArgs& a, const AttnShared& sh, int slot0, int k,
                                           int own, int b, int h) {
  const int tid = threadIdx.x;
  if (tid >= G * kHeadDim / 4) return;
  const int g = tid / (kHeadDim / 4), c4 = tid % (kHeadDim / 4);
  constexpr int kB = 8;
  const __amdgpu_buffer_rsrc_t rml =
      coherent_rsrc(a.part_ml + (size_t)slot0 * G * 2, (uint32_t)(k * G * 2 * 4));
  const __amdgpu_buffer_rsrc_t racc =
      coherent_rsrc(a.part_acc + (size_t)slot0 * G * kHeadDim, (uint32_t)(k * G * kHeadDim * 4));
  const f32x4_t own_acc = *reinterpret_cast<const f32x4_t*>(&const_cast<AttnShared&>(sh).u.s.beacon[0][0][0]
                                                              + g * kHeadDim + 4 * c4);
  const float own_m = sh.pml[g][0], own_l = sh.pml[g][1];
  float M = -INFINITY, L = 0.0f;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < k; s0 += kB) {
    // unconditional loads from clamped slots; surplus ones (and the own
    // slot's, whose values come from LDS) are not folded in
    uint32_t mlw[kB][2];
    u32x4_t v[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int s = min(s0 + u, k - 1);
      const int base = (s * G + g) * 8;
      mlw[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rml, base, 0, kCoherent);
      mlw[u][1] = __builtin_amdgcn_raw_buffer_load_b32(rml, base + 4, 0, kCoherent);
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(racc, ((s * G + g) * kHeadDim + 4 * c4) * 4, 0, kCoherent);
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (s0 + u < k) {
        const bool mine = s0 + u == own;
        if (mine) v[u] = __builtin_bit_cast(u32x4_t, own_acc);
        const float m = mine ? own_m : __uint_as_float(mlw[u][0]);
        const float l = mine ? own_l : __uint_as_float(mlw[u][1]);
        const float mn = fmaxf(M, m);
        if (mn != -INFINITY) {  // a partial with no rows (m = -inf, l = 0, sums 0) adds nothing
          const float a1 = __builtin_amdgcn_exp2f(M - mn), a2 = __builtin_amdgcn_exp2f(m - mn);
          L = L * a1 + l * a2;
          acc = acc * a1 + __builtin_bit_cast(f32x4_t, v[u]) * a2;
          M = mn;
        }
      }
    }
  }
  const float inv = 1.0f / L;
  float* out = a.out + (((size_t)b * a.num_q_heads + (size_t)h * G + g) * kHeadDim + 4 * c4);
  *reinterpret_cast<f32x4_t*>(out) = acc * inv;
  if (a.lse && c4 == 0)
    a.lse[(size_t)b * a.num_q_heads + (size_t)h * G + g] =
        (float)(0.69314718055994530942 * ((double)M + log2((double)L)));
}

// A value of the storage dtype, rounded once from double to nearest (ties
// to even), as storage bits: bf16 keeps 8 significant bits.
template <bool BF16>
__device__ __forceinline__ uint32_t storage_bits_from_f64(double x) {
  if constexpr (BF16) {
    if (x == 0.0 || !isfinite(x)) return __float_as_uint((float)x) >> 16;
    int e;
    const double m = frexp(x, &e);
    const double r = ldexp(rint(ldexp(m, 8)), e - 8);  // exact in fp32
    return __float_as_uint((float)r) >> 16;
  } else {
    return __float_as_uint((float)x);
  }
}

// The decode step's new token as a one-row partial, made by the unit's first
// workgroup in its prologue, while its first tile is in flight: thread
// (g, c4) owns 16-byte column c4 of head g.  The token's key is rotated at
// q_pos in fp64 and rounded once to the storage dtype -- the row the cache
// keeps: rotate() has thread p < 64 turn pair (p, p + 64), one angle each,
// into sh.tokk, which every head then reads -- and scored against the
// rotated, pre-scaled query in LDS (summed over the head's 32 threads);
// the partial (score, 1, value) goes to the
// unit's token slot (a.tok_slot0 + u) with device-coherent stores, for the
// merge.  The token's row is stored when the raw window has room (wlive <
// its capacity): no workgroup reads that row in this call.  PG: through the
// raw pages' ids at ptab[rtab0 ..] (no store if the id is out of range).
// ALIBI: an ALiBi backbone rotates nothing, so the key is scored and stored
// as given; it sits at the query's own position, so its bias is zero.
template <int G, bool BF16, bool ALIBI = false>
struct TokenPartial {
  static constexpr int kHalf = kHeadDim / 2;
  static constexpr int kThreadsUsed = G * kHeadDim / 4 > kHalf ? G * kHeadDim / 4 : kHalf;
  uint32_t kp1, kp2, v[4];  // storage bits: key pair (p, p + 64) with p = tid % 64; values
  // Run by threads tid < kThreadsUsed of the unit's first workgroup.
  __device__ __forceinline__ void issue(const AttnArgs& a, int u) {
    const int tid = threadIdx.x;
    const int c4 = tid % (kHeadDim / 4), p = tid % kHalf;
    const size_t kb = (size_t)u * kHeadDim;
    kp1 = ld_bits<BF16>(a.k_new, kb + p);
    kp2 = ld_bits<BF16>(a.k_new, kb + p + kHalf);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = ld_bits<BF16>(a.v_new, kb + 4 * c4 + e);
  }
  // Run by every thread of the unit's first workgroup; the caller's LDS
  // barrier follows before finish().
  __device__ __forceinline__ void rotate(const AttnArgs& a, AttnShared& sh, int pos) const {
    const int tid = threadIdx.x;
    if (tid < kHalf) {
      uint32_t b1 = kp1, b2 = kp2;
      if constexpr (!ALIBI) {
        double s64, c64;
        sincos(rope_angle(a, pos, tid), &s64, &c64);  // the reduced angle: no large-argument path
        const double k1 = (double)bits_to_float<BF16>(kp1), k2 = (double)bits_to_float<BF16>(kp2);
        b1 = storage_bits_from_f64<BF16>(k1 * c64 - k2 * s64);
        b2 = storage_bits_from_f64<BF16>(k2 * c64 + k1 * s64);
      }
      sh.tokk[tid] = b1;
      sh.tokk[tid + kHalf] = b2;
    }
  }
  template <bool PG>
  __device__ __forceinline__ void finish(const AttnArgs& a, const AttnShared& sh, int u, int b, int h,
                                         int wlive, const int32_t* ptab, int rtab0) const {
    const int tid = threadIdx.x;
    const int g = tid / (kHeadDim / 4), c4 = tid % (kHeadDim / 4);
    uint32_t kbits[4];
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * c4 + e;
      kbits[e] = sh.tokk[i];
      dot += sh.qrot[g][i] * bits_to_float<BF16>(kbits[e]);
    }
    dot = xor16_sum(row16_sum(dot));  // the 32 threads of head g; log2 units (pre-scaled query)
    const size_t slot = (size_t)a.tok_slot0 + u;
    if (c4 == 0) {
      store_coherent(&a.part_ml[(slot * G + g) * 2], dot);
      store_coherent(&a.part_ml[(slot * G + g) * 2 + 1], 1.0f);
    }
    f32x4_t vf;
#pragma unroll
    for (int e = 0; e < 4; ++e) vf[e] = bits_to_float<BF16>(v[e]);
    const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(a.part_acc + slot * G * kHeadDim, G * kHeadDim * 4);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, vf), rs, (g * kHeadDim + 4 * c4) * 4,
                                           0, kCoherent);
    size_t row = ((size_t)u * a.seg[1].rows + wlive) * kHeadDim + 4 * c4;
    bool store = g == 0 && wlive < a.seg[1].rows;
    if constexpr (PG) {
      const int sh_ = a.page_shift;
      const int pid = store ? ptab[rtab0 + (wlive >> sh_)] : -1;
      store = store && (uint32_t)pid < (uint32_t)a.num_pages[1];
      row = (((((size_t)pid * a.num_kv_heads + h) << sh_) + (wlive & ((1 << sh_) - 1))) * kHeadDim) +
            4 * c4;
    }
    if (store) {
      if constexpr (BF16) {
        uint32_t* kd = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.k_store) + row);
        uint32_t* vd = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.v_store) + row);
        kd[0] = kbits[0] | (kbits[1] << 16);
        kd[1] = kbits[2] | (kbits[3] << 16);
        vd[0] = v[0] | (v[1] << 16);
        vd[1] = v[2] | (v[3] << 16);
      } else {
        float* kd = static_cast<float*>(a.k_store) + row;
        float* vd = static_cast<float*>(a.v_store) + row;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kd[e] = __uint_as_float(kbits[e]);
          vd[e] = __uint_as_float(v[e]);
        }
      }
    }
  }
};

// Merge for ragged calls (run by the unit's last workgroup): fold the unit's
// nslots partials (slots slot0 ..) as merge_unit does, then the decode
// step's new token's one-row partial (see TokenPartial; its loads are
// requested with the first partials', so the merge waits for memory
// once); write out and lse.  Thread (g, c4) owns 16-byte column c4 of head
// g.  With no rows at all the unit gets out 0 and lse -inf.
template <int G, bool BF16>
__device__ __forceinline__ void ragged_finish(const AttnArgs& a, const AttnShared& sh, int u, int b,
                                              int h, int slot0, int nslots, int own) {
  const int tid = threadIdx.x;
  if (tid >= G * kHeadDim / 4) return;
  const int g = tid / (kHeadDim / 4), c4 = tid % (kHeadDim / 4);
  const f32x4_t own_acc = *reinterpret_cast<const f32x4_t*>(&const_cast<AttnShared&>(sh).u.s.beacon[0][0][0]
                                                              + g * kHeadDim + 4 * c4);
  const float own_m = sh.pml[g][0], own_l = sh.pml[g][1];
  constexpr int kB = 8;
  float M = -INFINITY, L = 0.0f;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const bool tok = a.k_new != nullptr;
  uint32_t tml = 0;
  u32x4_t tacc = {0u, 0u, 0u, 0u};
  if (tok) {
    const size_t ts = (size_t)a.tok_slot0 + u;
    const __amdgpu_buffer_rsrc_t tm = coherent_rsrc(a.part_ml + ts * G * 2, G * 2 * 4);
    const __amdgpu_buffer_rsrc_t ta = coherent_rsrc(a.part_acc + ts * G * kHeadDim, G * kHeadDim * 4);
    tml = __builtin_amdgcn_raw_buffer_load_b32(tm, g * 8, 0, kCoherent);
    tacc = __builtin_amdgcn_raw_buffer_load_b128(ta, (g * kHeadDim + 4 * c4) * 4, 0, kCoherent);
  }
  if (nslots > 0) {
    const __amdgpu_buffer_rsrc_t rml =
        coherent_rsrc(a.part_ml + (size_t)slot0 * G * 2, (uint32_t)(nslots * G * 2 * 4));
    const __amdgpu_buffer_rsrc_t racc =
        coherent_rsrc(a.part_acc + (size_t)slot0 * G * kHeadDim, (uint32_t)(nslots * G * kHeadDim * 4));
    for (int s0 = 0; s0 < nslots; s0 += kB) {
      uint32_t mlw[kB][2];
      u32x4_t v[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const int s = min(s0 + k, nslots - 1);
        const int base = (s * G + g) * 8;
        mlw[k][0] = __builtin_amdgcn_raw_buffer_load_b32(rml, base, 0, kCoherent);
        mlw[k][1] = __builtin_amdgcn_raw_buffer_load_b32(rml, base + 4, 0, kCoherent);
        v[k] = __builtin_amdgcn_raw_buffer_load_b128(racc, ((s * G + g) * kHeadDim + 4 * c4) * 4, 0,
                                                    kCoherent);
      }
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        if (s0 + k < nslots) {
          const bool mine = s0 + k == own;
          if (mine) v[k] = __builtin_bit_cast(u32x4_t, own_acc);
          const float m = mine ? own_m : __uint_as_float(mlw[k][0]);
          const float l = mine ? own_l : __uint_as_float(mlw[k][1]);
          const float mn = fmaxf(M, m);
          if (mn != -INFINITY) {
            const float a1 = __builtin_amdgcn_exp2f(M - mn), a2 = __builtin_amdgcn_exp2f(m - mn);
            L = L * a1 + l * a2;
            acc = acc * a1 + __builtin_bit_cast(f32x4_t, v[k]) * a2;
            M = mn;
          }
        }
      }
    }
  }
  if (tok) {  // the token's partial: (score, 1, value)
    const float s2 = __uint_as_float(tml);
    const float mn = fmaxf(M, s2);
    const float a1 = __builtin_amdgcn_exp2f(M - mn), a2 = __builtin_amdgcn_exp2f(s2 - mn);
    L = L * a1 + a2;
    acc = acc * a1 + __builtin_bit_cast(f32x4_t, tacc) * a2;
    M = mn;
  }
  const size_t hq = (size_t)b * a.num_q_heads + (size_t)h * G + g;
  float* out = a.out + hq * kHeadDim + 4 * c4;
  if (L > 0.0f) {
    *reinterpret_cast<f32x4_t*>(out) = acc * (1.0f / L);
    if (a.lse && c4 == 0) a.lse[hq] = (float)(0.69314718055994530942 * ((double)M + log2((double)L)));
  } else {
    *reinterpret_cast<f32x4_t*>(out) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (a.lse && c4 == 0) a.lse[hq] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// The work of one workgroup: workgroup c of the k that share unit (b, h)'s
// rows.  Workgroup c hosts the unit's waves 4c .. 4c+3.  The unit's tiles --
// beacon tiles, then raw tiles, all about the same size in bytes -- are
// handed out in order (see TileFeed), so the waves of a unit advance through
// one sliding window of rows; each wave keeps one tile in flight, across the
// segment boundary too.  The workgroup writes one partial (slot slot0 + c);
// the workgroup that finishes last merges the unit.  nbr, wr: the unit's
// live beacon and raw rows (the arrays hold a.seg[*].rows per unit).
// RAGGED: the unit's first workgroup also makes the decode step's new
// token's partial (TokenPartial), which the merge (ragged_finish) folds in.
// PG (ragged only): the rows are paged; ptab (LDS) holds the unit's beacon
// page ids, then its raw page ids.
// NCH > 0: latent beacons swept in NCH MFMA chunks; NCH == 0: beacon rows
// are full width (rebuilt beacons) or absent.
template <int G, int NCH, bool BF16, bool RAGGED, bool PG = false, bool ALIBI = false, int D = 1>
__device__ __forceinline__ void attend_unit(const AttnArgs& a, AttnShared& sh, int unit, int b, int h,
                                            int c, int k, int nbr, int wr, int slot0,
                                            const int32_t* ptab = nullptr) {
  constexpr bool BLAT = NCH > 0;
  constexpr int kFullNch = BF16 ? 4 : 8;
  constexpr int BN = BLAT ? NCH : kFullNch;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int n = lane & 15, kg = lane >> 4;
  const int nwaves = kWaves * k;
  // this wave's number within the unit (the order in which tiles are
  // dealt); a ragged unit's first workgroup, which also makes the new
  // token's partial, is dealt last, so that it is the one that gets a tile
  // fewer when the unit's tiles do not divide evenly
  const int wu = kWaves * (RAGGED ? (c + k - 1) % k : c) + wave;

  SegView<BN, BF16, PG, D> bv;        // beacon rows
  SegView<kFullNch, BF16, PG, D> rw;  // raw rows
  const int brk = BLAT ? a.seg[0].rk : kHeadDim, brv = BLAT ? a.seg[0].rv : kHeadDim;
  int nbp = 0;  // the unit's beacon pages (paged)
  if constexpr (PG) {
    nbp = (nbr + (1 << a.page_shift) - 1) >> a.page_shift;
    bv.init_paged(a.seg[0].K, a.seg[0].V, a.page_shift, a.num_pages[0], nbr, brk, brv, h,
                  a.num_kv_heads, ptab, 0, lane);
    rw.init_paged(a.seg[1].K, a.seg[1].V, a.page_shift, a.num_pages[1], wr, kHeadDim, kHeadDim, h,
                  a.num_kv_heads, ptab, nbp, lane);
  } else {
    bv.init(a.seg[0].K, a.seg[0].V, a.seg[0].rows, nbr, brk, brv, unit, lane);
    rw.init(a.seg[1].K, a.seg[1].V, a.seg[1].rows, wr, kHeadDim, kHeadDim, unit, lane);
  }
  // tile positions: beacon tiles 0 .. nbt-1, then raw tiles; this wave's
  // first is wu, later ones round-robin or from the unit's counter
  const int nbt = bv.ntiles, total = nbt + rw.ntiles;
  TileFeed feed;
  feed.grab = a.counters + (size_t)unit * kCounterStride + 1;
  feed.base = nwaves;
  feed.fixed = a.deterministic != 0;
  feed.pending = 0;
  feed.request(lane);
  // after its last tile a wave loads its U_V rows for the lift (bf16 latent
  // beacons); otherwise the tail loads fall outside a 16-byte window on q
  // and return zeros
  TailRows tail;
  if constexpr (BF16 && BLAT) {
    tail.r = make_rsrc(static_cast<const char*>(a.U_V) + (size_t)h * kHeadDim * a.rank_v * 2,
                       (uint32_t)(kHeadDim * a.rank_v * 2));
    tail.klane = ((16 * wave + n) * a.rank_v + 8 * kg) * 2;
    tail.vlane = tail.klane + 64 * a.rank_v * 2;
  } else {
    tail.r = make_rsrc(a.q, 16);
    tail.klane = tail.vlane = 64;
  }

  // the prologue's inputs, then the wave's first tile: the prologue's
  // arithmetic runs while the tile is in flight
  QueryPrologue<G, BF16, NCH, !ALIBI> pro;
  pro.issue(a, b, h, wave);
  // ragged calls: the unit's first workgroup makes the new token's partial
  TokenPartial<G, BF16, ALIBI> tokp;
  const bool tokwg = RAGGED && c == 0 && a.k_new != nullptr;  // workgroup-uniform
  const bool tok = tokwg && tid < G * kHeadDim / 4;
  if (tokwg && tid < TokenPartial<G, BF16, ALIBI>::kThreadsUsed) tokp.issue(a, unit);
  u32x4_t kbuf[Traits<BF16>::kMaxLoads * D], vbuf[Traits<BF16>::kMaxLoads * D];
  int j = wu;
  {
    // (ALiBi: each segment's tiles in reverse, as in sweep)
    const int tb = (ALIBI ? nbt - 1 - j : j) * SegView<BN, BF16, PG, D>::kRows;
    const int tr = (ALIBI ? rw.ntiles - 1 - (j - nbt) : j - nbt) * SegView<kFullNch, BF16, PG, D>::kRows;
    const bool ub = j < nbt, ur = j >= nbt && j < total;
    const int pid = tile_page(bv, tb, ub, rw, tr, ur);
    load_tile_keys<true>(bv, tb, ub, rw, tr, ur, tail, pid, kbuf);
    load_tile_values<true>(bv, tb, ub, rw, tr, ur, tail, pid, vbuf);
  }
  pro.finish(a, sh, wave);
  if constexpr (RAGGED) {
    if (tokwg) {
      tokp.rotate(a, sh, pro.pos);  // the query's position
      lds_barrier();
      if (tok) tokp.template finish<PG>(a, sh, unit, b, h, wr, ptab, nbp);
    }
  }

  float* pw = sh.u.s.t.p[wave];
  // ALiBi: this lane's heads' slopes in log2 units, and each segment's
  // k_pos - q_pos as row * step - dist0
  float slope2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int bdist0 = 0, rdist0 = 0;
  if constexpr (ALIBI) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      slope2[i] = a.alibi_slopes[h * G + min(4 * kg + i, G - 1)] * 1.4426950408889634f;
    bdist0 = a.q_pos[b] - a.beacon_first;
    // raw row t sits at q_pos - wr + t when the call brings the decode
    // step's new token (which follows the raw rows, at q_pos), at
    // q_pos - wr + 1 + t when the query's own token is the last raw row
    rdist0 = (RAGGED && a.k_new) ? wr : wr - 1;
  }
  WaveState<G, BF16> st;
  st.reset();
  sweep<G, BN, BF16, true, kFullNch, PG, ALIBI, D>(bv, 0, rw, nbt, total, j, feed, tail,
                                          BLAT ? &sh.qlat[0][0] : &sh.qrot[0][0], bv.rk, kbuf, vbuf,
                                          pw, st, slope2, bdist0, a.beacon_stride);
  wave_reduce<G, BF16>(st, bv.lpr);
  wave_park<G, BN, BF16, PG, D>(st, bv, sh.u.s.beacon[wave], sh.wml[0][wave]);
  st.reset();
  sweep<G, kFullNch, BF16, false, kFullNch, PG, ALIBI, D>(rw, nbt, rw, total, total, j, feed, tail,
                                                       &sh.qrot[0][0], kHeadDim, kbuf, vbuf, pw, st,
                                                       slope2, rdist0, 1);
  // From here on the wave only finishes the unit: raise its issue priority
  // over the waves on its SIMD that are still streaming tiles, so the tail
  // (on the critical path of the whole call) is not starved by them.
  __builtin_amdgcn_s_setprio(2);
  // bf16 latent beacons: the tile registers now hold the lift's U_V rows
  // 16 wave + n (t = 0) and 64 + 16 wave + n (t = 1), features 32c + 8kg ..
  // +7 (past r_V they read on into the next row, or zeros past the end, and
  // meet zero latent entries)
  u32x4_t uw[2][4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    uw[0][cc] = kbuf[cc];
    uw[1][cc] = vbuf[cc];
  }
  wave_reduce<G, BF16>(st, rw.lpr);
  lds_barrier();  // every wave is done with its exp-weights (which alias the raw sums)
                    // and with the query (whose space takes the merged sums)
  // ---- Every wave of the workgroup has swept its last tile: count the
  // workgroup done now, so that the reply comes back while the partial is
  // formed.  The workgroup that brings the count to k merges the unit; the
  // others publish their partials and raise their slots' flags, which the
  // merger waits for (they counted themselves done first, so they are all
  // past their sweeps).  The merger keeps its own partial in LDS.
  uint32_t done = 0;
  if (tid == 0)
    done = __hip_atomic_fetch_add(&a.counters[(size_t)unit * kCounterStride], 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  wave_park<G, kFullNch, BF16, PG, D>(st, rw, sh.u.s.t.raw[wave], sh.wml[1][wave]);
  lds_barrier();
  wg_partial<G, BF16, BLAT>(a, sh, h, wave, bv.rv, uw);
  if (tid == 0) sh.is_last = done == (uint32_t)(k - 1);
  lds_barrier();
  if (!sh.is_last) {
    publish_partial<G>(a, sh, (size_t)slot0 + c);
    return;
  }
  bool ok = true;
  if (wave == 0) ok = wait_flags(a, slot0, k, c);
  if (tid == 0) sh.is_last = ok ? 1 : 2;
  lds_barrier();
  // ready for the next call: lower the other slots' flags; once this
  // workgroup's own requests to the unit's counters have completed (the
  // other workgroups' completed before they raised their flags), clear the
  // counters
  if (tid < k && tid != c)
    __hip_atomic_store(&a.flags[(size_t)slot0 + tid], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid < 2)
    __hip_atomic_store(&a.counters[(size_t)unit * kCounterStride + tid], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (sh.is_last != 1) {
    // a partial never arrived (its workgroup did not run to its end): the
    // unit's results are undefined and are written as NaN
    if (tid < G * kHeadDim / 4) {
      const int g = tid / (kHeadDim / 4), c4 = tid % (kHeadDim / 4);
      float* out = a.out + (((size_t)b * a.num_q_heads + (size_t)h * G + g) * kHeadDim + 4 * c4);
      *reinterpret_cast<f32x4_t*>(out) = f32x4_t{NAN, NAN, NAN, NAN};
      if (a.lse && c4 == 0) a.lse[(size_t)b * a.num_q_heads + (size_t)h * G + g] = NAN;
    }
    return;
  }
  if constexpr (RAGGED)
    ragged_finish<G, BF16>(a, sh, unit, b, h, slot0, k, c);
  else
    merge_unit<G>(a, sh, slot0, k, c, b, h);
}

// Grid: `chunks` workgroups per (b, kv head) unit, numbered chunk-major
// (block = c * units + (unit - c) mod units).  Workgroups are placed on the
// CUs in block order, the older workgroups on a CU are served first, and
// blocks are dealt to the XCDs in turn, whose speeds differ a little; so a
// unit made of consecutive blocks, or of blocks on one XCD, would run at the
// speed of its slot or its XCD.  This numbering gives every unit workgroups
// of every age on different XCDs, so the units finish together.
template <int G, int NCH, bool BF16, bool ALIBI = false>
__global__ __launch_bounds__(kThreads, (BF16 && G <= 4 && kAttnDepth == 1) ? 3 : 2) void attention_kernel(
    AttnArgs a) {
  constexpr int D = BF16 ? kAttnDepth : 1;
  __shared__ AttnShared sh;
  const int k = a.chunks;
  const int units = a.batch * a.num_kv_heads;
  const int c = blockIdx.x / units;
  // rotated by c, so that a unit's blocks sit on different XCDs
  const int unit = (int)(((int64_t)blockIdx.x - (int64_t)c * units + c) % units);
  const int b = unit / a.num_kv_heads;
  const int h = unit - b * a.num_kv_heads;
  attend_unit<G, NCH, BF16, false, false, ALIBI, D>(a, sh, unit, b, h, c, k, a.seg[0].rows,
                                                    a.seg[1].rows, unit * k);
}

// Workgroup slots the grid fills on the current device: CUs x resident
// workgroups of `kfn` per CU (at most kWgPerCu), cached per (device, kernel).
int device_slots(const void* kfn);

// The kernel for group size G; nch is the MFMA chunk count of a latent
// beacon segment (1..4 for bf16; fp32 uses 8), 0 for full-width or absent
// beacons.
template <int G, bool ALIBI>
const void* attention_kernel_for(int dtype, int nch) {
  if (dtype == 0)
    return nch == 0 ? reinterpret_cast<const void*>(&attention_kernel<G, 0, false, ALIBI>)
                    : reinterpret_cast<const void*>(&attention_kernel<G, 8, false, ALIBI>);
  switch (nch) {
    case 0: return reinterpret_cast<const void*>(&attention_kernel<G, 0, true, ALIBI>);
    case 1: return reinterpret_cast<const void*>(&attention_kernel<G, 1, true, ALIBI>);
    case 2: return reinterpret_cast<const void*>(&attention_kernel<G, 2, true, ALIBI>);
    case 3: return reinterpret_cast<const void*>(&attention_kernel<G, 3, true, ALIBI>);
    default: return reinterpret_cast<const void*>(&attention_kernel<G, 4, true, ALIBI>);
  }
}

// Workgroup slots of the kernel launch_attention_group<G> would run.
template <int G>
int attention_slots_group(int dtype, int nch, bool alibi) {
  return device_slots(alibi ? attention_kernel_for<G, true>(dtype, nch)
                            : attention_kernel_for<G, false>(dtype, nch));
}

// Launch for group size G (nch as for attention_kernel_for).
template <int G>
hipError_t launch_attention_group(AttnArgs a, int dtype, int nch, hipStream_t s, hipEvent_t ev0,
                                  hipEvent_t ev1) {
  const void* kfn;
  if (a.alibi_slopes) {
    kfn = attention_kernel_for<G, true>(dtype, nch);
  } else {
    kfn = attention_kernel_for<G, false>(dtype, nch);
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

#include "ragged_impl.h"
