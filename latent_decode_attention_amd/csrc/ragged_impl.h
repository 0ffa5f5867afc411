// ragged_impl.h -- decode attention over a ragged batch, with the decode
// step's new token (included by sweep_impl.h; instantiated per group size in
// sweep_g*.hip).
//
// What is computed is the latent decode attention of page "Can SlimKV
// compress KV cache jointly across tokens and features", section
// "Latent-space attention removes the rebuild step", in the setting of a
// serving decode step: every sequence b has its own number of live beacon
// rows and raw rows in capacity-sized arrays, and the step's new token --
// its key rotated at the query position, since the token attends to itself
// -- joins the raw rows.  When the raw window has room, the token's rotated
// key and its value are also written to the cache row after the live ones.
//
// Mapping onto CDNA4:
//   * Work is balanced over the grid by tiles, not by sequences: the tiles
//     of all (b, kv head) units, unit after unit, form one sequence of
//     positions, and workgroup r takes the r-th equal share of it.  A share
//     may cover the end of one unit and the start of the next; each piece
//     (share x unit) runs the same prologue, sweeps and workgroup partial as
//     the uniform kernel, into its own partial slot (r + unit, unique since
//     pieces advance r or the unit or both).
//   * Each workgroup recomputes the schedule from the lengths at its start:
//     one wave loads them and scans the tile counts into LDS.
//   * Ranks alternate between the CUs' first and second workgroup slots
//     (and the second-slot ranks are shifted by four blocks, so a unit's
//     shares sit on different XCDs): neighbouring shares of a unit then
//     stream at the mixed speed of both slots.
//   * The last piece of a unit to finish merges the unit's partials by
//     log-sum-exp, folds in the new token as a one-row partial (its score
//     computed there), writes out and lse, and stores the token's row.
//     Units without tiles are finished by workgroup (unit mod grid).
#pragma once

namespace slimkv {

// Per-workgroup schedule: sequence b's units start at tile position pre[b]
// (H_kv units of equal tile count each); nb, w are its live row counts.
struct RaggedShared {
  int32_t pre[kMaxRaggedBatch + 1];
  int32_t nb[kMaxRaggedBatch];
  int32_t w[kMaxRaggedBatch];
};

// Run by one wave: live rows clamped to [0, capacity], tiles per unit, and
// their exclusive scan over the sequences (lane L takes a run of
// consecutive sequences; every load is requested before any is used).
template <int TRB, int TRR>
__device__ __forceinline__ void ragged_schedule(const AttnArgs& a, RaggedShared& rs, int lane) {
  constexpr int kPer = kMaxRaggedBatch / 64;
  const int B = a.batch, ncap = a.seg[0].rows, wcap = a.seg[1].rows;
  const int per = (B + 63) / 64;
  const int b0 = lane * per;
  int nbv[kPer], wv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = min(b0 + k, B - 1);
    nbv[k] = a.seq_beacons ? a.seq_beacons[b] : ncap;
    wv[k] = a.seq_raw ? a.seq_raw[b] : wcap;
  }
  int tiles[kPer];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int nbc = min(max(nbv[k], 0), ncap), wc = min(max(wv[k], 0), wcap);
    const bool mine = k < per && b0 + k < B;
    tiles[k] = mine ? (nbc + TRB - 1) / TRB + (wc + TRR - 1) / TRR : 0;
    if (mine) {
      rs.nb[b0 + k] = nbc;
      rs.w[b0 + k] = wc;
    }
    sum += tiles[k];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  int run = incl - sum;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (k < per && b0 + k < B) rs.pre[b0 + k] = run * a.num_kv_heads;
    run += tiles[k];
  }
  if (lane == 63) rs.pre[B] = incl * a.num_kv_heads;
}

// Share (rank) of block blk in a grid of P: blocks of the first half take
// the even ranks, the second half the odd ones, shifted by four blocks.
__device__ __forceinline__ int ragged_rank(int blk, int P) {
  if (P & 1) return blk;
  const int half = P >> 1;
  if (blk < half) return 2 * blk;
  int m = (blk - half - 4) % half;
  if (m < 0) m += half;
  return 2 * m + 1;
}

// The rank whose share holds tile position x (0 <= x < T) when P <= T ranks
// share the tiles: the largest r with floor(r T / P) <= x.
__device__ __forceinline__ int ragged_owner(int64_t x, int64_t T, int P) {
  return (int)(((x + 1) * P - 1) / T);
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

// Finish unit u: fold its nslots partials (slots slot0 ..), then the new
// token as a one-row partial; write out and lse; store the token's row.
// Thread (g, c4) owns 16-byte column c4 of head g.  With no rows at all the
// unit gets out 0 and lse -inf.
template <int G, bool BF16>
__device__ __noinline__ void ragged_finish(const AttnArgs& a, int u, int b, int h, int slot0,
                                              int nslots, int wlive) {
  const int tid = threadIdx.x;
  if (tid >= G * kHeadDim / 4) return;
  const int g = tid / (kHeadDim / 4), c4 = tid % (kHeadDim / 4);
  constexpr int kB = 8;
  float M = -INFINITY, L = 0.0f;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
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
          const float m = __uint_as_float(mlw[k][0]), l = __uint_as_float(mlw[k][1]);
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
  const size_t hq = (size_t)b * a.num_q_heads + (size_t)h * G + g;
  if (a.k_new) {
    // the new token: key rotated at q_pos in fp64 and rounded once to the
    // storage dtype (the row the cache keeps), query rotated as in the
    // prologue; the score is summed over the 32 threads of head g
    const int pos = a.q_pos[b];
    const size_t qb = hq * kHeadDim, kb = (size_t)u * kHeadDim;
    float dot = 0.0f;
    uint32_t kbits[4];
    float vnew[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * c4 + e, pi = i & (kHeadDim / 2 - 1), ip = i ^ (kHeadDim / 2);
      const bool lo = i < kHeadDim / 2;
      float sn, cs;
      rope_sincos(a, pos, pi, sn, cs);
      const float qi = ld_elem<BF16>(a.q, qb + i), qp = ld_elem<BF16>(a.q, qb + ip);
      const float qr = lo ? qi * cs - qp * sn : qi * cs + qp * sn;
      double f = 1.0;
#pragma unroll
      for (int k = 0; k < 6; ++k) f *= ((pi >> k) & 1) ? a.inv_freq_pow2[k] : 1.0;
      double s64, c64;
      sincos((double)pos * f, &s64, &c64);
      const double ki = (double)ld_elem<BF16>(a.k_new, kb + i), kp = (double)ld_elem<BF16>(a.k_new, kb + ip);
      kbits[e] = storage_bits_from_f64<BF16>(lo ? ki * c64 - kp * s64 : ki * c64 + kp * s64);
      dot += qr * bits_to_float<BF16>(kbits[e]);
      vnew[e] = ld_elem<BF16>(a.v_new, kb + i);
    }
    dot = xor16_sum(row16_sum(dot));  // the 32 lanes of head g
    const float s2 = dot * (float)a.score_scale;
    const float mn = fmaxf(M, s2);
    const float a1 = __builtin_amdgcn_exp2f(M - mn), a2 = __builtin_amdgcn_exp2f(s2 - mn);
    L = L * a1 + a2;
    acc = acc * a1 + f32x4_t{vnew[0], vnew[1], vnew[2], vnew[3]} * a2;
    M = mn;
    if (g == 0 && wlive < a.seg[1].rows) {
      const size_t row = ((size_t)u * a.seg[1].rows + wlive) * kHeadDim + 4 * c4;
      if constexpr (BF16) {
        uint32_t* kd = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.k_store) + row);
        uint32_t* vd = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.v_store) + row);
        const uint16_t* vs = static_cast<const uint16_t*>(a.v_new) + kb + 4 * c4;
        kd[0] = kbits[0] | (kbits[1] << 16);
        kd[1] = kbits[2] | (kbits[3] << 16);
        vd[0] = (uint32_t)vs[0] | ((uint32_t)vs[1] << 16);
        vd[1] = (uint32_t)vs[2] | ((uint32_t)vs[3] << 16);
      } else {
        float* kd = static_cast<float*>(a.k_store) + row;
        float* vd = static_cast<float*>(a.v_store) + row;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kd[e] = __uint_as_float(kbits[e]);
          vd[e] = vnew[e];
        }
      }
    }
  }
  float* out = a.out + hq * kHeadDim + 4 * c4;
  if (L > 0.0f) {
    *reinterpret_cast<f32x4_t*>(out) = acc * (1.0f / L);
    if (a.lse && c4 == 0) a.lse[hq] = (float)(0.69314718055994530942 * ((double)M + log2((double)L)));
  } else {
    *reinterpret_cast<f32x4_t*>(out) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (a.lse && c4 == 0) a.lse[hq] = -INFINITY;
  }
}

// One piece: tile positions [lo, hi) of unit u (b, h), swept by the
// workgroup's four waves round-robin, reduced to the workgroup's partial in
// slot r + u; the unit's last piece finishes the unit.
template <int G, int NCH, bool BF16>
__device__ __forceinline__ void ragged_piece(const AttnArgs& a, AttnShared& sh, int b, int h, int u,
                                             int nbr, int wr, int lo, int hi, int r, int64_t T, int P,
                                             int64_t ustart, int tb) {
  constexpr bool BLAT = NCH > 0;
  constexpr int kFullNch = BF16 ? 4 : 8;
  constexpr int BN = BLAT ? NCH : kFullNch;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, kg = lane >> 4;

  SegView<BN, BF16> bv;  // this sequence's live beacon rows
  bv.init(a.seg[0].K, a.seg[0].V, a.seg[0].rows, nbr, BLAT ? a.seg[0].rk : kHeadDim,
          BLAT ? a.seg[0].rv : kHeadDim, u, lane);
  SegView<kFullNch, BF16> rw;  // its live raw rows
  rw.init(a.seg[1].K, a.seg[1].V, a.seg[1].rows, wr, kHeadDim, kHeadDim, u, lane);
  const int nbt = bv.ntiles;
  TileFeed feed;
  feed.grab = nullptr;
  feed.base = kWaves;
  feed.fixed = true;
  feed.pending = 0;
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

  QueryPrologue<G, BF16, NCH> pro;
  pro.issue(a, b, h, wave);
  u32x4_t kbuf[Traits<BF16>::kMaxLoads], vbuf[Traits<BF16>::kMaxLoads];
  int j = lo + wave;
  {
    const int tbr = j * SegView<BN, BF16>::kRows, trr = (j - nbt) * SegView<kFullNch, BF16>::kRows;
    const bool ub = j < min(nbt, hi), ur = j >= nbt && j < hi;
    load_tile_keys<true>(bv, tbr, ub, rw, trr, ur, tail, kbuf);
    load_tile_values<true>(bv, tbr, ub, rw, trr, ur, tail, vbuf);
  }
  pro.finish(a, sh, wave);

  float* pw = sh.u.s.t.p[wave];
  WaveState<G, BF16> st;
  st.reset();
  sweep<G, BN, BF16, true>(bv, 0, rw, nbt, hi, j, feed, tail,
                           BLAT ? &sh.qlat[0][0] : &sh.qrot[0][0], bv.rk, kbuf, vbuf, pw, st);
  wave_reduce<G, BF16>(st, bv.lpr);
  wave_park<G, BN, BF16>(st, bv, sh.u.s.beacon[wave], sh.wml[0][wave]);
  st.reset();
  sweep<G, kFullNch, BF16, false>(rw, nbt, rw, hi, hi, j, feed, tail, &sh.qrot[0][0], kHeadDim, kbuf,
                                  vbuf, pw, st);
  __builtin_amdgcn_s_setprio(2);
  u32x4_t uw[2][4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    uw[0][cc] = kbuf[cc];
    uw[1][cc] = vbuf[cc];
  }
  wave_reduce<G, BF16>(st, rw.lpr);
  lds_barrier();
  wave_park<G, kFullNch, BF16>(st, rw, sh.u.s.t.raw[wave], sh.wml[1][wave]);
  lds_barrier();
  const size_t slot = (size_t)r + u;
  wg_partial<G, BF16, BLAT>(a, sh, h, wave, bv.rv, uw, a.part_ml + slot * G * 2,
                            a.part_acc + slot * G * kHeadDim);

  // count the piece done once its partial is stored; the unit's last piece
  // (pieces are counted per unit, each by the workgroup that ran it)
  // finishes the unit
  const int first = ragged_owner(ustart, T, P), last = ragged_owner(ustart + tb - 1, T, P);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(&a.counters[(size_t)u * kCounterStride], 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.is_last = done == (uint32_t)(last - first);
  }
  lds_barrier();
  if (sh.is_last) {
    if (tid == 0)
      __hip_atomic_store(&a.counters[(size_t)u * kCounterStride], 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    ragged_finish<G, BF16>(a, u, b, h, first + u, last - first + 1, wr);
  }
  __builtin_amdgcn_s_setprio(0);
  lds_barrier();  // every wave has read is_last before the next piece reuses LDS
}

template <int G, int NCH, bool BF16>
__global__ __launch_bounds__(kThreads, kWgPerCu * kWaves / 4) void ragged_kernel(AttnArgs a) {
  constexpr bool BLAT = NCH > 0;
  constexpr int kFullNch = BF16 ? 4 : 8;
  constexpr int BN = BLAT ? NCH : kFullNch;
  constexpr int TRB = SegView<BN, BF16>::kRows, TRR = SegView<kFullNch, BF16>::kRows;
  __shared__ AttnShared sh;
  __shared__ RaggedShared rs;
  const int tid = threadIdx.x, lane = tid & 63;
  const int B = a.batch, Hkv = a.num_kv_heads;
  if ((tid >> 6) == 0) ragged_schedule<TRB, TRR>(a, rs, lane);
  lds_barrier();
  const int P = (int)gridDim.x;
  const int r = ragged_rank((int)blockIdx.x, P);
  const int64_t T = rs.pre[B];
  // shares of the tiles: ranks below Pw = min(P, T) each take a non-empty
  // one (so a unit's pieces are the ranks from its first tile's owner to
  // its last's), the others none
  const int Pw = (int)(T < P ? T : P);
  int64_t pos = r < Pw ? (int64_t)r * T / Pw : 0;
  const int64_t e = r < Pw ? (int64_t)(r + 1) * T / Pw : 0;
  while (pos < e) {  // workgroup-uniform
    // the sequence holding pos: the last b with pre[b] <= pos
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (rs.pre[mid] <= pos) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int nbr = rs.nb[b], wr = rs.w[b];
    const int tb = (nbr + TRB - 1) / TRB + (wr + TRR - 1) / TRR;
    const int h = (int)((pos - rs.pre[b]) / tb);
    const int64_t ustart = rs.pre[b] + (int64_t)h * tb;
    const int64_t uend = e < ustart + tb ? e : ustart + tb;
    ragged_piece<G, NCH, BF16>(a, sh, b, h, b * Hkv + h, nbr, wr, (int)(pos - ustart),
                               (int)(uend - ustart), r, T, Pw, ustart, tb);
    pos = uend;
  }
  // units without tiles (no live rows): only the new token, or nothing
  for (int u = r; u < B * Hkv; u += P) {
    const int b = u / Hkv;
    if (rs.pre[b + 1] == rs.pre[b]) ragged_finish<G, BF16>(a, u, b, u - b * Hkv, 0, 0, rs.w[b]);
  }
}

// Launch for group size G; nch as for launch_attention_group.
template <int G>
const void* ragged_kernel_for(int dtype, int nch) {
  if (dtype == 0)
    return nch == 0 ? reinterpret_cast<const void*>(&ragged_kernel<G, 0, false>)
                    : reinterpret_cast<const void*>(&ragged_kernel<G, 8, false>);
  switch (nch) {
    case 0: return reinterpret_cast<const void*>(&ragged_kernel<G, 0, true>);
    case 1: return reinterpret_cast<const void*>(&ragged_kernel<G, 1, true>);
    case 2: return reinterpret_cast<const void*>(&ragged_kernel<G, 2, true>);
    case 3: return reinterpret_cast<const void*>(&ragged_kernel<G, 3, true>);
    default: return reinterpret_cast<const void*>(&ragged_kernel<G, 4, true>);
  }
}

// grid: a.chunks workgroups in all (> 0: as given; <= 0: the device's slots),
// at most max_wgs
template <int G>
hipError_t launch_ragged_group(AttnArgs a, int dtype, int nch, int64_t max_wgs, hipStream_t s,
                               hipEvent_t ev0, hipEvent_t ev1) {
  const void* kfn = ragged_kernel_for<G>(dtype, nch);
  int64_t wgs = a.chunks;
  if (wgs <= 0) {
    wgs = device_slots(kfn);
    if (wgs <= 0) return hipErrorInvalidDeviceFunction;
  }
  wgs = std::min<int64_t>(wgs, max_wgs);
  a.chunks = (int32_t)wgs;
  const dim3 grid((unsigned)wgs), block(kThreads);
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
