// chunk_f32_impl.h -- the chunk call on fp32 caches.  It computes what
// chunk_impl.h computes (the attention of page "Can SlimKV compress KV cache
// jointly across tokens and features", section "Latent-space attention
// removes the rebuild step", for every query token of the chunk, with the
// chunk's own tokens appended causally) and shares its schedule, token
// partial and merge; the products run on the fp32 matrix instructions
// (v_mfma_f32_16x16x4_f32), so no operand is split or rounded:
//   * scores S^T = K Q^T per 16-row tile: A operand lane (n, kg) = key row
//     n, features 16c + 4kg + e (the fp32 tile layout of SegView); B operand
//     = query row n, the same features.  Lane (n, kg) ends with query row
//     n's scores for rows 4kg .. 4kg + 3, which after the exponent are the
//     B operand of O^T = V^T P^T;
//   * the value tile is transposed through LDS (fp32, rows padded);
//   * the latent query (q U_K) and the lift (U_V O_lat) read their bases
//     straight from memory: they are small and run once per workgroup.
// Included by chunk.hip after chunk_impl.h.
#pragma once

namespace slimkv {

struct alignas(16) ChunkSharedF32 {
  union {
    struct {
      union {
        float vt[kWaves][16 * (kHeadDim + kVPad)];   // each wave's value tile (16 rows)
        float tok[2][kChunkRows][kHeadDim];          // the chunk's keys and values
      } x;
      float qrot[kChunkRows][kHeadDim];  // rotated query rows, pre-scaled
      float qlat[kChunkRows][kHeadDim];  // the same projected by U_K
    } s;
    float park[kWaves][kChunkRows][kHeadDim];  // each wave's full-width sums
  } u;
  float wml[kWaves][kChunkRows][2];  // each wave's (max, sum) per query row
  int is_last;
};

// Query rows as ChunkPrologue (row m: token m / G, head m % G), fp32: rotate
// into sh.qrot, then (latent beacons) sh.qlat = qrot U_K, with U_K's rows
// read from memory as the B operand: lane (n, kg) takes U_K[i0 + kg][c0 + n].
template <bool ROTATE>
struct ChunkPrologueF32 {
  static constexpr int kHalf = kHeadDim / 2;
  static constexpr int kPairs = kChunkRows * kHalf / kThreads;  // 4
  uint32_t x1[kPairs], x2[kPairs];
  int pos0;

  __device__ __forceinline__ void issue(const AttnArgs& a, int b, int h, int M, int G) {
    const int tid = threadIdx.x;
    const int Q = a.num_tokens;
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
      const int p = min(tid + kThreads * j, M * kHalf - 1);
      const int m = p / kHalf, i = p % kHalf;
      const int t = m / G, g = m - t * G;
      const size_t base = (((size_t)b * Q + t) * a.num_q_heads + (size_t)h * G + g) * kHeadDim;
      x1[j] = ld_bits<false>(a.q, base + i);
      x2[j] = ld_bits<false>(a.q, base + i + kHalf);
    }
    pos0 = a.q_pos[b];
  }

  __device__ __forceinline__ void finish(const AttnArgs& a, ChunkSharedF32& sh, int wave, int h,
                                         int M, int G, bool lat) const {
    const int tid = threadIdx.x, lane = tid & 63;
    const int n = lane & 15, kg = lane >> 4;
    const float sc = (float)a.score_scale;
#pragma unroll
    for (int j = 0; j < kPairs; ++j) {
      const int p = tid + kThreads * j;
      const int m = p / kHalf, i = p % kHalf;
      float r1 = 0.0f, r2 = 0.0f;
      if (m < M) {
        const float v1 = bits_to_float<false>(x1[j]), v2 = bits_to_float<false>(x2[j]);
        if constexpr (ROTATE) {
          float sn, cs;
          rope_sincos(a, pos0 + m / G, i, sn, cs);
          r1 = (v1 * cs - v2 * sn) * sc;
          r2 = (v2 * cs + v1 * sn) * sc;
        } else {  // an ALiBi backbone rotates nothing
          r1 = v1 * sc;
          r2 = v2 * sc;
        }
      }
      sh.u.s.qrot[m][i] = r1;
      sh.u.s.qrot[m][i + kHalf] = r2;
    }
    lds_barrier();
    if (lat) {  // workgroup-uniform
      const int rk = a.rank_k;
      const float* U = static_cast<const float*>(a.U_K) + (size_t)h * kHeadDim * rk;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const int c0 = 16 * (wave + kWaves * jt);
        if (c0 < rk) {  // wave-uniform; rk is a multiple of 16
          f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
          for (int i0 = 0; i0 < kHeadDim; i0 += 4)
            d = __builtin_amdgcn_mfma_f32_16x16x4f32(sh.u.s.qrot[n][i0 + kg],
                                                     U[(size_t)(i0 + kg) * rk + c0 + n], d, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) sh.u.s.qlat[4 * kg + e][c0 + n] = d[e];
        }
      }
      lds_barrier();
    }
  }
};

// Query row n's features 16c + 4kg + e (zero from `width` on): B operands.
template <int C>
__device__ __forceinline__ void chunk_query_f32(const float (*src)[kHeadDim], int width,
                                                float (&qf)[C][4]) {
  const int lane = threadIdx.x & 63, n = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 16 * c + 4 * kg + e;
      qf[c][e] = k < width ? src[n][k] : 0.0f;
    }
}

// One 16-row tile (as chunk_tile): t0 its first row, nchk the 16-feature
// chunks carrying key features, width the value columns; RAW sums into
// accr, else into accb.  ALIBI: as chunk_tile.
template <bool RAW, int NB, bool PG, bool ALIBI = false>
__device__ __forceinline__ void chunk_tile_f32(const SegView<8, false, PG>& sv, int t0, int nchk,
                                               int width, const float (&qf)[8][4], ChunkState<NB>& st,
                                               float* vt, const SegView<8, false, PG>& bv,
                                               const SegView<8, false, PG>& rw, int jn, int nbt,
                                               int total, const TailRows& tail, u32x4_t* kbuf,
                                               u32x4_t* vbuf, float s2 = 0.0f, int ofs = 0,
                                               int step = 0) {
  constexpr int TR = SegView<8, false, PG>::kRows;  // 16
  constexpr int VMAX = Traits<false>::kMaxLoads;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, kg = lane >> 4;

  // scores S^T: lane (n = query row, kg) gets rows 4kg + e
  f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (c < nchk) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        d = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kbuf[c][e]), qf[c][e], d, 0, 0, 0);
    }
  }
  if constexpr (ALIBI) {
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = fmaf(s2, (float)((t0 + 4 * kg + e) * step - ofs), d[e]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (t0 + 4 * kg + e >= sv.rows) d[e] = -INFINITY;
  const bool ua = jn < nbt, ub = jn >= nbt && jn < total;
  const int pid = tile_page(bv, jn * TR, ua, rw, (jn - nbt) * TR, ub);
  load_tile_keys<true>(bv, jn * TR, ua, rw, (jn - nbt) * TR, ub, tail, pid, kbuf);

  // this tile's values into the wave's LDS tile, row-major with padded rows
  const int pitch = width + kVPad;
#pragma unroll
  for (int i = 0; i < VMAX; ++i) {
    const int rt = i * sv.rpi + sv.vrow;
    if (sv.vact && rt < TR) {
      float* dst = vt + rt * pitch + sv.vcc * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = __uint_as_float(vbuf[i][e]);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  load_tile_values<true>(bv, jn * TR, ua, rw, (jn - nbt) * TR, ub, tail, pid, vbuf);

  // online softmax per query row (max over the row's 4 k-group lanes)
  float mx = fmaxf(fmaxf(d[0], d[1]), fmaxf(d[2], d[3]));
  mx = xor32_max(xor16_max(mx));
  const float mnew = fmaxf(st.m, mx);
  if (__builtin_amdgcn_ballot_w64(mnew > st.m) != 0) {
    const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
    st.l *= alpha;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) st.accb[cb] *= alpha;
    if constexpr (RAW)
#pragma unroll
      for (int cb = 0; cb < kHeadDim / 16; ++cb) st.accr[cb] *= alpha;
    st.m = mnew;
  }
  f32x4_t p;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = __builtin_amdgcn_exp2f(d[e] - st.m);
    st.l += p[e];
  }

  // O^T[col][m] += sum over rows V[row][col] P[m][row]: A operand lane
  // (n = column within the block, kg) holds row 4kg + e
  constexpr int NA = RAW ? kHeadDim / 16 : NB;
  f32x4_t* acc = RAW ? st.accr : st.accb;
#pragma unroll
  for (int cb = 0; cb < NA; ++cb) {
    if (16 * cb < width) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(vt[(4 * kg + e) * pitch + 16 * cb + n], p[e],
                                                       acc[cb], 0, 0, 0);
    }
  }
  // the next tile overwrites the LDS tile: every lane has read it by now
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One workgroup of a chunk call on fp32 caches (as chunk_unit).
template <bool BLAT, bool PG, bool ALIBI = false>
__device__ __forceinline__ void chunk_unit_f32(const AttnArgs& a, ChunkSharedF32& sh, int unit, int b,
                                               int h, int c, int k, int nbr, int wr, int slot0,
                                               const int32_t* ptab) {
  constexpr int TR = SegView<8, false, PG>::kRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, kg = lane >> 4;
  const int G = a.group, M = G * a.num_tokens;
  const int nwaves = kWaves * k;
  const int wu = kWaves * ((c + k - 1) % k) + wave;  // the token workgroup dealt last
  const int rk = BLAT ? a.seg[0].rk : 0, rv = BLAT ? a.seg[0].rv : 0;

  SegView<8, false, PG> bv, rw;
  int nbp = 0;  // the unit's beacon pages (paged)
  if constexpr (PG) {
    nbp = (nbr + (1 << a.page_shift) - 1) >> a.page_shift;
    bv.init_paged(a.seg[0].K, a.seg[0].V, a.page_shift, a.num_pages[0], nbr,
                  BLAT ? rk : kHeadDim, BLAT ? rv : kHeadDim, h, a.num_kv_heads, ptab, 0, lane);
    rw.init_paged(a.seg[1].K, a.seg[1].V, a.page_shift, a.num_pages[1], wr, kHeadDim, kHeadDim, h,
                  a.num_kv_heads, ptab, nbp, lane);
  } else {
    bv.init(a.seg[0].K, a.seg[0].V, a.seg[0].rows, nbr, BLAT ? rk : kHeadDim, BLAT ? rv : kHeadDim,
            unit, lane);
    rw.init(a.seg[1].K, a.seg[1].V, a.seg[1].rows, wr, kHeadDim, kHeadDim, unit, lane);
  }
  const int nbt = bv.ntiles, total = nbt + rw.ntiles;
  // past its last tile a wave's slots read a 16-byte window on q past its
  // end (zeros, unused)
  TailRows tail;
  tail.r = make_rsrc(a.q, 16);
  tail.klane = tail.vlane = 64;

  ChunkPrologueF32<!ALIBI> pro;
  pro.issue(a, b, h, M, G);
  u32x4_t kbuf[Traits<false>::kMaxLoads], vbuf[Traits<false>::kMaxLoads];
  int j = wu;
  {
    const bool ub = j < nbt, ur = j >= nbt && j < total;
    const int pid = tile_page(bv, j * TR, ub, rw, (j - nbt) * TR, ur);
    load_tile_keys<true>(bv, j * TR, ub, rw, (j - nbt) * TR, ur, tail, pid, kbuf);
    load_tile_values<true>(bv, j * TR, ub, rw, (j - nbt) * TR, ur, tail, pid, vbuf);
  }
  pro.finish(a, sh, wave, h, M, G, BLAT && nbr > 0);
  if (c == 0 && a.k_new)  // workgroup-uniform
    chunk_token_partial<PG, ALIBI, false>(a, sh, unit, b, h, wr, M, G, ptab, nbp);
  float s2 = 0.0f;
  int bofs = 0, rofs = 0;
  if constexpr (ALIBI) {
    const int tm = n / G;
    s2 = n < M ? a.alibi_slopes[h * G + n % G] * 1.4426950408889634f : 0.0f;
    bofs = a.q_pos[b] - a.beacon_first + tm;
    rofs = (a.k_new ? wr : wr - 1) + tm;
  }

  constexpr int NB = BLAT ? kHeadDim / 16 : 1;  // latent sum blocks: r_V <= 16 NB
  ChunkState<NB> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) st.accb[cb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float* vt = sh.u.s.x.vt[wave];
  float qf[8][4];
  if constexpr (BLAT) {
    chunk_query_f32<8>(sh.u.s.qlat, rk, qf);
    const int nchk = rk / 16;
    for (; j < nbt; j += nwaves)
      chunk_tile_f32<false, NB, PG, ALIBI>(bv, j * TR, nchk, rv, qf, st, vt, bv, rw, j + nwaves, nbt,
                                           total, tail, kbuf, vbuf, s2, bofs, a.beacon_stride);
  }
#pragma unroll
  for (int cb = 0; cb < kHeadDim / 16; ++cb) st.accr[cb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  chunk_query_f32<8>(sh.u.s.qrot, kHeadDim, qf);
  for (; j < total; j += nwaves)
    chunk_tile_f32<true, NB, PG, ALIBI>(rw, (j - nbt) * TR, 8, kHeadDim, qf, st, vt, bv, rw,
                                        j + nwaves, nbt, total, tail, kbuf, vbuf, s2, rofs, 1);
  st.l = xor32_sum(xor16_sum(st.l));
  __builtin_amdgcn_s_setprio(2);  // from here on only the unit's finish: ahead of streaming waves
  if constexpr (BLAT) {
    // the lift accr^T[d][m] += sum_k U_V[d][k] accb^T[k][m]: A operand lane
    // (n, kg) = U_V row 16 db + n, columns 16 cb + 4kg + e, from memory
    const float* U = static_cast<const float*>(a.U_V) + (size_t)h * kHeadDim * rv;
    const int ncb = rv / 16;
#pragma unroll
    for (int db = 0; db < kHeadDim / 16; ++db) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        if (cb < ncb) {
          const f32x4_t ua =
              *reinterpret_cast<const f32x4_t*>(U + (size_t)(16 * db + n) * rv + 16 * cb + 4 * kg);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st.accr[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(ua[e], st.accb[cb][e], st.accr[db], 0, 0, 0);
        }
      }
    }
  }
  lds_barrier();  // every wave is done with the query and value tiles (the park aliases them)
  if (kg == 0) {
    sh.wml[wave][n][0] = st.m;
    sh.wml[wave][n][1] = st.l;
  }
#pragma unroll
  for (int db = 0; db < kHeadDim / 16; ++db)
    *reinterpret_cast<f32x4_t*>(&sh.u.park[wave][n][16 * db + 4 * kg]) = st.accr[db];
  lds_barrier();

  // the workgroup's partial: M rows of (max, sum) and d sums
  const size_t slot = (size_t)slot0 + c;
  float* ml_out = a.part_ml + slot * M * 2;
  float* acc_out = a.part_acc + slot * M * kHeadDim;
  const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(acc_out, (uint32_t)(M * kHeadDim * 4));
#pragma unroll
  for (int it = 0; it < kChunkRows * kHeadDim / 4 / kThreads; ++it) {
    const int idx = tid + kThreads * it;
    const int m = idx / (kHeadDim / 4), col = 4 * (idx % (kHeadDim / 4));
    if (m < M) {
      float Mx = sh.wml[0][m][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) Mx = fmaxf(Mx, sh.wml[w][m][0]);
      f32x4_t sum = {0.0f, 0.0f, 0.0f, 0.0f};
      float L = 0.0f;
      if (Mx != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float wt = __builtin_amdgcn_exp2f(sh.wml[w][m][0] - Mx);
          sum += wt * *reinterpret_cast<const f32x4_t*>(&sh.u.park[w][m][col]);
          L += wt * sh.wml[w][m][1];
        }
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, sum), rs, (m * kHeadDim + col) * 4,
                                             0, kCoherent);
      if (col == 0) {
        store_coherent(&ml_out[2 * m], Mx);
        store_coherent(&ml_out[2 * m + 1], L);
      }
    }
  }

  // the last workgroup of the unit merges (as chunk_unit)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(&a.counters[(size_t)unit * kCounterStride], 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.is_last = done == (uint32_t)(k - 1);
  }
  lds_barrier();
  if (!sh.is_last) return;
  if (tid < 2)
    __hip_atomic_store(&a.counters[(size_t)unit * kCounterStride + tid], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  chunk_finish(a, unit, b, h, slot0, k, M, G);
}

// The fp32 chunk kernel: pieces scheduled as chunk_kernel; BLAT: latent
// beacons (else full-width or none).
template <bool BLAT, bool PG, bool ALIBI = false>
__global__ __launch_bounds__(kThreads, kWgPerCu * kWaves / 4) void chunk_f32_kernel(AttnArgs a) {
  constexpr int TR = SegView<8, false>::kRows;
  __shared__ ChunkSharedF32 sh;
  __shared__ RaggedPick pick;
  __shared__ int32_t ptab[PG ? kMaxPageEntries : 1];
  const int tid = threadIdx.x;
  const int Hkv = a.num_kv_heads, P = a.chunks;
  const int pi = ragged_piece_of((int)blockIdx.x, P);
  ragged_schedule_wg<TR, TR>(a, pick, tid, P, pi);
  lds_barrier();
  const auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  if (pi >= uni(pick.total)) return;
  const int b = uni(pick.b), kb = uni(pick.k), first = uni(pick.first);
  const int h = (pi - first) / kb, c = pi - first - h * kb;
  const int nbr = uni(pick.nb), wr = uni(pick.w);
  if constexpr (PG) {
    const int sh_ = a.page_shift, pm = (1 << sh_) - 1;
    const int nbp = (nbr + pm) >> sh_;
    const int wst = a.k_new ? min(wr + a.num_tokens, a.seg[1].rows) : wr;
    const int n = nbp + ((wst + pm) >> sh_);
    const int32_t* bt = a.page_table[0] + (size_t)b * a.table_width[0];
    const int32_t* rt = a.page_table[1] + (size_t)b * a.table_width[1];
    for (int i = tid; i < n; i += kThreads) ptab[i] = i < nbp ? bt[i] : rt[i - nbp];
    lds_barrier();
  }
  chunk_unit_f32<BLAT, PG, ALIBI>(a, sh, b * Hkv + h, b, h, c, kb, nbr, wr, first + h * kb, ptab);
}

}  // namespace slimkv
